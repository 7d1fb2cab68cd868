// Work schedule of the split decode kernel: which K steps of which 128-row block each workgroup
// does (host side).
//
// Each XCD takes an eighth of every linear's row blocks (its units) and works through one list
// with its compute units, a workgroup starting whenever a compute unit frees up.  Whole units,
// longest first, leave a tail when the work does not divide evenly: a linear with more K steps
// than a compute unit's share, or a last round with few units.  The schedule cuts the long
// units at `head` steps and moves some trailing units of the last linear to a pool, which is
// handed out, once the heads are under way, as pieces of `sigma` steps; pieces of a unit meet in
// fp32 partial slots.  The choice is made by simulating the dispatch (each piece to the compute
// unit that frees first) over a small set of (cut, pooled, sigma), keeping the shortest
// makespan; the simulation walks the same piece list as the kernel (split_piece).
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <utility>

#include "bd_internal.h"

namespace bd {

namespace {

// Fixed cost of a piece, in K steps: filling the copy ring and the first activation loads before
// its first step, and storing its sums after the last.  Measured on the 256-token decode, a
// 14-step pool piece took as long as about 20 steps of a whole unit.
constexpr double kPieceCost = 5.0;

bool same_shape(const SplitShape& a, const SplitShape& b) {
  if (a.np != b.np || a.C != b.C || a.Mp != b.Mp || a.nslots != b.nslots ||
      a.slots_avail != b.slots_avail)
    return false;
  for (int q = 0; q < a.np; ++q)
    if (a.ns[q] != b.ns[q] || a.nb[q] != b.nb[q]) return false;
  return true;
}

// Pieces of one unit the kernel's counter can count: 6 bits per XCD field.
constexpr int kMaxParts = 63;
// Compute units of one XCD the dispatch simulation models at most.
constexpr int kMaxUnitsPerXcd = 256;

// list lengths, split units and partial slots of one XCD's list (the kernel's piece map); the
// return value is the largest number of pieces of one unit
int count_pieces(const SplitShape& sh, SplitSched* h) {
  int max_parts = 1;
  h->nheads = h->npool = h->nsplit = h->nslot = 0;
  for (int q = 0; q < sh.np; ++q) {
    const int cnt = (sh.nb[q] + 7) >> 3;
    const int nh = cnt - h->pooled[q], tail = sh.ns[q] - h->head[q];
    const int tp = tail > 0 ? (tail + h->sigma - 1) / h->sigma : 0;
    const int pp = (sh.ns[q] + h->sigma - 1) / h->sigma;
    const int ncut = tail > 0 ? nh : 0;
    h->nheads += nh;
    h->npool += ncut * tp + h->pooled[q] * pp;
    h->nsplit += ncut + h->pooled[q];
    h->nslot += ncut * (1 + tp) + h->pooled[q] * pp;
    if (ncut > 0) max_parts = std::max(max_parts, 1 + tp);
    if (h->pooled[q] > 0) max_parts = std::max(max_parts, pp);
  }
  return max_parts;
}

// Makespan, in K steps, of one XCD's list (with the largest eighth of every linear) on sh.C
// compute units: a piece costs its steps, c_piece for filling the copy ring and storing, and
// c_part for each partial slot it writes or (the last piece of a unit) reads.
double simulate(const SplitShape& sh, const SplitSched& h, double c_piece, double c_part) {
  double cu[kMaxUnitsPerXcd];  // a heap of the compute units' finishing times (no allocation)
  const int C = std::max(1, std::min(sh.C, kMaxUnitsPerXcd));
  std::fill(cu, cu + C, 0.0);
  for (int kk = 0; kk < h.nheads + h.npool; ++kk) {
    const SplitPiece pc = split_piece(h, sh.np, sh.ns, sh.nb, kk);
    double cost = (pc.k1 - pc.k0) + c_piece;
    if (pc.nparts > 1) cost += c_part * (pc.part == pc.nparts - 1 ? pc.nparts : 1);
    std::pop_heap(cu, cu + C, std::greater<double>());
    cu[C - 1] += cost;
    std::push_heap(cu, cu + C, std::greater<double>());
  }
  return *std::max_element(cu, cu + C);
}

SplitSched choose(const SplitShape& sh) {
  // a partial slot (128 rows x Mp tokens of fp32) against the bytes of a step (W_base rows and
  // every variant's sign words)
  const double c_piece = kPieceCost;
  const double c_part = (double)sh.Mp * kSplitRows * 4 /
                        (double)(kSplitRows * 128 * 2 + sh.nslots * kSplitRows * 16);
  int max_ns = 1;
  for (int q = 0; q < sh.np; ++q) max_ns = std::max(max_ns, sh.ns[q]);
  SplitSched best;
  memset(&best, 0, sizeof(best));
  for (int q = 0; q < sh.np; ++q) best.head[q] = sh.ns[q];
  best.sigma = max_ns;  // no pool
  count_pieces(sh, &best);
  double best_t = simulate(sh, best, c_piece, c_part);
  const int step = std::max(8, (max_ns / 32 + 7) / 8 * 8);
  const int last = sh.np - 1;
  const int max_pool = std::min((sh.nb[last] + 7) >> 3, 2 * sh.C);
  static const int kSigmas[] = {8, 16, 24, 32, 48, 64, 96, 128};
  for (int sigma : kSigmas) {
    if (sigma > max_ns) break;
    for (int cut = step; cut <= max_ns; cut += step) {
      for (int pooled = 0; pooled <= max_pool; ++pooled) {
        SplitSched c;
        memset(&c, 0, sizeof(c));
        for (int q = 0; q < sh.np; ++q) {
          c.head[q] = std::min(sh.ns[q], cut);
          c.pooled[q] = q == last ? pooled : 0;
        }
        c.sigma = sigma;
        if (count_pieces(sh, &c) > kMaxParts || c.nslot > sh.slots_avail) continue;
        const double t = simulate(sh, c, c_piece, c_part);
        if (t < best_t - 1e-9 || (t < best_t + 1e-9 && c.nslot < best.nslot)) {
          best = c;
          best_t = t;
        }
      }
    }
  }
  return best;
}

}  // namespace

SplitSched split_schedule(const SplitShape& sh) {
  // serving calls the same few shapes over and over: keep the 64 most recently computed
  // schedules in a fixed ring (no allocation)
  constexpr int kCache = 64;
  static std::mutex mu;
  static SplitShape shapes[kCache];
  static SplitSched scheds[kCache];
  static int filled = 0, next = 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < filled; ++i)
      if (same_shape(shapes[i], sh)) return scheds[i];
  }
  const SplitSched c = choose(sh);
  std::lock_guard<std::mutex> lk(mu);
  shapes[next] = sh;
  scheds[next] = c;
  next = (next + 1) % kCache;
  if (filled < kCache) ++filled;
  return c;
}

double split_schedule_makespan(const SplitShape& sh, const SplitSched& h) {
  const double c_part = (double)sh.Mp * kSplitRows * 4 /
                        (double)(kSplitRows * 128 * 2 + sh.nslots * kSplitRows * 16);
  return simulate(sh, h, kPieceCost, c_part);
}

int split_compute_units() {
  static std::atomic<int> cached[64];  // per device, 0 = not queried yet
  const int v = device_attribute_cached(cached, hipDeviceAttributeMultiprocessorCount, 256);
  return v < 8 ? 256 : v;
}

}  // namespace bd
