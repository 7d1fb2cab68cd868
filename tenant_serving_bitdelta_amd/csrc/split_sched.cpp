// Work schedule of the split decode kernel: which K steps of which 128-row block each workgroup
// does (host side).
//
// The linears' row blocks, in launch order, are cut into 8 runs of about equal work, one per XCD
// (its units), so that a linear's activations are fetched into the L2 of as few XCDs as the
// balance allows.  Each XCD works through one list with its compute units, a workgroup starting
// whenever a compute unit frees up.  Whole units, longest first, leave a tail when the work does
// not divide evenly: a linear with more K steps than a compute unit's share, or a last round with
// few units.  The XCD's schedule cuts the long units at `cut` steps and moves some trailing units
// of its last linear to a pool, which is handed out, once the heads are under way, as pieces of
// `sigma` steps; pieces of a unit meet in fp32 partial slots.  The choice is made per XCD by
// simulating the dispatch (each piece to the compute unit that frees first) over a small set of
// (cut, pooled, sigma), keeping the shortest makespan; the simulation walks the same piece list
// as the kernel (split_piece).
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

// Makespan, in K steps, of XCD X's list on sh.C compute units: a piece costs its steps, c_piece
// for filling the copy ring and storing, and c_part for each partial slot it writes or (the last
// piece of a unit) reads.
double simulate(const SplitShape& sh, const SplitXcd& X, double c_piece, double c_part) {
  double cu[kMaxUnitsPerXcd];  // a heap of the compute units' finishing times (no allocation)
  const int C = std::max(1, std::min(sh.C, kMaxUnitsPerXcd));
  std::fill(cu, cu + C, 0.0);
  for (int kk = 0; kk < X.nheads + X.npool; ++kk) {
    const SplitPiece pc = split_piece(X, sh.np, sh.ns, kk);
    double cost = (pc.k1 - pc.k0) + c_piece;
    if (pc.nparts > 1) cost += c_part * (pc.part == pc.nparts - 1 ? pc.nparts : 1);
    std::pop_heap(cu, cu + C, std::greater<double>());
    cu[C - 1] += cost;
    std::push_heap(cu, cu + C, std::greater<double>());
  }
  return *std::max_element(cu, cu + C);
}

// Sets the counts of X from its parameters; false if a unit would have too many pieces or the
// XCD more partial slots than the workspace gives it.
bool count(const SplitShape& sh, SplitXcd* X) {
  int nh, npl, nsp, nsl;
  const int max_parts = split_xcd_counts(*X, sh.np, sh.ns, &nh, &npl, &nsp, &nsl);
  X->nheads = (int16_t)nh;
  X->npool = (int16_t)npl;
  X->nsplit = (int16_t)nsp;
  X->nslot = (int16_t)nsl;
  return max_parts <= kMaxParts && nsl <= sh.slots_avail && nsp <= sh.slots_avail &&
         nh + npl <= 32767;
}

// a partial slot (128 rows x Mp tokens of fp32) against the bytes of a step (W_base rows and
// every variant's sign words), in steps
double part_cost(const SplitShape& sh) {
  return (double)sh.Mp * kSplitRows * 4 /
         (double)(kSplitRows * 128 * 2 + sh.nslots * kSplitRows * 16);
}

// Steps left over (in absolute value) when linears from..np-1, with avail[q] blocks left, fill r
// steps greedily, each taking the blocks whose middles fall within what is left.
int64_t leftover(const SplitShape& sh, const int* avail, int from, int64_t r) {
  for (int q = from; q < sh.np; ++q) {
    const int64_t k = std::min<int64_t>(avail[q], std::max<int64_t>(0, (2 * r + sh.ns[q]) / (2 * sh.ns[q])));
    r -= k * sh.ns[q];
  }
  return r < 0 ? -r : r;
}

// The XCDs' runs: XCD x takes, linear by linear in launch order, the next blocks of each linear
// that fit an eighth of the total steps (the cumulative target of XCDs 0..x less what they took),
// one block fewer of a linear when the smaller linears after it then fill the eighth more
// exactly (28 blocks of 224 steps and 4 of 64 rather than 29 of 224 and a gap); the last XCD
// takes what is left.  Each linear's blocks are so split into consecutive runs in XCD order.
void assign(const SplitShape& sh, SplitSched* h) {
  int64_t total = 0;
  for (int q = 0; q < sh.np; ++q) total += (int64_t)sh.nb[q] * sh.ns[q];
  int avail[kMaxProblems], next[kMaxProblems];
  for (int q = 0; q < kMaxProblems; ++q) avail[q] = next[q] = 0;
  for (int q = 0; q < sh.np; ++q) avail[q] = sh.nb[q];
  int64_t done = 0;
  for (int x = 0; x < 8; ++x) {
    SplitXcd& X = h->x[x];
    int64_t r = (2 * (int64_t)(x + 1) * total + 8) / 16 - done;  // round((x + 1) total / 8) - done
    for (int q = 0; q < sh.np; ++q) {
      if (avail[q] == 0) continue;
      int k;
      if (x == 7) {
        k = avail[q];
      } else {
        k = (int)std::min<int64_t>(avail[q], std::max<int64_t>(0, (2 * r + sh.ns[q]) / (2 * sh.ns[q])));
        if (k > 0 && k < avail[q] &&
            leftover(sh, avail, q + 1, r - (int64_t)(k - 1) * sh.ns[q]) <
                leftover(sh, avail, q + 1, r - (int64_t)k * sh.ns[q]))
          --k;
      }
      if (k > 0) {
        X.first[q] = (int16_t)next[q];
        X.cnt[q] = (int16_t)k;
        next[q] += k;
        avail[q] -= k;
        r -= (int64_t)k * sh.ns[q];
        done += (int64_t)k * sh.ns[q];
      }
    }
  }
}

// (cut, pooled, sigma) of one XCD: the shortest simulated makespan, ties to fewer partial slots
void choose_xcd(const SplitShape& sh, SplitXcd* X) {
  const double c_piece = kPieceCost, c_part = part_cost(sh);
  int max_ns = 1, last = -1;
  for (int q = 0; q < sh.np; ++q)
    if (X->cnt[q] > 0) {
      max_ns = std::max(max_ns, sh.ns[q]);
      last = q;
    }
  SplitXcd best = *X;
  best.cut = (int16_t)max_ns;
  best.pooled = 0;
  best.sigma = (int16_t)max_ns;  // whole units, no pool
  count(sh, &best);
  if (last < 0) {
    *X = best;
    return;
  }
  double best_t = simulate(sh, best, c_piece, c_part);
  const int step = std::max(8, (max_ns / 32 + 7) / 8 * 8);
  const int max_pool = std::min((int)X->cnt[last], 2 * sh.C);
  static const int kSigmas[] = {8, 16, 24, 32, 48, 64, 96, 128};
  for (int sigma : kSigmas) {
    if (sigma > max_ns) break;
    for (int cut = step; cut <= max_ns; cut += step) {
      for (int pooled = 0; pooled <= max_pool; ++pooled) {
        SplitXcd c = *X;
        c.cut = (int16_t)cut;
        c.pooled = (int16_t)pooled;
        c.sigma = (int16_t)sigma;
        if (!count(sh, &c)) continue;
        const double t = simulate(sh, c, c_piece, c_part);
        if (t < best_t - 1e-9 || (t < best_t + 1e-9 && c.nslot < best.nslot)) {
          best = c;
          best_t = t;
        }
      }
    }
  }
  *X = best;
}

SplitSched choose(const SplitShape& sh) {
  SplitSched h;
  memset(&h, 0, sizeof(h));
  assign(sh, &h);
  int split0 = 0, slot0 = 0;
  for (int x = 0; x < 8; ++x) {
    choose_xcd(sh, &h.x[x]);
    h.x[x].split0 = (int16_t)split0;
    h.x[x].slot0 = (int16_t)slot0;
    split0 += h.x[x].nsplit;
    slot0 += h.x[x].nslot;
  }
  return h;
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
  double t = 0.0;
  for (int x = 0; x < 8; ++x) t = std::max(t, simulate(sh, h.x[x], kPieceCost, part_cost(sh)));
  return t;
}

int split_compute_units() {
  static std::atomic<int> cached[64];  // per device, 0 = not queried yet
  const int v = device_attribute_cached(cached, hipDeviceAttributeMultiprocessorCount, 256);
  return v < 8 ? 256 : v;
}

}  // namespace bd
