// Host check of the split decode schedule: for seeded random launch shapes, the piece lists the
// kernel walks (split_piece) under the chosen schedule cover every (linear, row block, K step)
// of every XCD exactly once, split units have consistent piece counts and in-range partial
// slots and counters, the workspace's slot budget holds, and the simulated makespan is never
// worse than running whole units.  Prints "ok" and exits 0 when every case passes.
#include <stdio.h>
#include <string.h>

#include <map>
#include <tuple>

#include "../tenant_serving_bitdelta_amd/csrc/bd_internal.h"

using bd::SplitPiece;
using bd::SplitSched;
using bd::SplitShape;

static unsigned g_seed = 12345u;
static int rnd(int n) {
  g_seed = g_seed * 1103515245u + 12345u;
  return (int)((g_seed >> 8) % (unsigned)n);
}

static int check(const SplitShape& sh, const SplitSched& h) {
  int bad = 0;
  if (h.nslot > sh.slots_avail) { printf("slot budget exceeded\n"); ++bad; }
  for (int xcd = 0; xcd < 8; ++xcd) {
    std::map<std::tuple<int, int, int>, int> cover;
    std::map<int, std::pair<int, int>> split_info;
    std::map<int, int> slot_use;
    for (int kk = 0; kk < h.nheads + h.npool; ++kk) {
      const SplitPiece pc = bd::split_piece(h, sh.np, sh.ns, sh.nb, kk);
      if (pc.p < 0) { printf("piece %d of the list maps to nothing\n", kk); ++bad; continue; }
      const int lo = (xcd * sh.nb[pc.p]) >> 3, len = (((xcd + 1) * sh.nb[pc.p]) >> 3) - lo;
      if (pc.lrb >= len) continue;  // this XCD's eighth is shorter
      if (!(0 <= pc.k0 && pc.k0 < pc.k1 && pc.k1 <= sh.ns[pc.p])) { printf("bad K range\n"); ++bad; }
      for (int s = pc.k0; s < pc.k1; ++s) cover[std::make_tuple(pc.p, lo + pc.lrb, s)]++;
      if (pc.nparts > 1) {
        if (pc.sid < 0 || pc.sid >= h.nsplit || pc.part < 0 || pc.part >= pc.nparts ||
            pc.slot0 < 0 || pc.slot0 + pc.part >= h.nslot) { printf("split index out of range\n"); ++bad; }
        auto it = split_info.find(pc.sid);
        if (it == split_info.end()) split_info[pc.sid] = std::make_pair(pc.nparts, pc.slot0);
        else if (it->second != std::make_pair(pc.nparts, pc.slot0)) { printf("inconsistent split unit\n"); ++bad; }
        if (slot_use[pc.slot0 + pc.part]++) { printf("partial slot used twice\n"); ++bad; }
      }
    }
    // every split unit gets all its pieces on this XCD
    for (const auto& e : split_info) {
      int n = 0;
      for (int k = 0; k < e.second.first; ++k) n += slot_use.count(e.second.second + k) ? 1 : 0;
      if (n != e.second.first) { printf("split unit %d has %d of %d pieces\n", e.first, n, e.second.first); ++bad; }
    }
    for (int q = 0; q < sh.np; ++q) {
      const int lo = (xcd * sh.nb[q]) >> 3, len = (((xcd + 1) * sh.nb[q]) >> 3) - lo;
      for (int r = lo; r < lo + len; ++r)
        for (int s = 0; s < sh.ns[q]; ++s)
          if (cover[std::make_tuple(q, r, s)] != 1) {
            if (bad < 8) printf("xcd %d linear %d block %d step %d covered %d times\n", xcd, q, r, s,
                                cover[std::make_tuple(q, r, s)]);
            ++bad;
          }
    }
  }
  SplitSched whole;
  memset(&whole, 0, sizeof(whole));
  int max_ns = 1;
  for (int q = 0; q < sh.np; ++q) { whole.head[q] = sh.ns[q]; if (sh.ns[q] > max_ns) max_ns = sh.ns[q]; }
  whole.sigma = max_ns;
  whole.nheads = 0;
  for (int q = 0; q < sh.np; ++q) whole.nheads += (sh.nb[q] + 7) >> 3;
  if (bd::split_schedule_makespan(sh, h) > bd::split_schedule_makespan(sh, whole) + 1e-9) {
    printf("schedule slower than whole units\n");
    ++bad;
  }
  return bad;
}

int main() {
  int bad = 0, cases = 0;
  // a 70B decoder block (q, k, v, o, gate, up, down; launched longest K first), 14 variants
  {
    SplitShape sh;
    memset(&sh, 0, sizeof(sh));
    const int d_out[7] = {8192, 8192, 1024, 1024, 8192, 28672, 28672};
    const int d_in[7] = {28672, 8192, 8192, 8192, 8192, 8192, 8192};
    sh.np = 7; sh.C = 32; sh.nslots = 14; sh.slots_avail = 7 * bd::kSplitSlotsPerLinear / 8;
    for (int q = 0; q < 7; ++q) { sh.ns[q] = d_in[q] / 128; sh.nb[q] = d_out[q] / 128; }
    for (int mp : {64, 256}) {
      sh.Mp = mp;
      const SplitSched h = bd::split_schedule(sh);
      bad += check(sh, h);
      ++cases;
      // whole units leave a tail here (the 224-step down blocks and a last round of 64-step
      // blocks on few compute units; 204 steps per compute unit on average): the schedule must
      // end at least 10% sooner than whole units do in the same cost model
      SplitSched w;
      memset(&w, 0, sizeof(w));
      for (int q = 0; q < sh.np; ++q) {
        w.head[q] = sh.ns[q];
        w.nheads += (sh.nb[q] + 7) >> 3;
      }
      w.sigma = 224;
      const double t = bd::split_schedule_makespan(sh, h);
      const double tw = bd::split_schedule_makespan(sh, w);
      if (t > 0.9 * tw) {
        printf("70B block, Mp %d: makespan %.1f steps, whole units %.1f\n", mp, t, tw);
        ++bad;
      }
    }
  }
  for (int it = 0; it < 400; ++it) {
    SplitShape sh;
    memset(&sh, 0, sizeof(sh));
    sh.np = 1 + rnd(8);
    sh.C = it % 5 == 0 ? 1 + rnd(40) : 32;
    sh.Mp = 16 * (1 + rnd(16));
    sh.nslots = rnd(17);
    sh.slots_avail = std::min(sh.np, bd::kMaxProblems) * bd::kSplitSlotsPerLinear / 8;
    for (int q = 0; q < sh.np; ++q) {
      sh.nb[q] = 1 + rnd(it % 3 == 0 ? 300 : 40);
      sh.ns[q] = 1 + rnd(it % 2 ? 240 : 70);
    }
    // launch order: longest K first
    for (int a = 0; a < sh.np; ++a)
      for (int b = a + 1; b < sh.np; ++b)
        if (sh.ns[b] > sh.ns[a]) { std::swap(sh.ns[a], sh.ns[b]); std::swap(sh.nb[a], sh.nb[b]); }
    bad += check(sh, bd::split_schedule(sh));
    ++cases;
  }
  if (bad) { printf("%d problems in %d cases\n", bad, cases); return 1; }
  printf("ok %d cases\n", cases);
  return 0;
}
