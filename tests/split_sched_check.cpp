// Host check of the split decode schedule: for seeded random launch shapes, the XCDs' runs tile
// each linear's row blocks in XCD order with about an eighth of the work each, the piece lists
// the kernel walks (split_piece) under the chosen schedule cover every (linear, row block, K
// step) exactly once, split units keep all their pieces on one XCD with consistent piece counts
// and in-range partial slots and counters numbered XCD after XCD, the workspace's slot budget
// holds, and the simulated makespan is never worse than running whole units.  Prints "ok" and
// exits 0 when every case passes.
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

// whole units on every XCD's run (no cut, no pool), for comparison
static SplitSched whole_units(const SplitShape& sh, const SplitSched& h) {
  SplitSched w = h;
  int split0 = 0, slot0 = 0;
  for (int x = 0; x < 8; ++x) {
    bd::SplitXcd& X = w.x[x];
    int max_ns = 1;
    for (int q = 0; q < sh.np; ++q)
      if (X.cnt[q] > 0 && sh.ns[q] > max_ns) max_ns = sh.ns[q];
    X.cut = (int16_t)max_ns;
    X.sigma = (int16_t)max_ns;
    X.pooled = 0;
    int nh, npl, nsp, nsl;
    bd::split_xcd_counts(X, sh.np, sh.ns, &nh, &npl, &nsp, &nsl);
    X.nheads = (int16_t)nh; X.npool = (int16_t)npl; X.nsplit = (int16_t)nsp; X.nslot = (int16_t)nsl;
    X.split0 = (int16_t)split0; X.slot0 = (int16_t)slot0;
    split0 += nsp; slot0 += nsl;
  }
  return w;
}

static int check(const SplitShape& sh, const SplitSched& h) {
  int bad = 0;
  std::map<std::tuple<int, int, int>, int> cover;
  std::map<int, std::pair<int, int>> split_info;  // sid -> (nparts, first slot)
  std::map<int, int> split_xcd;                   // sid -> the XCD whose list holds it
  std::map<int, int> slot_use;
  int split_end = 0, slot_end = 0;
  int64_t total = 0, max_ns = 1;
  for (int q = 0; q < sh.np; ++q) {
    total += (int64_t)sh.nb[q] * sh.ns[q];
    if (sh.ns[q] > max_ns) max_ns = sh.ns[q];
  }
  int pos[bd::kMaxProblems] = {0};
  for (int xcd = 0; xcd < 8; ++xcd) {
    const bd::SplitXcd& X = h.x[xcd];
    if (X.nslot > sh.slots_avail || X.nsplit > sh.slots_avail) { printf("slot budget exceeded\n"); ++bad; }
    if (X.split0 != split_end || X.slot0 != slot_end) { printf("counters or slots not numbered XCD after XCD\n"); ++bad; }
    split_end += X.nsplit;
    slot_end += X.nslot;
    int nh, npl, nsp, nsl;
    bd::split_xcd_counts(X, sh.np, sh.ns, &nh, &npl, &nsp, &nsl);
    if (nh != X.nheads || npl != X.npool || nsp != X.nsplit || nsl != X.nslot) { printf("list counts differ\n"); ++bad; }
    // runs: each linear's blocks tiled by the XCDs in order; the XCD's work near an eighth
    int64_t work = 0;
    for (int q = 0; q < sh.np; ++q) {
      if (X.cnt[q] > 0) {
        if (X.first[q] != pos[q]) { printf("xcd %d linear %d run starts at %d, not %d\n", xcd, q, X.first[q], pos[q]); ++bad; }
        pos[q] += X.cnt[q];
      }
      work += (int64_t)X.cnt[q] * sh.ns[q];
    }
    if (8 * work > total + 8 * max_ns || 8 * work < total - 8 * max_ns) {
      printf("xcd %d has %lld of %lld steps\n", xcd, (long long)work, (long long)total);
      ++bad;
    }
    for (int kk = 0; kk < X.nheads + X.npool; ++kk) {
      const SplitPiece pc = bd::split_piece(X, sh.np, sh.ns, kk);
      if (pc.p < 0) { printf("piece %d of the list maps to nothing\n", kk); ++bad; continue; }
      if (pc.rb < X.first[pc.p] || pc.rb >= X.first[pc.p] + X.cnt[pc.p]) { printf("block outside the XCD's run\n"); ++bad; }
      if (!(0 <= pc.k0 && pc.k0 < pc.k1 && pc.k1 <= sh.ns[pc.p])) { printf("bad K range\n"); ++bad; }
      for (int s = pc.k0; s < pc.k1; ++s) cover[std::make_tuple(pc.p, pc.rb, s)]++;
      if (pc.nparts > 1) {
        if (pc.sid < X.split0 || pc.sid >= X.split0 + X.nsplit || pc.part < 0 || pc.part >= pc.nparts ||
            pc.slot0 < X.slot0 || pc.slot0 + pc.part >= X.slot0 + X.nslot) { printf("split index out of range\n"); ++bad; }
        auto it = split_info.find(pc.sid);
        if (it == split_info.end()) split_info[pc.sid] = std::make_pair(pc.nparts, pc.slot0);
        else if (it->second != std::make_pair(pc.nparts, pc.slot0)) { printf("inconsistent split unit\n"); ++bad; }
        auto ix = split_xcd.find(pc.sid);
        if (ix == split_xcd.end()) split_xcd[pc.sid] = xcd;
        else if (ix->second != xcd) { printf("split unit %d on two XCDs\n", pc.sid); ++bad; }
        if (slot_use[pc.slot0 + pc.part]++) { printf("partial slot used twice\n"); ++bad; }
      }
    }
  }
  if (split_end > sh.slots_avail * 8 || slot_end > sh.slots_avail * 8) { printf("workspace exceeded\n"); ++bad; }
  // every split unit gets all its pieces
  for (const auto& e : split_info) {
    int n = 0;
    for (int k = 0; k < e.second.first; ++k) n += slot_use.count(e.second.second + k) ? 1 : 0;
    if (n != e.second.first) { printf("split unit %d has %d of %d pieces\n", e.first, n, e.second.first); ++bad; }
  }
  // every (linear, block, step) exactly once
  for (int q = 0; q < sh.np; ++q) {
    if (pos[q] != sh.nb[q]) { printf("linear %d: runs cover %d of %d blocks\n", q, pos[q], sh.nb[q]); ++bad; }
    for (int r = 0; r < sh.nb[q]; ++r)
      for (int s = 0; s < sh.ns[q]; ++s)
        if (cover[std::make_tuple(q, r, s)] != 1) {
          if (bad < 8) printf("linear %d block %d step %d covered %d times\n", q, r, s,
                              cover[std::make_tuple(q, r, s)]);
          ++bad;
        }
  }
  if (bd::split_schedule_makespan(sh, h) > bd::split_schedule_makespan(sh, whole_units(sh, h)) + 1e-9) {
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
      const SplitSched w = whole_units(sh, h);
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
