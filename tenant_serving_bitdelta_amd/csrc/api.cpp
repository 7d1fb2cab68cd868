// C ABI of libbitdelta: argument validation, variant-segment planning and kernel dispatch.
// Every argument error is detected here, on the host, before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "../../include/bitdelta.h"
#include "bd_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 31;

thread_local hipError_t g_last_hip_error = hipSuccess;

bitdelta_status map_hip(hipError_t e) {
  if (e == hipSuccess) return BITDELTA_OK;
  g_last_hip_error = e;
  return BITDELTA_ERR_HIP;
}

struct Segment {
  int begin, len, variant;
};

// The non-empty segments of a call (at most BITDELTA_MAX_SEGMENTS), in a fixed array so that
// planning allocates no memory.
struct SegList {
  Segment s[BITDELTA_MAX_SEGMENTS];
  int n = 0;
  const Segment* begin() const { return s; }
  const Segment* end() const { return s + n; }
  void push_back(const Segment& x) { s[n++] = x; }
  bool empty() const { return n == 0; }
};

// Variant of token t (a position of the batch in segment order); segments are sorted by begin.
int variant_at(const SegList& segs, int t) {
  int lo = 0, hi = segs.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (segs.s[mid].begin <= t) lo = mid;
    else hi = mid - 1;
  }
  return segs.s[lo].variant;
}

// Validates the shared segmentation; drops empty segments.
bitdelta_status check_segments(int64_t M, const int32_t* seg_offsets, const int32_t* seg_variant,
                               int32_t num_segments, SegList* out) {
  if (M < 0 || M >= kMaxDim) return BITDELTA_ERR_INVALID_ARG;
  if (num_segments < 0 || num_segments > BITDELTA_MAX_SEGMENTS) return BITDELTA_ERR_INVALID_ARG;
  if (M == 0 && num_segments == 0) return BITDELTA_OK;
  if (!seg_offsets || (num_segments > 0 && !seg_variant)) return BITDELTA_ERR_INVALID_ARG;
  if (seg_offsets[0] != 0 || seg_offsets[num_segments] != M) return BITDELTA_ERR_SHAPE;
  for (int s = 0; s < num_segments; ++s) {
    if (seg_offsets[s + 1] < seg_offsets[s]) return BITDELTA_ERR_SHAPE;
    if (seg_variant[s] < -1 || seg_variant[s] >= BITDELTA_MAX_VARIANTS)
      return BITDELTA_ERR_INVALID_ARG;
    const int len = seg_offsets[s + 1] - seg_offsets[s];
    if (len > 0 && out) out->push_back({seg_offsets[s], len, seg_variant[s]});
  }
  return BITDELTA_OK;
}

bitdelta_status check_problem(const bitdelta_problem& p, int64_t M, const SegList& segs) {
  // an empty batch may come with empty (null) activation and output buffers
  if (!p.w_base || (M > 0 && (!p.x || !p.y))) return BITDELTA_ERR_INVALID_ARG;
  if (p.d_out <= 0 || p.d_in <= 0 || p.d_out >= kMaxDim || p.d_in >= kMaxDim)
    return BITDELTA_ERR_INVALID_ARG;
  if (p.d_in % 32 != 0) return BITDELTA_ERR_SHAPE;
  if (p.num_variants < 0 || p.num_variants > BITDELTA_MAX_VARIANTS) return BITDELTA_ERR_INVALID_ARG;
  if (p.num_variants > 0 && !p.variants) return BITDELTA_ERR_INVALID_ARG;
  if (!aligned(p.x, 16) || !aligned(p.w_base, 16) || !aligned(p.y, 16))
    return BITDELTA_ERR_ALIGNMENT;
  for (const Segment& s : segs) {
    if (s.variant >= p.num_variants) return BITDELTA_ERR_INVALID_ARG;
    if (s.variant >= 0) {
      const bitdelta_variant& v = p.variants[s.variant];
      if (!v.alpha || (!v.sign_words && !v.sign_words_t128)) return BITDELTA_ERR_INVALID_ARG;
      if (v.alpha_per_row != 0 && v.alpha_per_row != 1) return BITDELTA_ERR_INVALID_ARG;
      if (v.sign_words_t128 && p.d_in % 128 != 0) return BITDELTA_ERR_SHAPE;
      if (!aligned(v.sign_words, 4) || !aligned(v.sign_words_t128, 16) || !aligned(v.alpha, 4))
        return BITDELTA_ERR_ALIGNMENT;
    }
  }
  return BITDELTA_OK;
}

// The sign words the kernels read for a variant: the tiled layout when the variant has it (each
// kernel then streams one 128-row block's words of a step as 2 KiB contiguous), else the
// row-major words.
const uint32_t* kernel_words(const bitdelta_variant& v, bool* tiled) {
  *tiled = v.sign_words_t128 != nullptr;
  return *tiled ? v.sign_words_t128 : v.sign_words;
}

int pick_path(int64_t M) {
  if (M <= 4) return BITDELTA_PATH_GEMV;
  if (M <= bd::kSplitMaxM) return BITDELTA_PATH_SPLIT;
  return BITDELTA_PATH_PREFILL;
}

size_t workspace_for(int64_t M, int64_t d_in, int path) {
  if (M <= 0 || d_in <= 0 || M >= kMaxDim || d_in >= kMaxDim) return 0;
  if (path == BITDELTA_PATH_AUTO) path = pick_path(M);
  return path == BITDELTA_PATH_SPLIT ? bd::split_workspace_bytes(M, d_in) : 0;
}

// The streaming kernels read sign words 16 bytes (4 K steps) per row at a time: the tiled
// layout, or 16-byte aligned row-major words.
bool stream_eligible(const bitdelta_problem* probs, int np, const SegList& segs) {
  for (int p = 0; p < np; ++p) {
    if (probs[p].d_in % 128 != 0) return false;
    for (const Segment& s : segs) {
      if (s.variant < 0) continue;
      const bitdelta_variant& v = probs[p].variants[s.variant];
      if (!v.sign_words_t128 && !aligned(v.sign_words, 16)) return false;
    }
  }
  return true;
}

// The split path reads the tiled sign words and addresses its activation layouts and the tiled
// words with 31-bit offsets.
bool split_eligible(const bitdelta_problem* probs, int np, int64_t M, const SegList& segs) {
  for (int p = 0; p < np; ++p) {
    const bitdelta_problem& P = probs[p];
    if (P.d_in % 128 != 0) return false;
    if ((M + 15) / 16 * 16 * 2 * P.d_in >= (int64_t(1) << 31)) return false;
    if ((P.d_out + 127) / 128 * 128 * (P.d_in / 8) >= (int64_t(1) << 31)) return false;
    // the schedule numbers row blocks and list entries in 16 bits
    if ((P.d_out + 127) / 128 > 8192) return false;
    for (const Segment& s : segs) {
      if (s.variant < 0) continue;
      const uint32_t* t = P.variants[s.variant].sign_words_t128;
      if (!t || !aligned(t, 16)) return false;
    }
  }
  return true;
}

// ---- GEMV: one launch per linear ----------------------------------------------------------
bitdelta_status run_gemv(const bitdelta_problem* probs, int np, int64_t M, const SegList& segs,
                         int y_f32, hipStream_t st) {
  for (int p = 0; p < np; ++p) {
    const bitdelta_problem& P = probs[p];
    bd::GemvArgs a;
    memset(&a, 0, sizeof(a));
    a.x = static_cast<const uint16_t*>(P.x);
    a.w = static_cast<const uint16_t*>(P.w_base);
    a.y = P.y;
    a.d_out = (int)P.d_out;
    a.d_in = (int)P.d_in;
    a.M = (int)M;
    a.y_f32 = y_f32;
    int nslot = 0, last = -2;
    for (const Segment& s : segs) {
      int slot = -1;
      if (s.variant >= 0) {
        if (s.variant != last) {
          bool tiled = false;
          a.words[nslot] = kernel_words(P.variants[s.variant], &tiled);
          if (tiled) a.tiled |= 1u << nslot;
          a.alpha[nslot] = P.variants[s.variant].alpha;
          if (P.variants[s.variant].alpha_per_row) a.alpha_rows |= 1u << nslot;
          ++nslot;
        }
        slot = nslot - 1;
      }
      last = s.variant;
      for (int t = s.begin; t < s.begin + s.len; ++t) a.tok_slot[t] = slot;
    }
    bitdelta_status st2 = map_hip(bd::launch_gemv(a, st));
    if (st2 != BITDELTA_OK) return st2;
  }
  return BITDELTA_OK;
}

// ---- streaming decode: batches of <= 24 tiles, <= 16 variants, <= 256 rows per launch -------
struct Tile {
  int row, valid, variant;
};

bitdelta_status run_stream(const bitdelta_problem* probs, int np, const SegList& segs, int y_f32,
                           hipStream_t st) {
  std::vector<Tile> tiles;
  for (const Segment& s : segs)
    for (int r = 0; r < s.len; r += 16) tiles.push_back({s.begin + r, s.len - r < 16 ? s.len - r : 16, s.variant});
  size_t t0 = 0;
  while (t0 < tiles.size()) {
    // greedy chunk [t0, t1)
    std::vector<int> slot_var;
    size_t t1 = t0;
    const int base_row = tiles[t0].row;
    while (t1 < tiles.size() && (int)(t1 - t0) < bd::kStreamMaxTiles) {
      const Tile& t = tiles[t1];
      if (t.row + t.valid - base_row > 32767) break;  // tile offsets are 16-bit
      if (t.variant >= 0) {
        bool have = !slot_var.empty() && slot_var.back() == t.variant;
        if (!have && (int)slot_var.size() == bd::kMaxSlots) break;
        if (!have) slot_var.push_back(t.variant);
      }
      ++t1;
    }
    const int rows = tiles[t1 - 1].row + tiles[t1 - 1].valid - base_row;
    bd::StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.ntiles = (int)(t1 - t0);
    // base-only batches still get one (dummy) slot: the kernel reads it and scales it by 0
    a.nslots = slot_var.empty() ? 1 : (int)slot_var.size();
    a.M = rows;
    a.y_f32 = y_f32;
    for (size_t i = t0; i < t1; ++i) {
      const Tile& t = tiles[i];
      int slot = -1;
      if (t.variant >= 0)
        for (int q = 0; q < (int)slot_var.size(); ++q)
          if (slot_var[q] == t.variant) slot = q;
      a.tile_slot[i - t0] = (int8_t)slot;
      a.tile_valid[i - t0] = (uint8_t)t.valid;
      a.tile_src[i - t0] = (int16_t)(t.row - base_row);
    }
    // problems, at most kMaxProblems per launch
    for (int p0 = 0; p0 < np; p0 += bd::kMaxProblems) {
      const int pn = np - p0 < bd::kMaxProblems ? np - p0 : bd::kMaxProblems;
      a.nprob = pn;
      int blocks = 0;
      for (int q = 0; q < pn; ++q) {
        const bitdelta_problem& P = probs[p0 + q];
        bd::StreamProblem& S = a.prob[q];
        S.x = static_cast<const uint16_t*>(P.x) + (size_t)base_row * P.d_in;
        S.w = static_cast<const uint16_t*>(P.w_base);
        S.y = static_cast<char*>(P.y) + (size_t)base_row * P.d_out * (y_f32 ? 4 : 2);
        S.d_out = (int)P.d_out;
        S.d_in = (int)P.d_in;
        S.block_begin = blocks;
        S.alpha_rows = 0;
        S.tiled = 0;
        for (int s = 0; s < (int)slot_var.size(); ++s) {
          bool tiled = false;
          S.words[s] = kernel_words(P.variants[slot_var[s]], &tiled);
          if (tiled) S.tiled |= 1u << s;
          S.alpha[s] = P.variants[slot_var[s]].alpha;
          if (P.variants[slot_var[s]].alpha_per_row) S.alpha_rows |= 1u << s;
        }
        if (slot_var.empty()) {
          // W_base is at least 16x larger than a sign-word matrix of the same shape
          S.words[0] = static_cast<const uint32_t*>(P.w_base);
          S.alpha[0] = nullptr;
        }
        blocks += (int)((P.d_out + bd::kStreamRowsPerBlock - 1) / bd::kStreamRowsPerBlock);
      }
      bitdelta_status r = map_hip(bd::launch_stream(a, blocks, st));
      if (r != BITDELTA_OK) return r;
    }
    t0 = t1;
  }
  return BITDELTA_OK;
}

// ---- split-activation decode ----------------------------------------------------------------
// A launch covers the tokens [t_begin, t_end) of at most 16 aligned 16-token blocks (dense
// tiles) and at most 16 variants.  The distinct variants of a tile's tokens form (tile, variant)
// pairs.  Neighbouring tiles are handed out together (2 per wave when there are more than 8
// tiles), because tokens arrive grouped by variant and the pairs of one variant in both tiles of
// a wave share one expansion of the sign words; a wave's pairs are arranged as slot groups, one
// variant per group.  Tile units go to the waves longest first, each to the SIMD (waves w and
// w + 4) with the least estimated work.  A launch ends before the first run of same-variant
// tokens that would give a wave more than kSplitMaxGroups groups.  With two tiles per wave every
// wave issues one share of the global->LDS copies; with one, the less loaded wave of each SIMD
// issues that SIMD's share.
struct SplitPlan {
  int t_begin = 0, t_end = 0, tok_base = 0, nd = 1, ng = 0, nslot = 0;
  int slot_var[bd::kMaxSlots];
  bd::SplitWave wv[8];
  int8_t token_slot[bd::kSplitMaxM];
};

// Estimated SIMD cycles per K step: the base product of one dense tile (32 bf16 MFMAs), one
// pair (16 fp4 x fp6 MFMAs and the lane masking) and one expansion of a variant's sign words.
constexpr int kCostTile = 512, kCostPair = 320, kCostExpand = 224;

// max_tiles: dense 16-token tiles one launch may hold (16).
bool plan_split(const SegList& segs, int t_begin, int t_end, int max_tiles, SplitPlan* pl) {
  const int tok_base = t_begin / 16 * 16;
  const int ntiles = (t_end - 1 - tok_base) / 16 + 1;
  if (ntiles > max_tiles) return false;
  int slot_var[bd::kMaxSlots];
  int nslot = 0;
  int8_t token_slot[bd::kSplitMaxM];
  memset(token_slot, -1, sizeof(token_slot));
  for (int t = t_begin; t < t_end; ++t) {
    const int v = variant_at(segs, t);
    if (v < 0) continue;
    int slot = -1;
    for (int q = 0; q < nslot; ++q)
      if (slot_var[q] == v) slot = q;
    if (slot < 0) {
      if (nslot == bd::kMaxSlots) return false;
      slot_var[nslot] = v;
      slot = nslot++;
    }
    token_slot[t - tok_base] = (int8_t)slot;
  }
  const int nd = ntiles <= 8 ? 1 : 2;
  // the distinct slots of each tile, as a bit set
  unsigned tset[bd::kSplitMaxM / 16] = {0u};
  for (int i = 0; i < ntiles; ++i)
    for (int t = 16 * i; t < 16 * i + 16; ++t)
      if (token_slot[t] >= 0) tset[i] |= 1u << token_slot[t];
  // units: single tiles, or neighbouring pairs of tiles
  struct Unit {
    int tile[2];
    int ngroups, cost;
  };
  Unit units[bd::kSplitMaxM / 16];
  int nunits = 0;
  for (int i = 0; i < ntiles; i += nd) {
    Unit u;
    u.tile[0] = i;
    u.tile[1] = (nd == 2 && i + 1 < ntiles) ? i + 1 : -1;
    const unsigned s0 = tset[i], s1 = u.tile[1] >= 0 ? tset[i + 1] : 0u;
    const int n0 = __builtin_popcount(s0), n1 = __builtin_popcount(s1);
    const int shared = __builtin_popcount(s0 & s1);
    u.ngroups = shared + std::max(n0 - shared, n1 - shared);
    u.cost = kCostTile * (u.tile[1] >= 0 ? 2 : 1) + kCostPair * (n0 + n1) +
             kCostExpand * __builtin_popcount(s0 | s1);
    if (u.ngroups > bd::kSplitMaxGroups) return false;
    units[nunits++] = u;
  }
  // units by cost, longest first (insertion sort: stable, no allocation)
  int order[bd::kSplitMaxM / 16];
  for (int k = 0; k < nunits; ++k) {
    int i = k;
    while (i > 0 && units[order[i - 1]].cost < units[k].cost) {
      order[i] = order[i - 1];
      --i;
    }
    order[i] = k;
  }
  int simd_load[4] = {0, 0, 0, 0}, simd_waves[4] = {0, 0, 0, 0};
  int wave_of[bd::kSplitMaxM / 16];
  for (int oi = 0; oi < nunits; ++oi) {
    const int k = order[oi];
    int best = -1;
    for (int sm = 0; sm < 4; ++sm)
      if (simd_waves[sm] < 2 && (best < 0 || simd_load[sm] < simd_load[best])) best = sm;
    wave_of[k] = best + 4 * simd_waves[best]++;
    simd_load[best] += units[k].cost;
  }
  pl->t_begin = t_begin;
  pl->t_end = t_end;
  pl->tok_base = tok_base;
  pl->nd = nd;
  pl->nslot = nslot;
  memcpy(pl->slot_var, slot_var, sizeof(slot_var));
  memcpy(pl->token_slot, token_slot, sizeof(token_slot));
  pl->ng = 0;
  for (int w = 0; w < 8; ++w) {
    bd::SplitWave& W = pl->wv[w];
    W.tile[0] = W.tile[1] = -1;
    for (int q = 0; q < bd::kSplitMaxGroups; ++q) W.slot[q][0] = W.slot[q][1] = -1;
    W.copier = nd == 2 ? w : -1;
    W.pad_ = 0;
  }
  if (nd == 1) {
    int wave_load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < nunits; ++k) wave_load[wave_of[k]] = units[k].cost;
    // waves w and w + 4 share a SIMD: the lighter one copies (ties: wave w + 4)
    for (int sm = 0; sm < 4; ++sm)
      pl->wv[wave_load[sm] < wave_load[sm + 4] ? sm : sm + 4].copier = sm;
  }
  for (int k = 0; k < nunits; ++k) {
    bd::SplitWave& W = pl->wv[wave_of[k]];
    const Unit& u = units[k];
    W.tile[0] = u.tile[0];
    W.tile[1] = u.tile[1];
    const unsigned s0 = tset[u.tile[0]], s1 = u.tile[1] >= 0 ? tset[u.tile[1]] : 0u;
    int g = 0;
    for (int q = 0; q < bd::kMaxSlots; ++q)  // variants of both tiles: one group each
      if ((s0 & s1) >> q & 1u) {
        W.slot[g][0] = W.slot[g][1] = q;
        ++g;
      }
    int g0 = g, g1 = g;  // the others side by side
    for (int q = 0; q < bd::kMaxSlots; ++q) {
      if ((s0 & ~s1) >> q & 1u) W.slot[g0++][0] = q;
      if ((s1 & ~s0) >> q & 1u) W.slot[g1++][1] = q;
    }
    pl->ng = std::max(pl->ng, std::max(g0, g1));
  }
  return true;
}

bitdelta_status run_split(const bitdelta_problem* probs, int np, int64_t M, const SegList& segs,
                          int y_f32, void* workspace, hipStream_t st) {
  // workspace: per problem bf16 pieces, fp6 pieces, block scales; then every problem's share of
  // partial slots, then of split counters, then of statistics blocks
  const int Mp = (int)((M + 15) / 16 * 16);
  unsigned char *xb[BITDELTA_MAX_PROBLEMS], *xq[BITDELTA_MAX_PROBLEMS], *xs[BITDELTA_MAX_PROBLEMS],
      *xc[BITDELTA_MAX_PROBLEMS];
  size_t off = 0;
  for (int p = 0; p < np; ++p) {
    unsigned char* base = static_cast<unsigned char*>(workspace) + off;
    size_t bb, qb, cb, kb;
    bd::split_workspace_parts(M, probs[p].d_in, &bb, &qb, &cb, &kb);
    xb[p] = base;
    xq[p] = base + bb;
    xs[p] = base + bb + qb;
    xc[p] = base + bb + qb + cb;
    off += bb + qb + cb + kb;
  }
  const size_t slot_bytes = bd::split_slot_bytes(M);
  const int slots_total = np * bd::kSplitSlotsPerLinear;  // counters: as many
  float* partial = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + off);
  // slot_bytes is a multiple of 256, so the slots of all problems end on a 256-byte boundary
  unsigned char* after_slots = static_cast<unsigned char*>(workspace) + off +
                               (size_t)slots_total * slot_bytes;
  uint64_t* counter = reinterpret_cast<uint64_t*>(after_slots);
  // statistics: the first word of the first problem's block (it accumulates, never cleared)
  uint32_t* stats = reinterpret_cast<uint32_t*>(after_slots + (size_t)np * bd::kSplitCounterBytes);
  const int C = bd::split_compute_units() / 8;
  // problems with longer rows first, so the longest workgroups do not form the tail (insertion
  // sort: stable, no allocation)
  int order[BITDELTA_MAX_PROBLEMS];
  for (int p = 0; p < np; ++p) {
    int i = p;
    while (i > 0 && probs[order[i - 1]].d_in < probs[p].d_in) {
      order[i] = order[i - 1];
      --i;
    }
    order[i] = p;
  }

  const int max_tiles = bd::kSplitMaxM / 16;

  int t_begin = 0;
  while (t_begin < M) {
    // grow the launch one run (same variant, same 16-token block) at a time
    SplitPlan plan;
    const int limit = (int)std::min<int64_t>(M, t_begin / 16 * 16 + 16 * max_tiles);
    int t = t_begin;
    while (t < limit) {
      // the run of token t: same variant (segment), same 16-token block
      int seg_end = t + 1;
      for (const Segment& sg : segs)
        if (sg.begin <= t && t < sg.begin + sg.len) seg_end = sg.begin + sg.len;
      const int e = std::min(std::min(seg_end, limit), (t / 16 + 1) * 16);
      SplitPlan cand;
      if (!plan_split(segs, t_begin, e, max_tiles, &cand)) break;
      plan = cand;
      t = e;
    }
    // one run fits any launch (one tile, at most one pair, one variant)
    if (plan.t_end <= t_begin) return BITDELTA_ERR_UNSUPPORTED;

    bd::SplitArgs a;
    memset(&a, 0, sizeof(a));
    a.tok_base = plan.tok_base;
    a.lo = plan.t_begin - plan.tok_base;
    a.hi = plan.t_end - plan.tok_base;
    a.Mp = Mp;
    a.nslots = plan.nslot;
    a.y_f32 = y_f32;
    memcpy(a.wv, plan.wv, sizeof(a.wv));
    memcpy(a.token_slot, plan.token_slot, sizeof(a.token_slot));
    bd::SplitActArgs act;
    memset(&act, 0, sizeof(act));
    act.Mp = Mp;
    act.tok_base = a.tok_base;
    act.lo = a.lo;
    act.hi = a.hi;
    memcpy(act.token_slot, plan.token_slot, sizeof(act.token_slot));
    for (int p0 = 0; p0 < np; p0 += bd::kMaxProblems) {
      const int pn = std::min(np - p0, bd::kMaxProblems);
      a.nprob = pn;
      act.nprob = pn;
      bd::SplitShape sh;
      memset(&sh, 0, sizeof(sh));
      sh.np = pn;
      sh.C = C;
      sh.Mp = Mp;
      sh.nslots = a.nslots;
      // partial slots (and split counters) per XCD: an eighth of the launch's linears' share
      sh.slots_avail = std::min(slots_total, pn * bd::kSplitSlotsPerLinear) / 8;
      for (int q = 0; q < pn; ++q) {
        const bitdelta_problem& P = probs[order[p0 + q]];
        sh.ns[q] = (int)(P.d_in / 128);
        sh.nb[q] = (int)((P.d_out + bd::kSplitRows - 1) / bd::kSplitRows);
      }
      bd::SplitSched& H = a.sch;
      H = bd::split_schedule(sh);
      H.slot_bytes = (uint32_t)slot_bytes;
      H.partial = partial;
      H.counter = counter;
      H.stats = stats;
      act.counter = counter;
      act.ncounter = 0;
      for (int x = 0; x < 8; ++x) act.ncounter += H.x[x].nsplit;
      for (int q = 0; q < pn; ++q) {
        const int p = order[p0 + q];
        const bitdelta_problem& P = probs[p];
        act.x[q] = static_cast<const uint16_t*>(P.x);
        act.xb[q] = xb[p];
        act.xq[q] = xq[p];
        act.xs[q] = xs[p];
        act.xc[q] = reinterpret_cast<float*>(xc[p]);
        act.d_in[q] = (int)P.d_in;
        bd::SplitProblem& S = a.prob[q];
        S.x = xb[p];
        S.xq = xq[p];
        S.xs = xs[p];
        S.xc = reinterpret_cast<const float*>(xc[p]);
        S.w = static_cast<const uint16_t*>(P.w_base);
        S.y = P.y;
        S.d_out = (int)P.d_out;
        S.d_in = (int)P.d_in;
        S.nblocks = (int)((P.d_out + bd::kSplitRows - 1) / bd::kSplitRows);
        S.alpha_rows = 0;
        for (int s = 0; s < plan.nslot; ++s) {
          const bitdelta_variant& V = P.variants[plan.slot_var[s]];
          S.words[s] = V.sign_words_t128;
          // per-matrix alpha scales x in the prologue; per-row alphas are applied by the kernel
          act.alpha[q][s] = V.alpha_per_row ? nullptr : V.alpha;
          S.alpha[s] = V.alpha_per_row ? V.alpha : nullptr;
          if (V.alpha_per_row) S.alpha_rows |= 1u << s;
        }
      }
      bitdelta_status r = map_hip(bd::launch_split_act(act, st));
      if (r != BITDELTA_OK) return r;
      r = map_hip(bd::launch_split(a, plan.nd, plan.ng, st));
      if (r != BITDELTA_OK) return r;
    }
    t_begin = plan.t_end;
  }
  return BITDELTA_OK;
}

// ---- prefill: per-segment tiles of 256 tokens ---------------------------------------------
bitdelta_status run_prefill(const bitdelta_problem* probs, int np, const SegList& segs, int y_f32,
                            hipStream_t st) {
  struct MT {
    int row, rows, variant;
  };
  std::vector<MT> mts;
  for (const Segment& s : segs)
    for (int r = 0; r < s.len; r += bd::kPrefillBM)
      mts.push_back({s.begin + r, s.len - r < bd::kPrefillBM ? s.len - r : bd::kPrefillBM, s.variant});
  for (int p = 0; p < np; ++p) {
    const bitdelta_problem& P = probs[p];
    size_t m0 = 0;
    while (m0 < mts.size()) {
      bd::PrefillArgs a;
      memset(&a, 0, sizeof(a));
      std::vector<int> slot_var;
      size_t m1 = m0;
      while (m1 < mts.size() && (int)(m1 - m0) < bd::kPrefillMaxMTiles) {
        const MT& t = mts[m1];
        int slot = -1;
        if (t.variant >= 0) {
          for (int q = 0; q < (int)slot_var.size(); ++q)
            if (slot_var[q] == t.variant) slot = q;
          if (slot < 0) {
            if ((int)slot_var.size() == bd::kMaxSlots) break;
            slot_var.push_back(t.variant);
            slot = (int)slot_var.size() - 1;
          }
        }
        a.mt_row[m1 - m0] = t.row;
        a.mt_rows[m1 - m0] = (int16_t)t.rows;
        a.mt_slot[m1 - m0] = (int8_t)slot;
        ++m1;
      }
      a.x = static_cast<const uint16_t*>(P.x);
      a.w = static_cast<const uint16_t*>(P.w_base);
      a.y = P.y;
      a.d_out = (int)P.d_out;
      a.d_in = (int)P.d_in;
      a.y_f32 = y_f32;
      a.n_mtiles = (int)(m1 - m0);
      a.n_ntiles = (int)((P.d_out + bd::kPrefillBN - 1) / bd::kPrefillBN);
      // bit s of vec_signs: slot s's words are read 16 bytes (one 128-column step) at a time,
      // which the tiled layout always allows and row-major words when 16-byte aligned
      const unsigned vec_all = P.d_in % 128 == 0 ? 0xFFFFFFFFu : 0u;
      a.vec_signs = (int)vec_all;
      a.alpha_rows = 0;
      a.tiled = 0;
      for (int s = 0; s < (int)slot_var.size(); ++s) {
        bool tiled = false;
        a.words[s] = kernel_words(P.variants[slot_var[s]], &tiled);
        if (tiled) a.tiled |= 1u << s;
        a.alpha[s] = P.variants[slot_var[s]].alpha;
        if (P.variants[slot_var[s]].alpha_per_row) a.alpha_rows |= 1u << s;
        if (!tiled && !aligned(a.words[s], 16)) a.vec_signs &= ~(1 << s);
      }
      bitdelta_status r = map_hip(bd::launch_prefill(a, st));
      if (r != BITDELTA_OK) return r;
      m0 = m1;
    }
  }
  return BITDELTA_OK;
}

}  // namespace

namespace bd {
bitdelta_status status_of_hip(hipError_t e) { return map_hip(e); }

// bitdelta_matmul_grouped restricted to the SPLIT path, with the workspace supplied by the
// library (the scratch-backed entry point): every argument is checked as for the grouped call;
// a batch the SPLIT path does not serve (AUTO would pick another path, or a variant lacks the
// tiled words or has per-row scales) is UNSUPPORTED; a workspace need above `ws_bytes` is
// WORKSPACE.  Nothing is enqueued on an error.
bitdelta_status matmul_grouped_split(const bitdelta_problem* problems, int32_t num_problems,
                                     int64_t M, const int32_t* seg_offsets,
                                     const int32_t* seg_variant, int32_t num_segments,
                                     int32_t y_dtype, int32_t path, void* workspace,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!problems || num_problems <= 0 || num_problems > BITDELTA_MAX_PROBLEMS)
    return BITDELTA_ERR_INVALID_ARG;
  if (y_dtype != BITDELTA_OUT_BF16 && y_dtype != BITDELTA_OUT_F32) return BITDELTA_ERR_INVALID_ARG;
  if (path != BITDELTA_PATH_AUTO && path != BITDELTA_PATH_SPLIT) return BITDELTA_ERR_UNSUPPORTED;
  SegList segs;
  bitdelta_status s = check_segments(M, seg_offsets, seg_variant, num_segments, &segs);
  if (s != BITDELTA_OK) return s;
  for (int p = 0; p < num_problems; ++p) {
    s = check_problem(problems[p], M, segs);
    if (s != BITDELTA_OK) return s;
  }
  if (M == 0) return BITDELTA_OK;
  if (path == BITDELTA_PATH_AUTO && pick_path(M) != BITDELTA_PATH_SPLIT) return BITDELTA_ERR_UNSUPPORTED;
  if (!split_eligible(problems, num_problems, M, segs)) return BITDELTA_ERR_UNSUPPORTED;
  size_t need = 0;
  for (int p = 0; p < num_problems; ++p) need += workspace_for(M, problems[p].d_in, BITDELTA_PATH_SPLIT);
  if (!workspace || need > ws_bytes) return BITDELTA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITDELTA_ERR_ALIGNMENT;
  return run_split(problems, num_problems, M, segs, y_dtype == BITDELTA_OUT_F32, workspace, stream);
}
}  // namespace bd

extern "C" {

int bitdelta_abi_version(void) { return BITDELTA_ABI_VERSION; }

const char* bitdelta_status_string(int status) {
  switch (status) {
    case BITDELTA_OK: return "ok";
    case BITDELTA_ERR_INVALID_ARG: return "invalid argument";
    case BITDELTA_ERR_SHAPE: return "invalid shape";
    case BITDELTA_ERR_ALIGNMENT: return "misaligned pointer";
    case BITDELTA_ERR_WORKSPACE: return "workspace too small";
    case BITDELTA_ERR_UNSUPPORTED: return "unsupported size";
    case BITDELTA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t bitdelta_last_hip_error(void) { return (int32_t)g_last_hip_error; }

const char* bitdelta_last_hip_error_string(void) { return hipGetErrorString(g_last_hip_error); }

int64_t bitdelta_sign_words(int64_t d_out, int64_t d_in) {
  if (d_out < 0 || d_in <= 0 || d_in % 32 != 0 || d_out >= kMaxDim || d_in >= kMaxDim) return -1;
  return d_out * (d_in / 32);
}

int64_t bitdelta_sign_words_t128(int64_t d_out, int64_t d_in) {
  if (d_out < 0 || d_in <= 0 || d_in % 128 != 0 || d_out >= kMaxDim || d_in >= kMaxDim) return -1;
  return (d_out + 127) / 128 * 128 * (d_in / 32);
}

size_t bitdelta_compress_workspace_bytes(int64_t d_out, int64_t d_in) {
  if (d_out <= 0 || d_in <= 0 || d_in % 32 != 0 || d_out >= kMaxDim || d_in >= kMaxDim) return 0;
  return (size_t)bd::compress_partials(d_out, d_in) * sizeof(double);
}

bitdelta_status bitdelta_compress(const float* delta, int64_t d_out, int64_t d_in,
                                  uint32_t* sign_words, uint32_t* sign_words_t128, float* alpha,
                                  void* workspace, size_t workspace_bytes, bitdelta_stream stream) {
  if (!delta || (!sign_words && !sign_words_t128) || !alpha || !workspace)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0) return BITDELTA_ERR_SHAPE;
  if (sign_words_t128 && d_in % 128 != 0) return BITDELTA_ERR_SHAPE;
  if (!aligned(delta, 16) || !aligned(sign_words, 4) || !aligned(alpha, 4) ||
      !aligned(workspace, 8) || !aligned(sign_words_t128, 16))
    return BITDELTA_ERR_ALIGNMENT;
  if (workspace_bytes < bitdelta_compress_workspace_bytes(d_out, d_in)) return BITDELTA_ERR_WORKSPACE;
  return map_hip(bd::launch_compress(delta, d_out, d_in, sign_words, sign_words_t128, alpha,
                                     static_cast<double*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

bitdelta_status bitdelta_compress_from_weights(const void* w_ft, const void* w_base, int64_t d_out,
                                               int64_t d_in, uint32_t* sign_words,
                                               uint32_t* sign_words_t128, float* alpha,
                                               void* workspace, size_t workspace_bytes,
                                               bitdelta_stream stream) {
  if (!w_ft || !w_base || (!sign_words && !sign_words_t128) || !alpha || !workspace)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0) return BITDELTA_ERR_SHAPE;
  if (sign_words_t128 && d_in % 128 != 0) return BITDELTA_ERR_SHAPE;
  if (!aligned(w_ft, 16) || !aligned(w_base, 16) || !aligned(sign_words, 4) ||
      !aligned(alpha, 4) || !aligned(workspace, 8) || !aligned(sign_words_t128, 16))
    return BITDELTA_ERR_ALIGNMENT;
  if (workspace_bytes < bitdelta_compress_workspace_bytes(d_out, d_in)) return BITDELTA_ERR_WORKSPACE;
  return map_hip(bd::launch_compress_pair(static_cast<const uint16_t*>(w_ft),
                                          static_cast<const uint16_t*>(w_base), d_out, d_in,
                                          sign_words, sign_words_t128, alpha,
                                          static_cast<double*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

bitdelta_status bitdelta_reconstruct(const void* w_base, int64_t d_out, int64_t d_in,
                                     const bitdelta_variant* variant, void* w_eff,
                                     bitdelta_stream stream) {
  if (!w_base || !variant || !w_eff || !variant->alpha ||
      (!variant->sign_words && !variant->sign_words_t128))
    return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim) return BITDELTA_ERR_INVALID_ARG;
  if (variant->alpha_per_row != 0 && variant->alpha_per_row != 1) return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0 || (variant->sign_words_t128 && d_in % 128 != 0)) return BITDELTA_ERR_SHAPE;
  if (!aligned(w_base, 16) || !aligned(w_eff, 16) || !aligned(variant->sign_words, 4) ||
      !aligned(variant->sign_words_t128, 16) || !aligned(variant->alpha, 4))
    return BITDELTA_ERR_ALIGNMENT;
  bool tiled = false;
  const uint32_t* words = kernel_words(*variant, &tiled);
  return map_hip(bd::launch_reconstruct(static_cast<const uint16_t*>(w_base), words, tiled ? 1 : 0,
                                        variant->alpha, variant->alpha_per_row, d_out, d_in,
                                        static_cast<uint16_t*>(w_eff),
                                        static_cast<hipStream_t>(stream)));
}

bitdelta_status bitdelta_upload_variant(const uint32_t* host_words, const float* host_alpha,
                                        int64_t alpha_count, int64_t d_out, int64_t d_in,
                                        uint32_t* sign_words, uint32_t* sign_words_t128,
                                        float* alpha, void* staging, size_t staging_bytes,
                                        bitdelta_stream stream) {
  if (!host_words || !host_alpha || !alpha || (!sign_words && !sign_words_t128))
    return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim) return BITDELTA_ERR_INVALID_ARG;
  if (alpha_count != 1 && alpha_count != d_out) return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0 || (sign_words_t128 && d_in % 128 != 0)) return BITDELTA_ERR_SHAPE;
  const size_t nbytes = (size_t)d_out * (size_t)(d_in / 32) * 4;
  // the row-major words on the device: the caller's sign_words, else the staging buffer
  uint32_t* rm = sign_words;
  if (!rm) {
    if (!staging || staging_bytes < nbytes) return BITDELTA_ERR_WORKSPACE;
    rm = static_cast<uint32_t*>(staging);
  }
  if (!aligned(alpha, 4) || !aligned(rm, sign_words_t128 ? 16 : 4) || !aligned(sign_words_t128, 16))
    return BITDELTA_ERR_ALIGNMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  bd::clear_stale_error();
  bitdelta_status r = map_hip(hipMemcpyAsync(rm, host_words, nbytes, hipMemcpyHostToDevice, st));
  if (r != BITDELTA_OK) return r;
  if (sign_words_t128) {
    r = map_hip(bd::launch_retile(rm, d_out, d_in, sign_words_t128, st));
    if (r != BITDELTA_OK) return r;
  }
  return map_hip(hipMemcpyAsync(alpha, host_alpha, (size_t)alpha_count * sizeof(float),
                                hipMemcpyHostToDevice, st));
}

size_t bitdelta_compress_rows_workspace_bytes(int64_t d_out, int64_t d_in) {
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim || d_in % 32 != 0) return 0;
  return (size_t)bd::compress_rows_partials(d_out, d_in) * sizeof(double);
}

bitdelta_status bitdelta_compress_rows(const float* delta, int64_t d_out, int64_t d_in,
                                       uint32_t* sign_words, uint32_t* sign_words_t128,
                                       float* alpha, void* workspace, size_t workspace_bytes,
                                       bitdelta_stream stream) {
  if (!delta || (!sign_words && !sign_words_t128) || !alpha || !workspace)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim) return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0) return BITDELTA_ERR_SHAPE;
  if (sign_words_t128 && d_in % 128 != 0) return BITDELTA_ERR_SHAPE;
  if (!aligned(delta, 16) || !aligned(sign_words, 4) || !aligned(alpha, 4) ||
      !aligned(workspace, 8) || !aligned(sign_words_t128, 16))
    return BITDELTA_ERR_ALIGNMENT;
  if (workspace_bytes < bitdelta_compress_rows_workspace_bytes(d_out, d_in))
    return BITDELTA_ERR_WORKSPACE;
  return map_hip(bd::launch_compress_rows(delta, d_out, d_in, sign_words, sign_words_t128, alpha,
                                          static_cast<double*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

bitdelta_status bitdelta_plan_segments(const int32_t* token_variant, int64_t M,
                                       int32_t num_variants, int32_t* perm,
                                       int32_t* seg_offsets, int32_t* seg_variant,
                                       int32_t* num_segments) {
  if (M < 0 || M >= kMaxDim || num_variants < 0 || num_variants > BITDELTA_MAX_VARIANTS)
    return BITDELTA_ERR_INVALID_ARG;
  if (!seg_offsets || !seg_variant || !num_segments || (M > 0 && (!token_variant || !perm)))
    return BITDELTA_ERR_INVALID_ARG;
  std::vector<int64_t> count(num_variants + 1, 0);  // index v + 1
  for (int64_t t = 0; t < M; ++t) {
    const int32_t v = token_variant[t];
    if (v < -1 || v >= num_variants) return BITDELTA_ERR_INVALID_ARG;
    ++count[v + 1];
  }
  std::vector<int64_t> start(num_variants + 1, 0);
  int32_t ns = 0;
  int64_t acc = 0;
  seg_offsets[0] = 0;
  for (int v = 0; v <= num_variants; ++v) {
    start[v] = acc;
    if (count[v] > 0) {
      acc += count[v];
      seg_variant[ns] = v - 1;
      seg_offsets[ns + 1] = (int32_t)acc;
      ++ns;
    }
  }
  for (int64_t t = 0; t < M; ++t) perm[start[token_variant[t] + 1]++] = (int32_t)t;
  *num_segments = ns;
  return BITDELTA_OK;
}

int32_t bitdelta_auto_path(int64_t M, const int32_t* seg_offsets, const int32_t* seg_variant,
                           int32_t num_segments) {
  if (check_segments(M, seg_offsets, seg_variant, num_segments, nullptr) != BITDELTA_OK) return -1;
  return pick_path(M);
}

size_t bitdelta_matmul_workspace_bytes(int64_t M, int64_t d_in, int32_t path) {
  if (path < BITDELTA_PATH_AUTO || path > BITDELTA_PATH_SPLIT) return 0;
  return workspace_for(M, d_in, path);
}

bitdelta_status bitdelta_matmul_grouped(const bitdelta_problem* problems, int32_t num_problems,
                                        int64_t M, const int32_t* seg_offsets,
                                        const int32_t* seg_variant, int32_t num_segments,
                                        int32_t y_dtype, int32_t path, void* workspace,
                                        size_t workspace_bytes, bitdelta_stream stream) {
  if (!problems || num_problems <= 0 || num_problems > BITDELTA_MAX_PROBLEMS)
    return BITDELTA_ERR_INVALID_ARG;
  if (y_dtype != BITDELTA_OUT_BF16 && y_dtype != BITDELTA_OUT_F32) return BITDELTA_ERR_INVALID_ARG;
  if (path < BITDELTA_PATH_AUTO || path > BITDELTA_PATH_SPLIT) return BITDELTA_ERR_INVALID_ARG;
  SegList segs;
  bitdelta_status s = check_segments(M, seg_offsets, seg_variant, num_segments, &segs);
  if (s != BITDELTA_OK) return s;
  for (int p = 0; p < num_problems; ++p) {
    s = check_problem(problems[p], M, segs);
    if (s != BITDELTA_OK) return s;
  }
  if (M == 0) return BITDELTA_OK;
  const bool explicit_path = path != BITDELTA_PATH_AUTO;
  if (path == BITDELTA_PATH_AUTO) path = pick_path(M);
  if (path == BITDELTA_PATH_GEMV && M > 4) return BITDELTA_ERR_UNSUPPORTED;
  if (path == BITDELTA_PATH_SPLIT && !split_eligible(problems, num_problems, M, segs)) {
    if (explicit_path) return BITDELTA_ERR_UNSUPPORTED;
    path = BITDELTA_PATH_STREAM;
  }
  if (path == BITDELTA_PATH_STREAM && !stream_eligible(problems, num_problems, segs)) {
    if (explicit_path) return BITDELTA_ERR_UNSUPPORTED;
    path = BITDELTA_PATH_PREFILL;
  }
  if (path == BITDELTA_PATH_SPLIT) {
    size_t need = 0;
    for (int p = 0; p < num_problems; ++p) need += workspace_for(M, problems[p].d_in, path);
    if (!workspace || workspace_bytes < need) return BITDELTA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return BITDELTA_ERR_ALIGNMENT;
  }
  const int y_f32 = y_dtype == BITDELTA_OUT_F32;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (path) {
    case BITDELTA_PATH_GEMV: return run_gemv(problems, num_problems, M, segs, y_f32, st);
    case BITDELTA_PATH_STREAM: return run_stream(problems, num_problems, segs, y_f32, st);
    case BITDELTA_PATH_SPLIT:
      return run_split(problems, num_problems, M, segs, y_f32, workspace, st);
    default: return run_prefill(problems, num_problems, segs, y_f32, st);
  }
}

bitdelta_status bitdelta_matmul(const void* x, const void* w_base, int64_t M, int64_t d_out,
                                int64_t d_in, const bitdelta_variant* variants,
                                int32_t num_variants, const int32_t* seg_offsets,
                                const int32_t* seg_variant, int32_t num_segments, void* y,
                                int32_t y_dtype, void* workspace, size_t workspace_bytes,
                                bitdelta_stream stream) {
  bitdelta_problem p;
  p.x = x;
  p.w_base = w_base;
  p.y = y;
  p.d_out = d_out;
  p.d_in = d_in;
  p.variants = variants;
  p.num_variants = num_variants;
  return bitdelta_matmul_grouped(&p, 1, M, seg_offsets, seg_variant, num_segments, y_dtype,
                                 BITDELTA_PATH_AUTO, workspace, workspace_bytes, stream);
}

}  // extern "C"
