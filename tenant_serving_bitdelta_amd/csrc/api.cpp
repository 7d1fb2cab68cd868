// C ABI of libbitdelta: argument validation, variant-segment planning and kernel dispatch.
// Every argument error is detected here, on the host, before anything is enqueued.
#include <stdint.h>
#include <string.h>

#include <utility>
#include <vector>

#include "../../include/bitdelta.h"
#include "bd_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = int64_t(1) << 31;

bitdelta_status map_hip(hipError_t e) { return e == hipSuccess ? BITDELTA_OK : BITDELTA_ERR_HIP; }

struct Segment {
  int begin, len, variant;
};

// Validates the shared segmentation; drops empty segments.
bitdelta_status check_segments(int64_t M, const int32_t* seg_offsets, const int32_t* seg_variant,
                               int32_t num_segments, std::vector<Segment>* out) {
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

bitdelta_status check_problem(const bitdelta_problem& p, int64_t M,
                              const std::vector<Segment>& segs) {
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
      if (!v.sign_words || !v.alpha) return BITDELTA_ERR_INVALID_ARG;
      if (!aligned(v.sign_words, 4) || !aligned(v.alpha, 4)) return BITDELTA_ERR_ALIGNMENT;
    }
  }
  return BITDELTA_OK;
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

// The streaming kernels read sign words 16 bytes (4 K steps) per row at a time.
bool stream_eligible(const bitdelta_problem* probs, int np, const std::vector<Segment>& segs) {
  for (int p = 0; p < np; ++p) {
    if (probs[p].d_in % 128 != 0) return false;
    for (const Segment& s : segs)
      if (s.variant >= 0 && !aligned(probs[p].variants[s.variant].sign_words, 16)) return false;
  }
  return true;
}

// The split path reads the tiled sign words and addresses its activation layouts and the tiled
// words with 31-bit offsets.
bool split_eligible(const bitdelta_problem* probs, int np, int64_t M,
                    const std::vector<Segment>& segs) {
  for (int p = 0; p < np; ++p) {
    const bitdelta_problem& P = probs[p];
    if (P.d_in % 128 != 0) return false;
    if ((M + 15) / 16 * 16 * 2 * P.d_in >= (int64_t(1) << 31)) return false;
    if ((P.d_out + 127) / 128 * 128 * (P.d_in / 8) >= (int64_t(1) << 31)) return false;
    for (const Segment& s : segs) {
      if (s.variant < 0) continue;
      const uint32_t* t = P.variants[s.variant].sign_words_t128;
      if (!t || !aligned(t, 16)) return false;
    }
  }
  return true;
}

// ---- GEMV: one launch per linear ----------------------------------------------------------
bitdelta_status run_gemv(const bitdelta_problem* probs, int np, int64_t M,
                         const std::vector<Segment>& segs, int y_f32, hipStream_t st) {
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
          a.words[nslot] = P.variants[s.variant].sign_words;
          a.alpha[nslot] = P.variants[s.variant].alpha;
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

bitdelta_status run_stream(const bitdelta_problem* probs, int np,
                           const std::vector<Segment>& segs, int y_f32, hipStream_t st) {
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
        for (int s = 0; s < (int)slot_var.size(); ++s) {
          S.words[s] = P.variants[slot_var[s]].sign_words;
          S.alpha[s] = P.variants[slot_var[s]].alpha;
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

// ---- split-activation decode: chunks of <= 256 tokens, <= 24 variant tiles, <= 16 variants ---
bitdelta_status run_split(const bitdelta_problem* probs, int np, int64_t M,
                          const std::vector<Segment>& segs, int y_f32, void* workspace,
                          hipStream_t st) {
  // workspace: per problem, fp8 hi/lo activations then the per-token scale codes
  bd::SplitActArgs act;
  memset(&act, 0, sizeof(act));
  const int Mp = (int)((M + 15) / 16 * 16);
  act.Mp = Mp;
  std::vector<unsigned char*> xb(np), xq(np);
  std::vector<int*> xs(np);
  size_t off = 0;
  for (int p = 0; p < np; ++p) {
    unsigned char* base = static_cast<unsigned char*>(workspace) + off;
    const size_t qbytes = ((size_t)Mp * 2 * (size_t)probs[p].d_in + 255) / 256 * 256;
    xb[p] = base;
    xq[p] = base + qbytes;
    xs[p] = reinterpret_cast<int*>(base + 2 * qbytes);
    off += bd::split_workspace_bytes(M, probs[p].d_in);
    act.x[p] = static_cast<const uint16_t*>(probs[p].x);
    act.xb[p] = xb[p];
    act.xq[p] = xq[p];
    act.xscale[p] = xs[p];
    act.d_in[p] = (int)probs[p].d_in;
  }
  bitdelta_status r = map_hip(bd::launch_split_act(act, (int)M, np, st));
  if (r != BITDELTA_OK) return r;

  // problems with longer rows first, so the longest workgroups do not form the tail
  std::vector<int> order(np);
  for (int p = 0; p < np; ++p) order[p] = p;
  for (int i = 1; i < np; ++i)
    for (int k = i; k > 0 && probs[order[k]].d_in > probs[order[k - 1]].d_in; --k)
      std::swap(order[k], order[k - 1]);

  struct Unit {
    int tok, n, variant;
  };
  std::vector<Unit> units;
  for (const Segment& s : segs)
    for (int r0 = 0; r0 < s.len; r0 += 16) units.push_back({s.begin + r0, s.len - r0 < 16 ? s.len - r0 : 16, s.variant});
  size_t u0 = 0;
  while (u0 < units.size()) {
    const int t_begin = units[u0].tok;
    const int tok_base = t_begin / 16 * 16;   // launches cover whole 16-token blocks
    std::vector<int> slot_var;
    int ntiles = 0;
    size_t u1 = u0;
    while (u1 < units.size()) {
      const Unit& u = units[u1];
      if (u.tok + u.n - tok_base > bd::kSplitMaxM) break;
      if (u.variant >= 0) {
        if (ntiles == bd::kSplitMaxTiles) break;
        bool have = false;
        for (int v : slot_var) have = have || v == u.variant;
        if (!have && (int)slot_var.size() == bd::kMaxSlots) break;
        if (!have) slot_var.push_back(u.variant);
        ++ntiles;
      }
      ++u1;
    }
    const int t_end = units[u1 - 1].tok + units[u1 - 1].n;
    bd::SplitArgs a;
    memset(&a, 0, sizeof(a));
    a.tok_base = tok_base;
    a.lo = t_begin - tok_base;
    a.hi = t_end - tok_base;
    a.Mp = Mp;
    a.ntiles = ntiles;
    a.nslots = (int)slot_var.size();
    a.y_f32 = y_f32;
    int ti = 0;
    for (size_t i = u0; i < u1; ++i) {
      const Unit& u = units[i];
      if (u.variant < 0) continue;
      int slot = 0;
      for (int q = 0; q < (int)slot_var.size(); ++q)
        if (slot_var[q] == u.variant) slot = q;
      a.tile_slot[ti] = (int8_t)slot;
      a.tile_valid[ti] = (uint8_t)u.n;
      a.tile_src[ti] = (int16_t)(u.tok - tok_base);
      ++ti;
      for (int t = u.tok - tok_base; t < u.tok - tok_base + u.n; ++t)
        a.has_delta[t >> 5] |= 1u << (t & 31);
    }
    for (int p0 = 0; p0 < np; p0 += bd::kMaxProblems) {
      const int pn = np - p0 < bd::kMaxProblems ? np - p0 : bd::kMaxProblems;
      a.nprob = pn;
      for (int q = 0; q < pn; ++q) {
        const int p = order[p0 + q];
        const bitdelta_problem& P = probs[p];
        bd::SplitProblem& S = a.prob[q];
        S.x = xb[p];
        S.xq = xq[p];
        S.xscale = xs[p];
        S.w = static_cast<const uint16_t*>(P.w_base);
        S.y = P.y;
        S.d_out = (int)P.d_out;
        S.d_in = (int)P.d_in;
        S.nblocks = (int)((P.d_out + bd::kSplitRows - 1) / bd::kSplitRows);
        for (int s = 0; s < (int)slot_var.size(); ++s) {
          S.words[s] = P.variants[slot_var[s]].sign_words_t128;
          S.alpha[s] = P.variants[slot_var[s]].alpha;
        }
      }
      r = map_hip(bd::launch_split(a, st));
      if (r != BITDELTA_OK) return r;
    }
    u0 = u1;
  }
  return BITDELTA_OK;
}

// ---- prefill: per-segment tiles of 256 tokens ---------------------------------------------
bitdelta_status run_prefill(const bitdelta_problem* probs, int np,
                            const std::vector<Segment>& segs, int y_f32, hipStream_t st) {
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
      for (int s = 0; s < (int)slot_var.size(); ++s) {
        a.words[s] = P.variants[slot_var[s]].sign_words;
        a.alpha[s] = P.variants[slot_var[s]].alpha;
      }
      bitdelta_status r = map_hip(bd::launch_prefill(a, st));
      if (r != BITDELTA_OK) return r;
      m0 = m1;
    }
  }
  return BITDELTA_OK;
}

}  // namespace

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
  return (size_t)bd::compress_grid(d_out * d_in) * sizeof(double);
}

bitdelta_status bitdelta_compress(const float* delta, int64_t d_out, int64_t d_in,
                                  uint32_t* sign_words, uint32_t* sign_words_t128, float* alpha,
                                  void* workspace, size_t workspace_bytes, bitdelta_stream stream) {
  if (!delta || !sign_words || !alpha || !workspace) return BITDELTA_ERR_INVALID_ARG;
  if (d_out <= 0 || d_in <= 0 || d_out >= kMaxDim || d_in >= kMaxDim)
    return BITDELTA_ERR_INVALID_ARG;
  if (d_in % 32 != 0) return BITDELTA_ERR_SHAPE;
  if (sign_words_t128 && d_in % 128 != 0) return BITDELTA_ERR_SHAPE;
  if (!aligned(delta, 16) || !aligned(sign_words, 4) || !aligned(alpha, 4) ||
      !aligned(workspace, 8) || !aligned(sign_words_t128, 16))
    return BITDELTA_ERR_ALIGNMENT;
  if (workspace_bytes < bitdelta_compress_workspace_bytes(d_out, d_in)) return BITDELTA_ERR_WORKSPACE;
  return map_hip(bd::launch_compress(delta, d_out * d_in, d_in, sign_words, sign_words_t128, alpha,
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
  std::vector<Segment> segs;
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
