// Internal declarations shared by the HIP kernels and the C-ABI layer of libbitdelta.
// Nothing here is part of the public ABI (include/bitdelta.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// bf16 <-> f32 helpers (bf16 is the upper half of an IEEE binary32).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(unsigned pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi_to_f32(unsigned pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Round-to-nearest-even f32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ unsigned f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Launch status: hipGetLastError() also returns an error left behind by an earlier runtime call
// of the same thread (another library's query, say), so each launcher clears it first and the
// check after the launch reports that launch alone.
inline void clear_stale_error() { (void)hipGetLastError(); }

// ---------------------------------------------------------------------------------------------
// Per-device one-time set-up, safe when several host threads launch at once: one bit per
// device id (ids below 64) in an atomic mask.  Setting a kernel attribute twice is harmless, so
// two threads that both find the bit clear may both set it; neither sees a torn value.
// ---------------------------------------------------------------------------------------------
struct DeviceOnce {
  std::atomic<unsigned long long> done{0};
};
// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes) once per device.
inline hipError_t set_dynamic_lds_once(DeviceOnce& once, const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (once.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (bit) once.done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}
// A device attribute of the current device, queried once per device and kept in `cache`
// (64 entries, 0 = not queried yet); `fallback` when the query fails or gives a value below 1.
inline int device_attribute_cached(std::atomic<int>* cache, hipDeviceAttribute_t attr,
                                   int fallback) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v != 0) return v;
  if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v < 1) v = fallback;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// ---------------------------------------------------------------------------------------------
// Sign-word layouts.  Row-major: word (r, c) at r * wpr + c (wpr = d_in / 32 words per row).
// 128-row tiled (d_in % 128 == 0): rows in blocks of 128, columns in steps of 128 (4 words), the
// 4 words of one row and one step at ((r / 128) * (wpr / 4) + c / 4) * 512 + (r % 128) * 4 + c % 4,
// so one block's words of one step are 2 KiB contiguous.  Either way the 4 words of a row and a
// 128-column step are 16 contiguous bytes; this is the word offset of word 4q of row r.
// ---------------------------------------------------------------------------------------------
__host__ __device__ __forceinline__ size_t sign_quad_offset(bool tiled, int r, int q, int wpr) {
  return tiled ? ((size_t)(r >> 7) * (size_t)(wpr >> 2) + (size_t)q) * 512 + (size_t)(r & 127) * 4
               : (size_t)r * (size_t)wpr + 4 * (size_t)q;
}

// ---------------------------------------------------------------------------------------------
// Compress (two passes)
// ---------------------------------------------------------------------------------------------
// fp64 partials (workspace doubles) pass 1 may write for a d_out x d_in matrix, whichever of
// its two forms runs
int64_t compress_partials(int64_t d_out, int64_t d_in);
int64_t compress_rows_partials(int64_t d_out, int64_t d_in);
hipError_t launch_compress_rows(const float* delta, int64_t d_out, int64_t d_in, uint32_t* words,
                                uint32_t* tiled, float* alpha, double* partials,
                                hipStream_t stream);
// words: row-major [d_out][d_in/32]; tiled: optional copy in the 128-row tiled layout (NULL for
// none; needs d_in % 128 == 0).
hipError_t launch_compress(const float* delta, int64_t d_out, int64_t d_in, uint32_t* words,
                           uint32_t* tiled, float* alpha, double* partials, hipStream_t stream);
// the same outputs for Delta = W_ft - W_base of two bf16 matrices [d_out][d_in]
hipError_t launch_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                                int64_t d_in, uint32_t* words, uint32_t* tiled, float* alpha,
                                double* partials, hipStream_t stream);

// W_eff = bf16_RNE(fp32(w) + (+-alpha)) written to HBM (the unfused reconstruction); words in
// either layout (tiled != 0: the 128-row tiled layout, d_in % 128 == 0).
hipError_t launch_reconstruct(const uint16_t* w, const uint32_t* words, int tiled,
                              const float* alpha, int alpha_per_row, int64_t d_out, int64_t d_in,
                              uint16_t* w_eff, hipStream_t stream);
// row-major sign words [d_out][d_in/32] (device) -> the 128-row tiled layout (d_in % 128 == 0)
hipError_t launch_retile(const uint32_t* src, int64_t d_out, int64_t d_in, uint32_t* dst,
                         hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// Matmul kernels
// ---------------------------------------------------------------------------------------------
constexpr int kMaxSlots = 16;     // distinct variants one streaming launch serves
constexpr int kMaxProblems = 8;   // linears one streaming launch serves

// GEMV (M <= 4): one launch per linear.
struct GemvArgs {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  int d_out, d_in, M, y_f32;
  // per token: the variant slot (-1 = base) and whether it differs from the previous token
  int tok_slot[4];
  const uint32_t* words[4];
  const float* alpha[4];
  unsigned alpha_rows;  // bit s set: slot s has one alpha per output row
  unsigned tiled;       // bit s set: slot s's words are in the 128-row tiled layout
};
hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream);

// Streaming decode: token tiles of 16 rows, each tile within one segment.  Needs d_in % 128 == 0
// and 16-byte aligned sign words; at least one slot (a readable dummy when no variant is used).
constexpr int kStreamMaxTiles = 24;
constexpr int kStreamMaxM = 256;   // batches up to this size go to the streaming path by default
constexpr int kStreamRowsPerBlock = 64;

struct StreamProblem {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  int d_out, d_in;
  int block_begin;
  unsigned alpha_rows;  // bit s set: slot s has one alpha per output row
  unsigned tiled;       // bit s set: slot s's words are in the 128-row tiled layout
  unsigned pad_;
  const uint32_t* words[kMaxSlots];
  const float* alpha[kMaxSlots];
};

struct StreamArgs {
  StreamProblem prob[kMaxProblems];
  int nprob, ntiles, nslots, M, y_f32, pad_;
  int8_t tile_slot[kStreamMaxTiles];   // slot of the tile's variant, -1 for the base model
  uint8_t tile_valid[kStreamMaxTiles]; // rows of the tile that are real tokens (1..16)
  int16_t tile_src[kStreamMaxTiles];   // first x row of the tile
};
hipError_t launch_stream(const StreamArgs& a, int nblocks, hipStream_t stream);
size_t stream_lds_bytes(int ntiles, int nslots);

// Prefill: per-segment tiles of 256 tokens x 256 output rows, W_eff rebuilt in registers from
// raw weights staged in LDS.
constexpr int kPrefillBM = 256;
constexpr int kPrefillBN = 256;
constexpr int kPrefillMaxMTiles = 256;

struct PrefillArgs {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  int d_out, d_in, y_f32, n_mtiles, n_ntiles;
  int vec_signs;                       // bit s set: slot s's words may be read 16 bytes (4 steps)
                                       // at a time (d_in % 128 == 0 and tiled or 16-byte aligned
                                       // row-major words); bit 31: base-model tiles.  The kernel
                                       // reads quads when every bit is set, else single words
  unsigned alpha_rows;                 // bit s set: slot s has one alpha per output row
  unsigned tiled;                      // bit s set: slot s's words are in the 128-row tiled
                                       // layout (then its vec_signs bit is set)
  const uint32_t* words[kMaxSlots];
  const float* alpha[kMaxSlots];
  // per M-tile: first x row, rows in the tile (1..256), variant slot (-1 = base)
  int mt_row[kPrefillMaxMTiles];
  int16_t mt_rows[kPrefillMaxMTiles];
  int8_t mt_slot[kPrefillMaxMTiles];
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Decode with the sign product on fp4 x fp6 MFMA.  A prologue kernel writes, per launch chunk,
// the bf16 activations and the variant-scaled activations x' = alpha_v * x as two fp6 (e2m3)
// terms with per-32-column block scales, in operand layouts, into caller workspace.  Needs
// d_in % 128 == 0 and the tiled sign words.  One launch serves the tokens of at most 16 aligned
// 16-token blocks and at most kMaxSlots distinct variants, with at most kSplitMaxGroups slot
// groups per wave.
constexpr int kSplitMaxM = 256;
constexpr int kSplitRows = 128;
constexpr int kSplitMaxGroups = 8;

struct SplitProblem {
  const unsigned char* x;     // bf16 activations in base-operand order (prologue layout)
  const unsigned char* xq;    // fp6 hi/lo terms of alpha * x in sign-operand order
  const unsigned char* xs;    // E8M0 block scales of the two terms
  const float* xc;            // [nsteps][Mp] per step and token: sum of x' over the unsigned columns
  const uint16_t* w;
  void* y;                    // [M][d_out] of the whole call
  int d_out, d_in;
  int nblocks;                // 128-row blocks of this linear
  unsigned alpha_rows;        // bit s set: slot s has one alpha per output row (alpha[s][row])
  const uint32_t* words[kMaxSlots];  // tiled sign words (128-row layout)
  const float* alpha[kMaxSlots];     // per-row scales of the slots in alpha_rows (else unused)
};

// Per-wave work of a split launch.  32-bit fields: the kernel reads them with scalar loads
// indexed by the wave, whose addresses must stay 4-byte aligned.
struct SplitWave {
  int32_t tile[2];                       // 16-token block (relative) of the dense tiles, -1 none
  int32_t slot[kSplitMaxGroups][2];      // slot group g: the variant slot of tile i's pair, -1 none
  int32_t copier;                        // this wave issues copy share `copier` (0..7 with two
                                         // tiles per wave, 0..3 with one), -1 none
  int32_t pad_;
};

// Work schedule of a split launch.  The 128-row blocks of the launch's linears, in launch order,
// are cut into 8 runs of about equal work (blocks times K steps), one per XCD, so that each
// linear's blocks, and the activations they multiply, are served by as few XCDs as the balance
// allows.  XCD x serves blocks first[q] .. first[q] + cnt[q] - 1 of linear q (its "units") and
// walks one list: first one piece per unit, linear by linear: steps [0, min(cut, ns)) of each of
// its units but the last `pooled` units of its last linear.  Then the pool: linear by linear, the
// steps [head, ns) of its cut units (head = min(cut, ns) < ns) in pieces of `sigma` steps, then
// its pooled units whole, also in pieces of `sigma` steps; pieces of the same steps of different
// units come one after another, so they run side by side and share the activations in L2.  A
// unit done in several pieces is "split": each piece leaves its fp32 sums in a partial slot, and
// the piece that finishes last adds the slots in piece order and writes y.  A split unit's counter
// (64 bits) holds in bits 0..7 the pieces counted in and in bits 8 + 6x .. 13 + 6x the pieces that
// ran on XCD x.  The XCD's split units use counters split0 .., its partial slots slot0 ...
struct SplitXcd {
  int16_t first[kMaxProblems];           // first row block of linear q this XCD serves
  int16_t cnt[kMaxProblems];             // row blocks of linear q it serves (0: none)
  int16_t cut;                           // steps of a unit's first piece (at most ns)
  int16_t pooled;                        // trailing units of its last linear done in the pool
  int16_t sigma;                         // pool piece length in K steps (>= 1)
  int16_t nheads, npool;                 // list lengths
  int16_t nsplit, nslot;                 // split units and partial slots
  int16_t split0, slot0;                 // its first split counter and first partial slot
  int16_t pad_;
};
struct SplitSched {
  SplitXcd x[8];
  uint32_t slot_bytes;                   // bytes of one partial slot (128 rows x 4 x Mp)
  int32_t pad_;
  float* partial;                        // partial slots of all XCDs
  uint64_t* counter;                     // finished pieces per split unit, all XCDs
  uint32_t* stats;                       // [0]: handoffs whose pieces ran on several XCDs
};

// The lists' counts of an XCD under its parameters, for linears with ns[q] K steps (q < nprob);
// returns the largest number of pieces of one unit.
__host__ __device__ inline int split_xcd_counts(const SplitXcd& X, int nprob, const int* ns,
                                                int* nheads, int* npool, int* nsplit, int* nslot) {
  int last = -1;
  for (int q = 0; q < nprob; ++q)
    if (X.cnt[q] > 0) last = q;
  int max_parts = 1;
  *nheads = *npool = *nsplit = *nslot = 0;
  for (int q = 0; q < nprob; ++q) {
    if (X.cnt[q] <= 0) continue;
    const int pooled = q == last ? X.pooled : 0;
    const int head = X.cut < ns[q] ? X.cut : ns[q];
    const int nh = X.cnt[q] - pooled, tail = ns[q] - head;
    const int tp = tail > 0 ? (tail + X.sigma - 1) / X.sigma : 0;
    const int pp = (ns[q] + X.sigma - 1) / X.sigma;
    const int ncut = tail > 0 ? nh : 0;
    *nheads += nh;
    *npool += ncut * tp + pooled * pp;
    *nsplit += ncut + pooled;
    *nslot += ncut * (1 + tp) + pooled * pp;
    if (ncut > 0 && 1 + tp > max_parts) max_parts = 1 + tp;
    if (pooled > 0 && pp > max_parts) max_parts = pp;
  }
  return max_parts;
}

// Piece kk of XCD X's list, for linears with ns[q] K steps (q < nprob): linear p (-1 past the
// end), row block rb, K steps [k0, k1); for a split unit (nparts > 1) its piece index, its split
// counter sid and its first partial slot slot0 (both counted over all XCDs).
struct SplitPiece {
  int p, rb, k0, k1, nparts, part, sid, slot0;
};
__host__ __device__ inline SplitPiece split_piece(const SplitXcd& X, int nprob, const int* ns,
                                                  int kk) {
  SplitPiece r = {-1, 0, 0, 0, 1, 0, 0, 0};
  const bool in_pool = kk >= X.nheads;
  if (in_pool) kk -= X.nheads;
  int last = -1;
#pragma unroll
  for (int q = 0; q < kMaxProblems; ++q)
    if (q < nprob && X.cnt[q] > 0) last = q;
  int sid_base = X.split0, slot_base = X.slot0;
#pragma unroll
  for (int q = 0; q < kMaxProblems; ++q) {
    if (q < nprob && X.cnt[q] > 0) {
      const int pooled = q == last ? X.pooled : 0;
      const int head = X.cut < ns[q] ? X.cut : ns[q];
      const int nh = X.cnt[q] - pooled;                  // units with a head piece
      const int tail = ns[q] - head;
      const int tp = tail > 0 ? (tail + X.sigma - 1) / X.sigma : 0;  // pool pieces of a cut unit
      const int pp = (ns[q] + X.sigma - 1) / X.sigma;                // pieces of a pooled unit
      const int ncut = tail > 0 ? nh : 0;
      if (r.p < 0) {
        if (!in_pool) {
          if (kk < nh) {
            r.p = q; r.rb = X.first[q] + kk; r.k0 = 0; r.k1 = head;
            if (tail > 0) {
              r.nparts = 1 + tp; r.part = 0; r.sid = sid_base + kk; r.slot0 = slot_base + kk * r.nparts;
            }
          } else {
            kk -= nh;
          }
        } else if (kk < ncut * tp) {  // same steps of the cut units one after another
          const int jj = kk / ncut, u = kk - jj * ncut;
          r.p = q; r.rb = X.first[q] + u; r.k0 = head + jj * X.sigma;
          r.k1 = r.k0 + X.sigma < ns[q] ? r.k0 + X.sigma : ns[q];
          r.nparts = 1 + tp; r.part = 1 + jj; r.sid = sid_base + u; r.slot0 = slot_base + u * r.nparts;
        } else {
          kk -= ncut * tp;
          if (kk < pooled * pp) {
            const int jj = kk / pooled, u = kk - jj * pooled;
            r.p = q; r.rb = X.first[q] + nh + u; r.k0 = jj * X.sigma;
            r.k1 = r.k0 + X.sigma < ns[q] ? r.k0 + X.sigma : ns[q];
            r.nparts = pp; r.part = jj; r.sid = sid_base + ncut + u;
            r.slot0 = slot_base + ncut * (1 + tp) + u * pp;
          } else {
            kk -= pooled * pp;
          }
        }
      }
      sid_base += ncut + pooled;
      slot_base += ncut * (1 + tp) + pooled * pp;
    }
  }
  return r;
}

struct SplitArgs {
  SplitProblem prob[kMaxProblems];
  int nprob, nslots, y_f32;
  int tok_base;                          // first token of this launch's 16-token blocks
  int lo, hi;                            // tokens [tok_base + lo, tok_base + hi) are this launch's
  int Mp, pad_;                          // token count of the layouts (call's M rounded up to 16)
  SplitSched sch;
  SplitWave wv[8];
  int8_t token_slot[kSplitMaxM];         // slot of token tok_base + t (-1 = base model); read per lane
};
// nd: dense tiles per wave (1 or 2); ng: slot groups per wave (at most kSplitMaxGroups).  A launch
// with per-row slots (any alpha_rows bit) needs nd == 1.
hipError_t launch_split(const SplitArgs& a, int nd, int ng, hipStream_t stream);

// What the schedule of a split launch depends on: the linears (in launch order) with ns K steps
// and nb row blocks, C compute units per XCD, the batch Mp, the launch's variant count and the
// partial slots per XCD the workspace holds.
struct SplitShape {
  int np, C, Mp, nslots, slots_avail;
  int ns[kMaxProblems], nb[kMaxProblems];
};
// head, pooled, sigma and the list counts (partial, counter and slot_bytes are left 0).
SplitSched split_schedule(const SplitShape& sh);
// The simulated makespan of a schedule, in K steps (for tests).
double split_schedule_makespan(const SplitShape& sh, const SplitSched& h);
int split_compute_units();  // compute units of the current device

struct SplitActArgs {
  const uint16_t* x[kMaxProblems];     // bf16 [M][d_in] row-major (the caller's activations)
  unsigned char* xb[kMaxProblems];     // out: bf16 in base-operand order
  unsigned char* xq[kMaxProblems];     // out: fp6 hi/lo terms of alpha * x in sign-operand order
  unsigned char* xs[kMaxProblems];     // out: their block scales
  float* xc[kMaxProblems];             // out: per step and token, the correction sums
  const float* alpha[kMaxProblems][kMaxSlots];  // null: the slot's tokens take x' = x (per-row
                                               // scales are applied by the main kernel)
  int d_in[kMaxProblems];
  int Mp, tok_base, lo, hi, nprob, pad_;  // tokens [tok_base + lo, tok_base + hi)
  uint64_t* counter;                   // out: ncounter split counters set to zero
  int ncounter, pad2_;
  int8_t token_slot[kSplitMaxM];       // slot of token tok_base + t (-1 = base model); read per lane
};
hipError_t launch_split_act(const SplitActArgs& a, hipStream_t stream);
// Workspace of one linear: bf16 pieces, fp6 pieces, scales, correction sums, and its share of
// the call's partial slots and split counters (kSplitSlotsPerLinear of each) and a 256-byte
// statistics block; each part a multiple of 256 bytes.
constexpr int kSplitSlotsPerLinear = 128;
size_t split_workspace_bytes(int64_t M, int64_t d_in);
void split_workspace_parts(int64_t M, int64_t d_in, size_t* xb_bytes, size_t* xq_bytes,
                           size_t* xs_bytes, size_t* xc_bytes);
size_t split_partial_bytes(int64_t M);   // one linear's share of partial slots, counters, stats
constexpr size_t kSplitCounterBytes = (size_t)kSplitSlotsPerLinear * 8;  // per linear
constexpr size_t kSplitStatsBytes = 256;                                 // per linear
size_t split_slot_bytes(int64_t M);      // one partial slot

}  // namespace bd
