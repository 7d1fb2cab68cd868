// Multi-variant decode with the sign product on the fp4 x fp8 matrix cores: the fused
// reconstruct-and-multiply of the BitDelta post ("Serving architecture") for a token batch
// grouped by variant, with W_base read from HBM once for the whole batch and each active
// variant's sign bits read once.
//
// For a token t of variant v and output row r,
//     y[t][r] = sum_k x[t][k] * w[r][k]  +  alpha_v * sum_k x[t][k] * s_v[r][k],   s = +-1.
// The two sums are computed separately and W_eff is never formed:
//   * base sum: bf16 x bf16 MFMA (v_mfma_f32_16x16x32_bf16) over DENSE 16-token tiles of the
//     batch (the base weights are the same for every token);
//   * sign sum: per 16-token tile of one variant, v_mfma_scale_f32_16x16x128_f8f6f4 with the
//     signs as fp4 (e2m1) +-1.0 and the activations as two fp8 (e4m3) terms, x = 2^e * (hi +
//     lo / 16), e one power of two per token (the E8M0 block scale of the instruction).  A bf16
//     value has 8 significant bits and hi carries the leading 4 (round to nearest), so the
//     remainder x - hi has at most 4 significant bits and lo holds it exactly: every product
//     is exact and accumulation is fp32, as in the bf16 path, except for elements smaller than
//     2^-14 of their token's largest magnitude, whose remainder may lose bits in fp8's subnormal
//     range (absolute error below 2^-22 of that largest magnitude).
// A sign word of 32 bits becomes the fp4 operand with one shift and one 3-input bit operation
// per 8 weights, instead of the 2 operations per 2 weights a bf16 +-1 operand costs.
//
// K order.  Inside one 128-wide K step the instruction's lane group G (lanes 16G..16G+15) holds
// K positions 32G..32G+31 of the fp4 operand, nibble n of dword d being position 32G + 8d + n.
// That position is mapped to weight column 32G + 4n + d, i.e. bit 4n + d of sign word G of the
// step, so dword d of the operand is ((word << (3 - d)) & 0x88888888) ^ 0xAAAAAAAA (0x2 = +1.0,
// 0xA = -1.0).  The fp8 operand's lane group G holds positions 16G..16G+15 and 64+16G..64+16G+15;
// the activation prologue writes each token's fp8 bytes in exactly that order, with the same
// position-to-column map, so both operands agree on every product.
//
// Work split.  A workgroup (8 waves, two per SIMD) owns 64 output rows of one linear.  Wave w
// owns dense tiles w and w+8 (base sum, ND per wave) and variant tiles [w*NS, w*NS+NS) (sign
// sum).  The K loop walks d_in in steps of 128:
//   * W_base (64 rows x 128, 16 KiB) and the sign words of every active variant (the tiled
//     copy: 64 rows x 16 B = 1 KiB contiguous per variant and step) are copied by direct
//     global->LDS loads (16 bytes per lane, whole cache lines) three steps ahead into a 4-stage
//     ring; W_base's 16-byte chunks are XOR-swizzled by row so MFMA operand reads are
//     conflict-free;
//   * each wave's activations (bf16 for dense tiles, fp8 hi/lo for variant tiles) go straight
//     from memory into MFMA B-operand registers, reloaded for the next step right after use;
//   * one workgroup barrier per step; before it each wave waits only for its copies that the
//     next step reads, never for the activation loads in flight.
// Epilogue: alpha_v * sign sum goes through LDS to the wave that owns the token's dense tile,
// which adds it to the base sum and stores y as bf16 (nearest-even) or fp32.
#include <type_traits>

#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kSplitRows;        // 64 output rows per workgroup
constexpr int kRT = kRows / 16;          // row tiles
constexpr int kKS = 128;                 // k per step
constexpr unsigned kWStage = kRows * kKS * 2;        // 16 KiB of W_base per step
constexpr unsigned kSSlot = kRows * 16;              // one variant's sign words, one step: 1 KiB
constexpr unsigned kStage = kWStage + kMaxSlots * kSSlot;  // W_base + signs of one step: 32 KiB
constexpr int kStages = 4;                           // LDS ring; copies run kStages-1 steps ahead
constexpr int kAhead = kStages - 1;
constexpr unsigned kLdsBytes = kStages * kStage;     // 128 KiB
constexpr int kEStride = kRows + 4;                  // floats per token row of the epilogue buffer
static_assert(kSplitMaxM * kEStride * 4 <= (int)kLdsBytes, "epilogue buffer exceeds LDS");

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp4 (e2m1) A operand x fp8 (e4m3) B operand, K = 128, B scaled by 2^(scale_b - 127).
__device__ __forceinline__ f32x4 mfma_sign(const u32x4& a, const i32x8& b, int scale_b,
                                           const f32x4& c) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 0, 0, 127, 0, scale_b);
}

// The 32 sign bits of one row and one 32-column group -> fp4 +-1.0 in the K order above.
__device__ __forceinline__ u32x4 expand_fp4(unsigned w) {
  u32x4 r;
  r[0] = ((w << 3) & 0x88888888u) ^ 0xAAAAAAAAu;
  r[1] = ((w << 2) & 0x88888888u) ^ 0xAAAAAAAAu;
  r[2] = ((w << 1) & 0x88888888u) ^ 0xAAAAAAAAu;
  r[3] = (w & 0x88888888u) ^ 0xAAAAAAAAu;
  return r;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + 2^31): offsets past the end read as zero, and every
// offset the kernel forms stays inside the tensor it addresses.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// 16 bytes per lane from base + voff straight into LDS at lds_base + 16 * lane.  The buffer
// (MUBUF) form is used rather than the global one so the compiler's wait-count tracking of the
// other loads stays exact; the copies themselves are waited for explicitly before barriers.
__device__ __forceinline__ void dma16(rsrc_t r, unsigned voff, unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// 16 bytes from a raw buffer; an offset at or past kOob reads as zero without touching memory.
constexpr unsigned kOob = 0x80000000u;
__device__ __forceinline__ u32x4 load16(rsrc_t r, unsigned voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding).
#define SPLIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier; the empty asm statements keep the compiler from moving memory accesses
// across it.  Visibility of LDS written by direct copies is ensured by the vmcnt wait before.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int ND, int NS>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(const SplitArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- which linear and which 64-row block (wave-uniform) ------------------------------------
  // Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD b % 8).  XCD x
  // serves the x-th eighth of every linear's row blocks, consecutively, so the workgroups that
  // run side by side on one XCD (sharing its L2) read the same activations at the same time.
  const int xcd = blockIdx.x & 7;
  int kk = blockIdx.x >> 3, p = -1, rb = 0;
#pragma unroll
  for (int q = 0; q < kMaxProblems; ++q) {
    if (q < a.nprob && p < 0) {
      const int n = a.prob[q].nblocks;
      const int lo = (xcd * n) >> 3, len = (((xcd + 1) * n) >> 3) - lo;
      if (kk < len) {
        p = q;
        rb = lo + kk;
      } else {
        kk -= len;
      }
    }
  }
  if (p < 0) return;  // this XCD's list is shorter than the longest one
  const SplitProblem& P = a.prob[p];
  const int d_in = P.d_in, d_out = P.d_out;
  const int row0 = rb * kRows;
  const int T = a.ntiles;
  const int nslots = a.nslots;
  const int nsteps = d_in / kKS;
  const int lo_tok = a.lo, hi_tok = a.hi;      // valid tokens, relative to a.tok_base

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;

  // ---- direct copies (global -> LDS), kAhead steps ahead, into stage s % kStages ---------------
  // W_base: copy b = 2*wave + u (of 16) moves rows 4b..4b+3 of the block for one step, 256 bytes
  // each, so every 4 consecutive lanes read 64 contiguous bytes.  Lane L writes LDS slot
  // (row 4b + L/16, 16-byte position L%16) and fetches 16-byte column chunk position ^ (row%16):
  // the XOR swizzle keeps the MFMA operand reads below conflict-free.
  const rsrc_t wrs = make_rsrc(P.w + (size_t)row0 * d_in);
  unsigned woff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rl = 4 * (2 * wave + u) + (lane >> 4);
    const int row = min(row0 + rl, d_out - 1) - row0;
    woff[u] = (unsigned)((row * d_in + 8 * ((lane & 15) ^ (rl & 15))) * 2);
  }
  // sign words (tiled layout): the 64 rows of this block for one step are 1 KiB contiguous at
  // word ((row0 / 128) * nsteps + s) * 512 + (row0 % 128) * 4; copy of slot wave + 8u.
  rsrc_t srs[2];
  bool sreal[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int slot = wave + kWaves * u;
    sreal[u] = slot < nslots;
    srs[u] = make_rsrc(P.words[sreal[u] ? slot : 0]);
  }
  const unsigned soff = (unsigned)((((row0 >> 7) * nsteps) * 512 + (row0 & 127) * 4) * 4) + lane * 16;
  auto issue = [&](int s) {  // copies for step s
    if (s < nsteps) {
      unsigned char* st = smem + (unsigned)(s % kStages) * kStage;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dma16(wrs, woff[u] + (unsigned)s * (kKS * 2), st + (2 * wave + u) * 1024);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (sreal[u])
          dma16(srs[u], soff + (unsigned)s * 2048, st + kWStage + (wave + kWaves * u) * kSSlot);
    }
  };

  // ---- activations: the prologue's layouts ------------------------------------------------------
  // Piece (s, o, g) of token t is 16 bytes at (((s * 4 + o) * nblk + t / 16) * 4 + g) * 256 +
  // (t % 16) * 16, nblk = Mp / 16: the 64 lanes of a 16-token aligned block read 1 KiB in lane
  // order.  o = bf16 chunk c for the base operand, o = 2 part + half for the fp8 terms.
  const rsrc_t xrs = make_rsrc(P.x);
  const rsrc_t qrs = make_rsrc(P.xq);
  const unsigned ostep = (unsigned)a.Mp * 64;   // bytes between consecutive o (= nblk KiB)
  const int tb0 = a.tok_base >> 4;              // first 16-token block of this launch
  unsigned xoff[ND];
  bool dreal[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int tile = wave + kWaves * i;
    const int t = 16 * tile + j;                // relative to tok_base
    dreal[i] = 16 * tile < hi_tok;
    xoff[i] = (t >= lo_tok && t < hi_tok) ? (unsigned)(tb0 + tile) * 1024 + (unsigned)lane * 16
                                          : kOob;
  }
  unsigned qoff[NS];
  int sc_hi[NS], sc_lo[NS];
  unsigned tslot[NS];
  bool treal[NS], tnew[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int ti_raw = wave * NS + i;
    const int ti = max(0, min(ti_raw, T - 1));  // T == 0: a batch of base-model tokens only
    const int valid = a.tile_valid[ti];
    const int tr = max(lo_tok, min(a.tile_src[ti] + j, hi_tok - 1));  // relative token
    const int t = a.tok_base + tr;
    // lanes past the tile's tokens read zeros without touching memory
    qoff[i] = (ti_raw < T && j < valid)
                  ? (unsigned)(t >> 4) * 1024 + (unsigned)g * 256 + (unsigned)(t & 15) * 16
                  : kOob;
    sc_hi[i] = P.xscale[t];
    sc_lo[i] = sc_hi[i] - 4;
    const int s = a.tile_slot[ti];
    tslot[i] = __builtin_amdgcn_readfirstlane((unsigned)s * kSSlot);
    treal[i] = ti_raw < T;
    tnew[i] = i == 0 || a.tile_slot[max(0, min(ti_raw - 1, T - 1))] != s;
  }

  // ---- registers ------------------------------------------------------------------------------------
  u32x4 xb[ND][4];           // bf16 activations of the dense tiles, 4 chunks of 32 columns
  i32x8 xh[NS], xl[NS];      // fp8 hi / lo activations of the variant tiles
  f32x4 accb[ND][kRT], accd[NS][kRT];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) accb[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) accd[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_xb = [&](int i, unsigned s) {
#pragma unroll
    for (int c = 0; c < 4; ++c) xb[i][c] = load16(xrs, xoff[i] + (s * 4 + c) * ostep);
  };
  // hi (part 0) or lo (part 1) fp8 term of variant tile i at step s: 32 bytes per lane
  auto load_xq_part = [&](int i, unsigned s, int part) {
    const unsigned o = qoff[i] + (s * 4 + 2 * part) * ostep;
    const u32x4 v0 = load16(qrs, o);
    const u32x4 v1 = load16(qrs, o + ostep);
    const i32x8 v = {(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                     (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
    if (part == 0) xh[i] = v;
    else xl[i] = v;
  };
  // vector-memory instructions per step that are activation loads
  constexpr int kX = 4 * ND + 4 * NS;

  // ---- prologue: stages 0..kAhead-1 and the activations of step 0 ------------------------------
#pragma unroll
  for (int s = 0; s < kAhead; ++s) issue(s);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < ND; ++i) load_xb(i, 0);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    load_xq_part(i, 0, 0);
    load_xq_part(i, 0, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  SPLIT_VMCNT(kX);
  raw_barrier();

  // per-lane LDS read offsets
  const unsigned a_lane = (unsigned)j * 256;                   // + stage + rt * 4096 + swizzled chunk
  const unsigned s_lane = kWStage + (unsigned)(j * 16 + 4 * g);  // + stage + slot + rt * 256

  u32x4 S[kRT];
  for (int s = 0; s < nsteps; ++s) {
    issue(s + kAhead);
    __builtin_amdgcn_sched_barrier(0);

    // Each activation operand is reloaded for step s+1 right after its last use in step s, so
    // every load has about one step to arrive.
    const unsigned knext = (unsigned)min(s + 1, nsteps - 1);
    const unsigned st = (unsigned)(s % kStages) * kStage;

    // base sum over the dense tiles, 32-column chunk by chunk
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 A[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        A[rt] = *reinterpret_cast<const u32x4*>(smem + st + a_lane + rt * 4096 +
                                                 (((4 * c + g) ^ j) * 16));
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        if (dreal[i]) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) accb[i][rt] = mfma_bf16(A[rt], xb[i][c], accb[i][rt]);
        }
        xb[i][c] = load16(xrs, xoff[i] + (knext * 4 + c) * ostep);
      }
    }

    // sign sum over this wave's variant tiles: hi terms, then lo terms
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (treal[i]) {
        if (tnew[i]) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            S[rt] = expand_fp4(
                *reinterpret_cast<const unsigned*>(smem + st + s_lane + tslot[i] + rt * 256));
        }
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          accd[i][rt] = mfma_sign(S[rt], xh[i], sc_hi[i], accd[i][rt]);
      }
      load_xq_part(i, knext, 0);
      if (treal[i]) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          accd[i][rt] = mfma_sign(S[rt], xl[i], sc_lo[i], accd[i][rt]);
      }
      load_xq_part(i, knext, 1);
    }

    // Before the barrier, each wave waits for its copies of step s+1 (issued at least two steps
    // ago, with at least 2 kX activation loads after them) but not for newer loads.
    __builtin_amdgcn_sched_barrier(0);
    SPLIT_VMCNT(2 * kX);
    raw_barrier();
  }

  // ---- epilogue ---------------------------------------------------------------------------------------
  // alpha_v * sign sum -> E[token][row] (fp32, row stride kEStride); the LDS ring is dead.
  float* E = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int ti = wave * NS + i;
    if (ti < T) {
      const float al = *P.alpha[a.tile_slot[ti]];
      if (j < (int)a.tile_valid[ti]) {
        float* e = E + (a.tile_src[ti] + j) * kEStride + 4 * g;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const f32x4 v = {al * accd[i][rt][0], al * accd[i][rt][1], al * accd[i][rt][2],
                           al * accd[i][rt][3]};
          *reinterpret_cast<f32x4*>(e + rt * 16) = v;
        }
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

  const bool vec_store = (d_out & 3) == 0;  // y rows start on 4-element boundaries
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int tr = 16 * (wave + kWaves * i) + j;  // relative token
    if (!dreal[i] || tr < lo_tok || tr >= hi_tok) continue;
    const bool hd = (a.has_delta[tr >> 5] >> (tr & 31)) & 1u;
    const float* e = E + tr * kEStride + 4 * g;
    const size_t ybase = (size_t)(a.tok_base + tr) * d_out;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int orow = row0 + rt * 16 + 4 * g;
      f32x4 v = accb[i][rt];
      if (hd) v += *reinterpret_cast<const f32x4*>(e + rt * 16);
      if (a.y_f32) {
        float* y = reinterpret_cast<float*>(P.y) + ybase;
        if (vec_store && orow + 3 < d_out) {
          *reinterpret_cast<f32x4*>(y + orow) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (orow + r < d_out) y[orow + r] = v[r];
        }
      } else {
        uint16_t* y = reinterpret_cast<uint16_t*>(P.y) + ybase;
        if (vec_store && orow + 3 < d_out) {
          u32x2 pk;
          pk[0] = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
          pk[1] = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<u32x2*>(y + orow) = pk;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (orow + r < d_out) y[orow + r] = (uint16_t)f32_to_bf16_rne(v[r]);
        }
      }
    }
  }
}

// ---- activation prologue: x (bf16) -> the kernel's operand layouts ----------------------------
// One workgroup per (token, linear).  Pass 1: the token's largest magnitude m; the fp8 scale is
// 2^e with e = ceil(log2 m) - 8, so |x| * 2^-e <= 256 < 448 (the largest e4m3 value).  Pass 2:
// one thread per 128-column step writes, in 1 KiB blocks of 16 tokens (piece (s, o, g) of token
// t at (((s * 4 + o) * Mp / 16 + t / 16) * 4 + g) * 256 + (t % 16) * 16),
//   * the bf16 activations in base-operand order: piece (s, c, g) = columns 128s+32c+8g..+7;
//   * hi = e4m3(v) and lo = e4m3(16 (v - hi)), v = x * 2^-e, each rounded to nearest even, in
//     sign-operand order: piece (s, 2 part + half, g) = bytes 16 half..16 half+15 of lane group
//     g's 32 fp8 values (part 0 = hi, 1 = lo), operand positions mapped to columns as above.
constexpr int kActThreads = 128;

__device__ __forceinline__ int col_of_position(int h) {  // operand position -> column, one step
  return 32 * (h >> 5) + 4 * (h & 7) + ((h >> 3) & 3);
}

__global__ __launch_bounds__(kActThreads) void split_act_kernel(const SplitActArgs a) {
  __shared__ float red[kActThreads / 64];
  const int t = blockIdx.x, p = blockIdx.y;
  const int d_in = a.d_in[p];
  const uint16_t* __restrict__ x = a.x[p] + (size_t)t * d_in;
  const size_t ostep = (size_t)a.Mp * 64;  // bytes between consecutive (s, o) block rows
  const size_t tpos = (size_t)(t >> 4) * 1024 + (size_t)(t & 15) * 16;
  unsigned char* __restrict__ xb = a.xb[p] + tpos;
  unsigned char* __restrict__ q = a.xq[p] + tpos;
  const int tid = threadIdx.x;

  float m = 0.f;
  for (int i = tid; i < d_in / 8; i += kActThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + 8 * i);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      m = fmaxf(m, fabsf(bf16lo_to_f32(v[d])));
      m = fmaxf(m, fabsf(bf16hi_to_f32(v[d])));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kActThreads / 64; ++w) m = fmaxf(m, red[w]);

  // e = ceil(log2 m) - 8, limited to [-123, 120] (lo's scale e - 4 must stay >= -127)
  const unsigned mb = __float_as_uint(m);
  const int ex = (int)(mb >> 23) - 127;
  int e = ex + ((mb & 0x7FFFFFu) != 0u ? 1 : 0) - 8;
  if (m == 0.f || ex == -127) e = -123;
  e = max(-123, min(120, e));
  if (tid == 0) a.xscale[p][t] = e + 127;
  const float inv = __uint_as_float((unsigned)(127 - e) << 23);  // 2^-e, a normal float

  const int nsteps = d_in / 128;
  for (int s = tid; s < nsteps; s += kActThreads) {
    unsigned v[64];  // bf16 pairs of columns 128 s .. 128 s + 127
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(x + (size_t)s * 128 + 8 * i);
      v[4 * i] = c[0];
      v[4 * i + 1] = c[1];
      v[4 * i + 2] = c[2];
      v[4 * i + 3] = c[3];
      // bf16 piece (s, c = i / 4, g = i % 4): columns 8i..8i+7
      *reinterpret_cast<u32x4*>(xb + ((size_t)s * 4 + (i >> 2)) * ostep + (size_t)(i & 3) * 256) = c;
    }
    unsigned hi[32], lo[32];
#pragma unroll
    for (int o = 0; o < 32; ++o) {  // output dword o: group o / 8, half (o / 4) % 2, dword o % 4
      const int G = o >> 3, half = (o >> 2) & 1, dw = o & 3;
      float f[4], r[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int h = (half ? 64 : 0) + 16 * G + 4 * dw + b;
        const int col = col_of_position(h);
        const unsigned pair = v[col >> 1];
        f[b] = ((col & 1) ? bf16hi_to_f32(pair) : bf16lo_to_f32(pair)) * inv;
      }
      unsigned hw = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      hw = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], (int)hw, true);
      r[0] = (f[0] - __builtin_amdgcn_cvt_f32_fp8((int)hw, 0)) * 16.f;
      r[1] = (f[1] - __builtin_amdgcn_cvt_f32_fp8((int)hw, 1)) * 16.f;
      r[2] = (f[2] - __builtin_amdgcn_cvt_f32_fp8((int)hw, 2)) * 16.f;
      r[3] = (f[3] - __builtin_amdgcn_cvt_f32_fp8((int)hw, 3)) * 16.f;
      unsigned lw = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
      lw = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], (int)lw, true);
      hi[o] = hw;
      lo[o] = lw;
    }
#pragma unroll
    for (int G = 0; G < 4; ++G)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int o = 8 * G + 4 * half;
        *reinterpret_cast<u32x4*>(q + ((size_t)s * 4 + half) * ostep + (size_t)G * 256) =
            u32x4{hi[o], hi[o + 1], hi[o + 2], hi[o + 3]};
        *reinterpret_cast<u32x4*>(q + ((size_t)s * 4 + 2 + half) * ostep + (size_t)G * 256) =
            u32x4{lo[o], lo[o + 1], lo[o + 2], lo[o + 3]};
      }
  }
}

template <int ND, int NS>
hipError_t launch_nd_ns(const SplitArgs& a, int nblocks, hipStream_t stream) {
  static bool configured = false;  // benign race: every caller sets the same value
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&split_kernel<ND, NS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL((split_kernel<ND, NS>), dim3(nblocks), dim3(kThreads), kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace

size_t split_workspace_bytes(int64_t M, int64_t d_in) {
  const size_t mp = (size_t)((M + 15) / 16) * 16;
  const size_t q = mp * 2 * (size_t)d_in;            // bf16 copy, and fp8 hi + lo, per element
  const size_t s = mp * sizeof(int);                 // scale code per token
  return 2 * ((q + 255) / 256) * 256 + ((s + 255) / 256) * 256;
}

hipError_t launch_split_act(const SplitActArgs& a, int M, int nprob, hipStream_t stream) {
  if (M <= 0 || nprob <= 0 || nprob > kMaxProblems) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_act_kernel, dim3(M, nprob), dim3(kActThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
  if (a.hi < 1 || a.hi > kSplitMaxM || a.lo < 0 || a.lo >= a.hi || (a.tok_base & 15) != 0 ||
      a.ntiles < 0 || a.ntiles > kSplitMaxTiles ||
      a.nslots < 0 || a.nslots > kMaxSlots || a.nprob < 1 || a.nprob > kMaxProblems)
    return hipErrorInvalidValue;
  // grid: 8 XCD lists, each as long as the longest (see the block map in the kernel)
  int longest = 0;
  for (int x = 0; x < 8; ++x) {
    int len = 0;
    for (int q = 0; q < a.nprob; ++q) {
      if (a.prob[q].nblocks < 1) return hipErrorInvalidValue;
      len += (((x + 1) * a.prob[q].nblocks) >> 3) - ((x * a.prob[q].nblocks) >> 3);
    }
    longest = len > longest ? len : longest;
  }
  const int nblocks = 8 * longest;
  const int nd = (a.hi + 16 * kWaves - 1) / (16 * kWaves);  // 1 or 2
  const int ns = a.ntiles == 0 ? 1 : (a.ntiles + kWaves - 1) / kWaves;  // 1..3
  if (nd == 1) {
    if (ns == 1) return launch_nd_ns<1, 1>(a, nblocks, stream);
    if (ns == 2) return launch_nd_ns<1, 2>(a, nblocks, stream);
    return launch_nd_ns<1, 3>(a, nblocks, stream);
  }
  if (ns == 1) return launch_nd_ns<2, 1>(a, nblocks, stream);
  if (ns == 2) return launch_nd_ns<2, 2>(a, nblocks, stream);
  return launch_nd_ns<2, 3>(a, nblocks, stream);
}

}  // namespace bd
