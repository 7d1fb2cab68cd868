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
//   * W_base (64 rows x 128, 16 KiB) is copied by direct global->LDS loads (16 bytes per lane)
//     four steps ahead into a 5-stage ring (64 KiB in flight per CU to cover HBM latency),
//     laid out so each MFMA A operand is 1 KiB of consecutive lanes (conflict-free reads);
//   * the sign words of every active variant (16 bytes per row per step) are copied the same
//     way, two steps (32 bytes per row) at a time, into a 2-group ring;
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
#ifndef SPLIT_WSTAGES
#define SPLIT_WSTAGES 5
#endif
#ifndef SPLIT_DMA_AUX
#define SPLIT_DMA_AUX 0
#endif
constexpr int kWStages = SPLIT_WSTAGES;             // W ring depth; copies run kWStages-1 ahead
constexpr int kWAhead = kWStages - 1;
constexpr unsigned kSBase = kWStages * kWStage;      // sign-word ring after the W ring
constexpr unsigned kSSlotG = kRows * 32;             // one slot, one two-step group: 64 rows x 32 B
constexpr unsigned kSGroup = kMaxSlots * kSSlotG;    // one group, every slot
constexpr unsigned kLdsBytes = kSBase + 2 * kSGroup; // 144 KiB with 5 W stages
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
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, SPLIT_DMA_AUX);
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
  const uint16_t* __restrict__ xg = P.x;
  const unsigned char* __restrict__ qg = P.xq;
  const uint16_t* __restrict__ wg = P.w;
  const int d_in = P.d_in, d_out = P.d_out;
  const int row0 = rb * kRows;
  const int M = a.M;
  const int T = a.ntiles;
  const int nslots = a.nslots;
  const int wpr = d_in >> 5;
  const int nsteps = d_in / kKS;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;

  // ---- direct copies this wave issues ----------------------------------------------------------
  // Offsets are relative to row row0 of the block; rows past d_out are clamped to d_out - 1.
  // W_base: copy b = 2*wave + u (of 16) moves rows 4b..4b+3 of the block for one step, 256 bytes
  // each, so every 4 consecutive lanes read 64 contiguous bytes.  Lane L writes LDS slot
  // (row 4b + L/16, 16-byte position L%16) and fetches 16-byte column chunk position ^ (row%16):
  // the XOR swizzle keeps the MFMA operand reads below conflict-free.
  const rsrc_t wrs = make_rsrc(wg + (size_t)row0 * d_in);
  unsigned woff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rl = 4 * (2 * wave + u) + (lane >> 4);
    const int row = min(row0 + rl, d_out - 1) - row0;
    woff[u] = (unsigned)((row * d_in + 8 * ((lane & 15) ^ (rl & 15))) * 2);
  }
  // sign words of a two-step group: copy c = wave + 8u (c < 2 * nslots) moves rows 32h..32h+31
  // (h = c % 2) of slot c / 2; lane L takes row 32h + L/2, step 2G + L%2 (16 bytes), so every two
  // lanes read 32 contiguous bytes.  LDS per slot and group: [64 rows][2 steps][16 B].
  const int sq = lane & 1;  // step of the group this lane copies
  rsrc_t srs[4];
  unsigned soff[4], sdst[4];
  bool sreal[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = wave + kWaves * u;
    sreal[u] = c < 2 * nslots;
    const int cc = sreal[u] ? c : 0;
    const int slot = cc >> 1, h = cc & 1;
    srs[u] = make_rsrc(a.prob[p].words[slot] + (size_t)row0 * wpr);
    soff[u] = (unsigned)((min(row0 + 32 * h + (lane >> 1), d_out - 1) - row0) * wpr * 4);
    sdst[u] = kSBase + (unsigned)slot * kSSlotG + (unsigned)h * 1024;
  }
  auto issue_w = [&](int s) {
    if (s < nsteps) {
      unsigned char* dst = smem + (unsigned)(s % kWStages) * kWStage;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dma16(wrs, woff[u] + (unsigned)s * (kKS * 2), dst + (2 * wave + u) * 1024);
    }
  };
  auto issue_signs = [&](int grp) {  // steps 2*grp, 2*grp + 1 (the second clamped at the end)
    if (2 * grp >= nsteps) return;
    const unsigned ring = (unsigned)(grp & 1) * kSGroup;
    const unsigned step = (unsigned)min(2 * grp + sq, nsteps - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sreal[u]) dma16(srs[u], soff[u] + step * 16, smem + ring + sdst[u]);
  };

  // ---- this wave's tiles --------------------------------------------------------------------------
  // Activations come from the prologue's layouts, token-major inside each (step, piece): piece
  // (s, r, g) of token t is 16 bytes at ((s * 16 + r) * Mp + t) * 16, with r = 4c + g for the bf16
  // chunk c of the base product and r = 8 part + 4 half + g for the fp8 terms, so the 16 lanes of
  // a lane group read 16 consecutive tokens (256 contiguous bytes).
  // dense tiles (base sum): tokens 16*(wave + 8i) + j; lanes past the batch read zeros
  const rsrc_t xrs = make_rsrc(xg);
  const rsrc_t qrs = make_rsrc(qg);
  const unsigned mp16 = (unsigned)a.Mp * 16;   // bytes between pieces of one token
  unsigned xoff[ND];
  bool dreal[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int tile = wave + kWaves * i;
    dreal[i] = 16 * tile < M;
    const int t = 16 * tile + j;
    xoff[i] = t < M ? (unsigned)g * mp16 + (unsigned)(a.tok0 + t) * 16 : kOob;
  }
  // variant tiles (sign sum)
  unsigned qoff[NS];
  int sc_hi[NS], sc_lo[NS];
  unsigned tslot[NS];
  bool treal[NS], tnew[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int ti_raw = wave * NS + i;
    const int ti = max(0, min(ti_raw, T - 1));  // T == 0: a batch of base-model tokens only
    const int valid = a.tile_valid[ti];
    // lanes past the tile's tokens read zeros without touching memory
    const int tok = a.tok0 + max(0, min(a.tile_src[ti] + j, M - 1));
    qoff[i] = (ti_raw < T && j < valid) ? (unsigned)g * mp16 + (unsigned)tok * 16 : kOob;
    sc_hi[i] = P.xscale[tok];
    sc_lo[i] = sc_hi[i] - 4;
    const int s = a.tile_slot[ti];
    tslot[i] = __builtin_amdgcn_readfirstlane((unsigned)s * kSSlotG);
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

  auto load_xb = [&](int i, int s) {
    const unsigned ks = (unsigned)min(s, nsteps - 1) * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c) xb[i][c] = load16(xrs, xoff[i] + (ks + 4 * c) * mp16);
  };
  // hi (part 0) or lo (part 1) fp8 term of variant tile i at step s: 32 bytes per lane
  auto load_xq_part = [&](int i, unsigned s, int part) {
    const unsigned o = qoff[i] + (s * 16 + (unsigned)part * 8) * mp16;
    const u32x4 v0 = load16(qrs, o);
    const u32x4 v1 = load16(qrs, o + 4 * mp16);
    const i32x8 v = {(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                     (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
    if (part == 0) xh[i] = v;
    else xl[i] = v;
  };
  auto load_xq = [&](int i, int s) {
    load_xq_part(i, (unsigned)min(s, nsteps - 1), 0);
    load_xq_part(i, (unsigned)min(s, nsteps - 1), 1);
  };
  // vector-memory instructions per step that are activation loads
  constexpr int kX = 4 * ND + 4 * NS;

  // ---- prologue: stage 0 and 1 of W, sign group 0, activations of step 0 ------------------------
  issue_w(0);
  issue_signs(0);
#pragma unroll
  for (int s = 1; s < kWAhead; ++s) issue_w(s);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < ND; ++i) load_xb(i, 0);
#pragma unroll
  for (int i = 0; i < NS; ++i) load_xq(i, 0);
  __builtin_amdgcn_sched_barrier(0);
  SPLIT_VMCNT(kX);
  raw_barrier();

  // per-lane LDS read offsets
  const unsigned a_lane = (unsigned)j * 256;                   // + stage + rt * 4096 + swizzled chunk
  const unsigned s_lane = (unsigned)(j * 32 + 4 * g);          // + ring + slot + rt * 512 + step * 16

  u32x4 S[kRT];
  for (int s = 0; s < nsteps; ++s) {
    issue_w(s + kWAhead);
    if ((s & 1) == 0) issue_signs((s >> 1) + 1);
    __builtin_amdgcn_sched_barrier(0);

    // Each activation operand is reloaded for step s+1 right after its last use in step s, so
    // every load has about one step to arrive.
    const unsigned knext = (unsigned)min(s + 1, nsteps - 1);

    // base sum over the dense tiles, 32-column chunk by chunk
    const unsigned wst = (unsigned)(s % kWStages) * kWStage + a_lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 A[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        A[rt] = *reinterpret_cast<const u32x4*>(smem + wst + rt * 4096 + (((4 * c + g) ^ j) * 16));
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        if (dreal[i]) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) accb[i][rt] = mfma_bf16(A[rt], xb[i][c], accb[i][rt]);
        }
        xb[i][c] = load16(xrs, xoff[i] + (knext * 16 + 4 * c) * mp16);
      }
    }

    // sign sum over this wave's variant tiles: hi terms, then lo terms
    const unsigned sst = kSBase + (unsigned)((s >> 1) & 1) * kSGroup + (unsigned)(s & 1) * 16 + s_lane;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (treal[i]) {
        if (tnew[i]) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            S[rt] = expand_fp4(*reinterpret_cast<const unsigned*>(smem + sst + tslot[i] + rt * 512));
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

    __builtin_amdgcn_sched_barrier(0);
    SPLIT_VMCNT(2 * kX);
    raw_barrier();
  }

  // ---- epilogue ---------------------------------------------------------------------------------------
  // alpha_v * sign sum -> E[token][row] (fp32, row stride kEStride); the W/sign rings are dead.
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
    const int t = 16 * (wave + kWaves * i) + j;
    if (!dreal[i] || t >= M) continue;
    const bool hd = (a.has_delta[t >> 5] >> (t & 31)) & 1u;
    const float* e = E + t * kEStride + 4 * g;
    const size_t ybase = (size_t)t * d_out;
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
// one thread per 128-column step writes, token-major inside each 16-byte piece slot,
//   * the bf16 activations in base-operand order: piece (s, 4c + g) = columns 128s+32c+8g..+7;
//   * hi = e4m3(v) and lo = e4m3(16 (v - hi)), v = x * 2^-e, each rounded to nearest even, in
//     sign-operand order: piece (s, 8 part + 4 half + g) = bytes 16 half..16 half+15 of lane
//     group g's 32 fp8 values (part 0 = hi, 1 = lo), positions mapped to columns as above.
constexpr int kActThreads = 128;

__device__ __forceinline__ int col_of_position(int h) {  // operand position -> column, one step
  return 32 * (h >> 5) + 4 * (h & 7) + ((h >> 3) & 3);
}

__global__ __launch_bounds__(kActThreads) void split_act_kernel(const SplitActArgs a) {
  __shared__ float red[kActThreads / 64];
  const int t = blockIdx.x, p = blockIdx.y;
  const int d_in = a.d_in[p];
  const uint16_t* __restrict__ x = a.x[p] + (size_t)t * d_in;
  const size_t mp16 = (size_t)a.Mp * 16;
  unsigned char* __restrict__ xb = a.xb[p] + (size_t)t * 16;
  unsigned char* __restrict__ q = a.xq[p] + (size_t)t * 16;
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
      // bf16 piece r = i (columns 8i..8i+7 = chunk i/4, group i%4)
      *reinterpret_cast<u32x4*>(xb + ((size_t)s * 16 + i) * mp16) = c;
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
        *reinterpret_cast<u32x4*>(q + ((size_t)s * 16 + 4 * half + G) * mp16) =
            u32x4{hi[o], hi[o + 1], hi[o + 2], hi[o + 3]};
        *reinterpret_cast<u32x4*>(q + ((size_t)s * 16 + 8 + 4 * half + G) * mp16) =
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
  if (a.M < 1 || a.M > kSplitMaxM || a.ntiles < 0 || a.ntiles > kSplitMaxTiles ||
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
  const int nd = (a.M + 16 * kWaves - 1) / (16 * kWaves);  // 1 or 2
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
