// Multi-variant decode with the sign product on the fp4 x fp6 matrix cores: the fused
// reconstruct-and-multiply of the BitDelta post ("Serving architecture") for a token batch
// grouped by variant, with W_base read from HBM once for the whole batch and each active
// variant's sign bits read once.
//
// For a token t of variant v and output row r,
//     y[t][r] = sum_k x[t][k] * w[r][k]  +  sum_k (alpha_v * x[t][k]) * s_v[r][k],   s = +-1.
// The two sums share one fp32 accumulator per (token, row); W_eff is never formed:
//   * base sum: bf16 x bf16 MFMA (v_mfma_f32_16x16x32_bf16) over DENSE 16-token tiles of the
//     batch (the base weights are the same for every token);
//   * sign sum: v_mfma_scale_f32_16x16x128_f8f6f4 with the signs as fp4 (e2m1) and the
//     variant-scaled activations x' = alpha_v * x (fp32 products) as two fp6 (e2m3) terms,
//     x' ~ 2^a * hi + 2^b * lo, with one pair of power-of-two scales (a, b) per token and
//     32-column block (the E8M0 block scales of the instruction): a puts the block's largest
//     |x'| at the top of the e2m3 range, hi = e2m3(x' 2^-a), and b does the same for the
//     remainders x' - 2^a hi, lo = e2m3((x' - 2^a hi) 2^-b), each rounded to nearest even.
//     The error of an element is below 2^-4 of the block's largest remainder, itself at most
//     2^-4 of the block's largest |x'|: about 2^-8 of the block maximum, the size of a bf16
//     rounding of x'.  The fp4 x fp6 instruction issues at twice the rate of fp4 x fp8, so the
//     two terms cost what one fp8 term would.  One instruction covers a (dense tile, variant)
//     pair: the tile's tokens of other variants get block scale 2^-127, so their products
//     vanish and the pair's products add straight into the dense tile's accumulators.
//
// K order and the sign operand.  Inside one 128-wide K step the instruction's lane group G
// (lanes 16G..16G+15) holds K positions 32G..32G+31 of both operands.  In the fp4 operand
// nibble n of dword d is position 32G + 8d + n, mapped to weight column 32d + 4n + G: bit
// 4n + G of sign word d of the step.  So lane group G keeps only the bits at one place of each
// nibble, and a dword of the operand is one AND of the word with a mask: for G = 0, 1, 2 a set
// bit reads as the fp4 value 0.5 * 2^G and a clear one as 0, i.e. the operand holds
// b = (s + 1) / 2 scaled by 0.5 * 2^G; for G = 3 the bit is the fp4 sign and the operand holds
// s as +-0.5 (one AND and one XOR).  The activation terms of lane group G carry the power of
// two that makes each product 2 b x' (G < 3) or s x' (G = 3), folded into their block scales,
// and since s x' = 2 b x' - x', the kernel subtracts, per token, the sum of x' over the columns
// of groups 0..2, which the prologue leaves per step.  In the fp6 operand field f (bits
// 6f..6f+5 of six dwords) is position 32G + f; the prologue writes column
// 32 (f / 8) + 4 (f % 8) + G there, so both operands agree on every product.  The block scale
// of lane group G covers the 32 columns c = G (mod 4) of the step.
//
// Work split.  A workgroup (8 waves, two per SIMD) owns 128 output rows of one linear and up to
// 256 tokens (16 dense tiles).  The host gives each wave up to ND dense tiles (neighbouring
// ones, which share variants) and their (tile, variant) pairs, as NG slot groups of one variant
// each, balancing the work of the SIMDs.  The K
// loop walks d_in in steps of 128:
//   * W_base (128 rows x 128, 32 KiB) and the sign words of every active variant (the tiled
//     copy: 128 rows x 16 B = 2 KiB contiguous per variant and step) are copied by direct
//     global->LDS loads (16 bytes per lane, whole cache lines) into a ring of 2 to 4 stages, as
//     many as LDS holds, one step per stage; W_base's 16-byte chunks are XOR-swizzled by row so
//     the MFMA operand reads are conflict-free;
//   * each wave's activations (bf16, fp6 terms and block scales of its dense tiles) go straight
//     from memory into registers, reloaded for the next step right after use; lanes that hold
//     no token of the launch read zeros without touching memory;
//   * one workgroup barrier per step; before it each wave waits only for its copies that the
//     next step reads, never for the activation loads in flight.
// The accumulators are stored as y (bf16, nearest-even, or fp32) by the waves that own them.
#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kSplitRows;        // 128 output rows per workgroup
constexpr int kRT = kRows / 16;          // row tiles
constexpr int kKS = 128;                 // k per step
constexpr unsigned kWStage = kRows * kKS * 2;        // 32 KiB of W_base per step
constexpr unsigned kSSlot = kRows * 16;              // one variant's sign words, one step: 2 KiB
constexpr unsigned kLdsCap = 160 * 1024;             // LDS of one compute unit
// waves that issue the global->LDS copies: all 8 with two dense tiles per wave; with one, the
// less loaded wave of each SIMD (often one without a tile)
constexpr int copy_waves(int nd) { return nd == 2 ? 8 : 4; }
// per-row scales of a block, fp32, one run of kRows + 4 floats per variant slot (the padding
// puts the runs of different slots on different LDS banks)
constexpr int kRScaleStride = kRows + 4;
constexpr unsigned kRowScaleBytes = kMaxSlots * kRScaleStride * 4;
static_assert(kWStage + kMaxSlots * kSSlot <= (kLdsCap - kRowScaleBytes) / 2,
              "two stages and the row scales must fit in LDS");

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp4 (e2m1) A operand x fp6 (e2m3) B operand, K = 128; B lane (token j, group g) is scaled by
// 2^(byte SEL of its scale register - 127).
template <int SEL>
__device__ __forceinline__ f32x4 mfma_sign(const u32x4& a, const i32x8& b, int scale_b,
                                           const f32x4& c) {
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b, c, 4, 2, 0, 127, SEL, scale_b);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + 2^31): offsets past the end read as zero, and every
// offset the kernel forms for real data stays inside the tensor it addresses.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// 16 bytes per lane from base + voff straight into LDS at lds_base + 16 * lane.  The buffer
// (MUBUF) form is used rather than the global one so the compiler's wait-count tracking of the
// other loads stays exact; the copies themselves are waited for explicitly before barriers.
// W_base and the sign words are read once per launch: the copies skip the compute unit's cache
// and are marked non-temporal, so they do not push out of the caches the activations that every
// workgroup on the XCD re-reads (measured: 1009 -> 981 us per 70B block at 256 tokens).
constexpr int kStreamOnce = 3;  // cache policy: sc0 (no compute-unit cache) | nt (streaming)
__device__ __forceinline__ void dma16(rsrc_t r, unsigned voff, unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, kStreamOnce);
}

// 16 or 4 bytes from a raw buffer; an offset at or past kOob reads as zero without touching
// memory.
constexpr unsigned kOob = 0x80000000u;
// cache policy of a buffer access that is coherent at device scope (it bypasses the compute
// unit's cache; the same policy as a relaxed device-scope atomic load or store)
constexpr int kDeviceCoherent = 16;
__device__ __forceinline__ u32x4 load16(rsrc_t r, unsigned voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ unsigned load4(rsrc_t r, unsigned voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding, n <= 63).
#define SPLIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier; the empty asm statements keep the compiler from moving memory accesses
// across it.  Visibility of LDS written by direct copies is ensured by the vmcnt wait before.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
constexpr int cmin63() { return N > 63 ? 63 : N; }

// RA: the launch has variants with one scale per output row; their pairs multiply x' = x (the
// prologue leaves it unscaled).  kRowsAcc (one dense tile per wave): the pairs sum into a second
// accumulator set, which each piece scales row by row and adds to the first before its sums
// leave the registers.  kRowsStep (two tiles per wave, where a second set does not fit the
// registers): each step, every pair of a dense tile sums into one temporary set, which is added
// to the accumulators times the scale of each lane's token and row (1 for a variant with one
// scale per matrix, whose activations already carry it); the scales of the block's 128 rows wait
// in LDS past the copy ring (kRowScaleBytes).
constexpr int kRowsNone = 0, kRowsAcc = 1, kRowsStep = 2;
template <int ND, int NG, int RA>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(const SplitArgs a, unsigned stage_bytes,
                                                            int nst) {
  static_assert(RA != kRowsAcc || ND == 1, "a second accumulator set fits one dense tile");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- which piece: linear, 128-row block and K steps (wave-uniform) ---------------------------
  // Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), and each
  // XCD takes its list (the schedule above) in order: its run of the linears' row blocks, so
  // that a linear's activations are fetched into few XCDs' L2, and the workgroups running side by
  // side on one XCD read the same activations at the same time.
  const SplitSched& H = a.sch;
  const int xcd = blockIdx.x & 7;
  int ns_q[kMaxProblems];
#pragma unroll
  for (int q = 0; q < kMaxProblems; ++q) ns_q[q] = q < a.nprob ? a.prob[q].d_in / kKS : 0;
  const SplitPiece pc0 = split_piece(H.x[xcd], a.nprob, ns_q, (int)(blockIdx.x >> 3));
  const int p = pc0.p, rb = pc0.rb, k0 = pc0.k0, k1 = pc0.k1, nparts = pc0.nparts,
            part = pc0.part, sid = pc0.sid, slot0 = pc0.slot0;
  if (p < 0) return;  // past the end of this XCD's list
  const SplitProblem& P = a.prob[p];
  const int d_in = P.d_in, d_out = P.d_out;
  const int row0 = rb * kRows;
  const int nslots = a.nslots;
  const int nsteps = d_in / kKS;
  const int ahead = nst - 1;
  const int lo_tok = a.lo, hi_tok = a.hi;      // valid tokens, relative to a.tok_base

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;

  // ---- direct copies (global -> LDS), `ahead` steps ahead, into stage s % nst ------------------
  // The copying waves (copy share cw, from the host) issue kCopies copies each per step in their
  // sign phase.  With two tiles per wave every wave copies: with 4 waves issuing 16
  // copies each, those waves took a tenth of a step longer than the others, which then waited
  // at the barrier.
  // W_base: copy b = kWCopies*cw + u (of 32) moves rows 4b..4b+3 of the block for one step, 256 bytes
  // each, so every 4 consecutive lanes read 64 contiguous bytes.  Lane L writes LDS slot
  // (row 4b + L/16, 16-byte position L%16) and fetches 16-byte column chunk position ^ (row%16):
  // the XOR swizzle keeps the MFMA operand reads below conflict-free.
  const int cw_raw = a.wv[wave].copier;
  const bool copier = cw_raw >= 0;
  const int cw = copier ? cw_raw : 0;
  constexpr int kCopyWaves = copy_waves(ND);
  constexpr int kWCopies = 32 / kCopyWaves;  // W_base copies per copying wave and step
  constexpr int kCopies = 2 * kWCopies;      // all copies per copying wave and step
  const rsrc_t wrs = make_rsrc(P.w + (size_t)row0 * d_in);
  unsigned woff[kWCopies];
#pragma unroll
  for (int u = 0; u < kWCopies; ++u) {
    const int rl = 4 * (kWCopies * cw + u) + (lane >> 4);
    const int row = min(row0 + rl, d_out - 1) - row0;
    woff[u] = (unsigned)((row * d_in + 8 * ((lane & 15) ^ (rl & 15))) * 2);
  }
  // sign words (tiled layout): the 128 rows of this block for one step are 2 KiB contiguous at
  // word (rb * nsteps + s) * 512; share cw moves both 1 KiB halves of slots cw,
  // cw + kCopyWaves, ...
  const unsigned soff = (unsigned)rb * (unsigned)nsteps * 2048u + (unsigned)lane * 16u;
  // copy k (< kCopies) of this wave for step s into the stage at byte st
  auto copy = [&](int k, int s, unsigned st) {
    if (k < kWCopies) {
      dma16(wrs, woff[k] + (unsigned)s * (kKS * 2), smem + st + (kWCopies * cw + k) * 1024);
    } else {
      const int j = k - kWCopies;
      const int q = 2 * (cw + kCopyWaves * (j >> 1)) + (j & 1);
      if (q < 2 * nslots)
        dma16(make_rsrc(P.words[q >> 1]), soff + (unsigned)(j & 1) * 1024u + (unsigned)s * 2048u,
              smem + st + kWStage + q * 1024);
    }
  };

  // ---- activations: the prologue's layouts ------------------------------------------------------
  // With nblk = Mp / 16 token blocks, the 64 lanes of a 16-token aligned block read, per step s,
  //   bf16 pieces (s, c), c < 4: 16 bytes per lane at ((s * 4 + c) * nblk + block) * 1024;
  //   fp6 pieces (s, o), o < 3:  16 bytes per lane at ((s * 3 + o) * nblk + block) * 1024
  //     (hi = dwords 0..5 of pieces 0,1, lo = dwords 2..7 of pieces 1,2);
  //   scales: 4 bytes per lane at (s * nblk + block) * 256 (byte 0 hi, byte 1 lo),
  // lane L at offset 16 L (4 L for scales).
  const rsrc_t xrs = make_rsrc(P.x);
  const rsrc_t qrs = make_rsrc(P.xq);
  const rsrc_t crs = make_rsrc(P.xs);
  const unsigned ostep = (unsigned)a.Mp * 64;   // bytes between consecutive pieces (= nblk KiB)
  const unsigned cstep = (unsigned)a.Mp * 16;   // bytes between consecutive scale steps
  const int tb0 = a.tok_base >> 4;              // first 16-token block of this launch
  unsigned xoff[ND], qoff[ND], coff[ND];
  bool dreal[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int tile = a.wv[wave].tile[i];
    const int t = 16 * tile + j;                // relative to tok_base
    dreal[i] = tile >= 0;
    const bool tv = tile >= 0 && t >= lo_tok && t < hi_tok;
    const bool tq = tv && a.token_slot[t] >= 0;  // the prologue wrote this token's fp6 terms
    xoff[i] = tv ? (unsigned)(tb0 + tile) * 1024 + (unsigned)lane * 16 : kOob;
    qoff[i] = tq ? (unsigned)(tb0 + tile) * 1024 + (unsigned)lane * 16 : kOob;
    coff[i] = tq ? (unsigned)(tb0 + tile) * 256 + (unsigned)lane * 4 : kOob;
  }
  // slot groups: group q holds the pair (dense tile i, variant slot gslot[q][i]) of each tile i
  // that has one (slot -1: none); pin marks the lanes whose token belongs to that variant; grow
  // marks the pairs whose variant has per-row scales (wave-uniform)
  int gslot[NG][ND];
  bool pin[NG][ND];
  bool grow[NG][ND];
#pragma unroll
  for (int q = 0; q < NG; ++q)
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int slot = a.wv[wave].slot[q][i];
      gslot[q][i] = slot;
      const int t = 16 * a.wv[wave].tile[i] + j;
      pin[q][i] = slot >= 0 && dreal[i] && t >= lo_tok && t < hi_tok && a.token_slot[t] == slot;
      grow[q][i] = RA != kRowsNone && slot >= 0 && ((P.alpha_rows >> slot) & 1u);
    }

  // ---- registers ------------------------------------------------------------------------------------
  u32x4 xb[ND][4];           // bf16 activations of the dense tiles, 4 chunks of 32 columns
  u32x4 xq[ND][3];           // fp6 hi / lo terms of the dense tiles
  unsigned xs[ND];           // their block scales
  f32x4 acc[ND][kRT];
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) acc[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 accs[RA == kRowsAcc ? kRT : 1];  // kRowsAcc: sign sums of the per-row pairs (tile 0)
#pragma unroll
  for (int rt = 0; rt < (RA == kRowsAcc ? kRT : 1); ++rt) accs[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kRowsStep: slot sl's scales of rows row0 .. row0 + 127 at float kRScaleStride * sl (rows
  // past d_out repeat the last row's; 1 for a slot with one scale per matrix), and each lane's
  // offset there for its token in dense tile i (slot 0 for lanes without a token)
  float* const rscale = reinterpret_cast<float*>(smem + (unsigned)nst * stage_bytes);
  unsigned rsl[ND];
  if (RA == kRowsStep) {
    for (int e = tid; e < nslots * kRows; e += kThreads) {
      const int sl = e / kRows, r = e - sl * kRows;
      rscale[sl * kRScaleStride + r] =
          ((P.alpha_rows >> sl) & 1u) ? P.alpha[sl][min(row0 + r, d_out - 1)] : 1.f;
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int t = 16 * a.wv[wave].tile[i] + j;
      const int ts = dreal[i] && t >= lo_tok && t < hi_tok ? a.token_slot[t] : -1;
      rsl[i] = (unsigned)(ts >= 0 ? ts : 0) * kRScaleStride + 4 * g;
    }
  }

  auto load_xb = [&](int i, unsigned s) {
#pragma unroll
    for (int c = 0; c < 4; ++c) xb[i][c] = load16(xrs, xoff[i] + (s * 4 + c) * ostep);
  };
  auto load_xq = [&](int i, unsigned s) {
#pragma unroll
    for (int o = 0; o < 3; ++o) xq[i][o] = load16(qrs, qoff[i] + (s * 3 + o) * ostep);
    xs[i] = load4(crs, coff[i] + s * cstep);
  };
  // vector-memory instructions per step that are activation loads
  constexpr int kX = 8 * ND;

  // ---- prologue: steps k0..k0+ahead-1 into stages 0..ahead-1, the activations of step k0 ------
  if (copier)
    for (int r = 0; r < ahead && k0 + r < k1; ++r)
#pragma unroll
      for (int k = 0; k < kCopies; ++k) copy(k, k0 + r, (unsigned)r * stage_bytes);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < ND; ++i) load_xq(i, (unsigned)k0);
#pragma unroll
  for (int i = 0; i < ND; ++i) load_xb(i, (unsigned)k0);
  __builtin_amdgcn_sched_barrier(0);
  SPLIT_VMCNT(cmin63<kX>());
  if (RA == kRowsStep) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): scale stores in LDS
  raw_barrier();

  // per-lane LDS read offsets
  const unsigned a_lane = (unsigned)j * 256;                      // + stage + rt*4096 + chunk
  const unsigned s_lane = kWStage + (unsigned)j * 16;            // + stage + slot + rt*256
  // sign operand of lane group g: the bit of column 32 d + 4 n + g as nibble n of dword d; groups
  // 0..2 keep it as 0.5 * 2^g when set (0 when clear), group 3 as +-0.5
  const unsigned sm1 = g < 3 ? 0x11111111u << g : 0x88888888u;
  const unsigned sm2 = g < 3 ? 0u : 0x99999999u;

  unsigned st = 0;                                     // stage of step s
  unsigned st_next = (unsigned)ahead * stage_bytes;    // stage of step s + ahead
  const unsigned ring = (unsigned)nst * stage_bytes;
  // sign sum over this wave's slot groups, into the dense tiles.  The fp4 operands of a group's
  // variant are expanded once for both of its tiles; each pair issues its 8 hi-term MFMAs before
  // its 8 lo-term MFMAs, so dependent MFMAs are 8 apart.  With copies, the wave issues all its
  // copies of step cs first (rather than spread over the groups: 1% faster per 70B block at 256
  // tokens, 2.5% at 64, the copies having longer to arrive).
  u32x4 S[kRT];
  // Lanes whose token is not of the pair's variant get block scale 2^-127 for both terms, so
  // their products vanish below fp32 resolution (at most 2^-120 in magnitude per product).
  // A per-row pair (rows, variant slot sl) sums 4 row tiles at a time from zero and adds the sums
  // times the rows' scales (lane: rows 4g .. 4g + 3 of each row tile).
  auto pair_mfma = [&](int i, bool in, bool rows) {
    const int sc = in ? (int)xs[i] : 0;
    const i32x8 bh = {(int)xq[i][0][0], (int)xq[i][0][1], (int)xq[i][0][2], (int)xq[i][0][3],
                      (int)xq[i][1][0], (int)xq[i][1][1], 0, 0};
    const i32x8 bl = {(int)xq[i][1][2], (int)xq[i][1][3], (int)xq[i][2][0], (int)xq[i][2][1],
                      (int)xq[i][2][2], (int)xq[i][2][3], 0, 0};
    if (RA == kRowsAcc && rows) {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) accs[rt] = mfma_sign<0>(S[rt], bh, sc, accs[rt]);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) accs[rt] = mfma_sign<1>(S[rt], bl, sc, accs[rt]);
    } else {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) acc[i][rt] = mfma_sign<0>(S[rt], bh, sc, acc[i][rt]);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) acc[i][rt] = mfma_sign<1>(S[rt], bl, sc, acc[i][rt]);
    }
  };
  auto expand = [&](int slot, unsigned st) {
    const unsigned char* sw = smem + st + s_lane + (unsigned)slot * kSSlot;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(sw + rt * 256);
      S[rt] = u32x4{(w[0] & sm1) ^ sm2, (w[1] & sm1) ^ sm2, (w[2] & sm1) ^ sm2, (w[3] & sm1) ^ sm2};
    }
  };
  // kRowsStep: the sign sums of pair (dense tile i, the expanded variant) into t
  auto pair_into = [&](f32x4(&t)[kRT], int i, bool in) {
    const int sc = in ? (int)xs[i] : 0;
    const i32x8 bh = {(int)xq[i][0][0], (int)xq[i][0][1], (int)xq[i][0][2], (int)xq[i][0][3],
                      (int)xq[i][1][0], (int)xq[i][1][1], 0, 0};
    const i32x8 bl = {(int)xq[i][1][2], (int)xq[i][1][3], (int)xq[i][2][0], (int)xq[i][2][1],
                      (int)xq[i][2][2], (int)xq[i][2][3], 0, 0};
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) t[rt] = mfma_sign<0>(S[rt], bh, sc, t[rt]);
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) t[rt] = mfma_sign<1>(S[rt], bl, sc, t[rt]);
  };
  auto sign_phase = [&](bool copies, int cs, unsigned cst, unsigned st) {
    if (RA == kRowsStep) {
      // tile by tile: tile 0 takes its groups last to first and tile 1 first to last, so a
      // variant of both tiles (the first groups) is expanded once when it is the only one
      int cur = -1;
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        f32x4 t[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) t[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < NG; ++qq) {
          // copies spread over the groups here (issued all first, this form measured 1% slower)
          if (copies) {
            const int it = i * NG + qq;
#pragma unroll
            for (int k = it * kCopies / (ND * NG); k < (it + 1) * kCopies / (ND * NG); ++k)
              copy(k, cs, cst);
          }
          const int q = i == 0 ? NG - 1 - qq : qq;
          const int sl = gslot[q][i];
          if (sl >= 0) {
            if (sl != cur) {
              expand(sl, st);
              cur = sl;
            }
            pair_into(t, i, pin[q][i]);
          }
        }
        if (dreal[i]) {
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            acc[i][rt] += *reinterpret_cast<const f32x4*>(rscale + rsl[i] + 16 * rt) * t[rt];
        }
      }
      return;
    }
    if (copies) {
#pragma unroll
      for (int k = 0; k < kCopies; ++k) copy(k, cs, cst);
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int s0 = gslot[q][0];
      if (s0 >= 0) {
        expand(s0, st);
        pair_mfma(0, pin[q][0], grow[q][0]);
      }
      if (ND == 2) {
        const int s1 = gslot[q][ND - 1];
        if (s1 >= 0) {
          if (s1 != s0) expand(s1, st);
          pair_mfma(ND - 1, pin[q][ND - 1], grow[q][ND - 1]);
        }
      }
    }
  };
  // base sum over the dense tiles, 32-column chunk by chunk, reloading each bf16 chunk for
  // step kn right after its use
  auto base_phase = [&](unsigned kn, unsigned st) {
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
          for (int rt = 0; rt < kRT; ++rt) acc[i][rt] = mfma_bf16(A[rt], xb[i][c], acc[i][rt]);
        }
        xb[i][c] = load16(xrs, xoff[i] + (kn * 4 + c) * ostep);
      }
    }
  };

  for (int s = k0; s < k1; ++s) {
    // Each activation operand is reloaded for step s+1 right after its last use in step s, so
    // every load has most of a step to arrive.
    const unsigned knext = (unsigned)min(s + 1, k1 - 1);
    sign_phase(copier && s + ahead < k1, s + ahead, st_next, st);
#pragma unroll
    for (int i = 0; i < ND; ++i) load_xq(i, knext);
    base_phase(knext, st);

    // Before the barrier, each wave waits for its copies of step s+1 but not for newer loads:
    // after those copies it issued `ahead` steps of activation loads (kX each) and ahead - 1
    // steps of copies, and the activation loads of the older steps have completed (their values
    // were used).  Waves without copies wait for nothing that is still needed.
    __builtin_amdgcn_sched_barrier(0);
    if (ahead == 1) SPLIT_VMCNT(cmin63<kX>());
    else if (ahead == 2) SPLIT_VMCNT(cmin63<2 * kX>());
    else SPLIT_VMCNT(cmin63<3 * kX>());
    raw_barrier();
    st += stage_bytes;
    if (st == ring) st = 0;
    st_next += stage_bytes;
    if (st_next == ring) st_next = 0;
  }

  // ---- correction of the unsigned sign columns ----------------------------------------------------
  // Lane groups 0..2 added 2 b x' for the columns c % 4 < 3 where s x' = 2 b x' - x': subtract the
  // token's sum of x' over those columns and this piece's steps (lanes 16 g + j of token j add
  // every fourth step, then combine).
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    if (!dreal[i]) continue;
    const int tr = 16 * a.wv[wave].tile[i] + j;
    float cs = 0.f;
    if (tr >= lo_tok && tr < hi_tok) {
      const float* xc = P.xc + (size_t)(a.tok_base + tr);
      for (int s = k0 + g; s < k1; s += 4) cs += xc[(size_t)s * a.Mp];
    }
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    if (RA == kRowsAcc) {
      // a token of a per-row variant: its sign sum is in accs, to be scaled row by row
      const int ts = tr >= lo_tok && tr < hi_tok ? a.token_slot[tr] : -1;
      const bool lrow = ts >= 0 && ((P.alpha_rows >> ts) & 1u);
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        if (lrow) accs[rt] -= cs;
        else acc[i][rt] -= cs;
      }
      if (lrow) {
        // acc += alpha_r * (sign sum) for the 4 rows 4g..4g+3 of each row tile the lane holds
        const float* al = P.alpha[ts];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const int orow = row0 + rt * 16 + 4 * g;
          f32x4 av;
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = al[min(orow + e, d_out - 1)];
          acc[i][rt] += av * accs[rt];
        }
      }
    } else if (RA == kRowsStep) {
      // a token of a per-row variant: its sign sums were added times alpha_r, and so is the
      // correction (the lane's rows 4g..4g+3 of each row tile)
      const int ts = tr >= lo_tok && tr < hi_tok ? a.token_slot[tr] : -1;
      const bool lrow = ts >= 0 && ((P.alpha_rows >> ts) & 1u);
      const float* rs = rscale + (lrow ? ts : 0) * kRScaleStride + 4 * g;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        if (lrow) acc[i][rt] -= *reinterpret_cast<const f32x4*>(rs + 16 * rt) * cs;
        else acc[i][rt] -= cs;
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) acc[i][rt] -= cs;
    }
  }

  // ---- split unit: leave the sums in this piece's slot; the last piece adds all slots ------------
  // A slot holds, per dense tile i of the launch and row tile rt, the 64 lanes' f32x4 in lane
  // order, so each wave reads back exactly what the same wave of another piece wrote.  The slots
  // are written and read with device-coherent accesses (which skip the compute unit's own
  // cache); each wave waits until its stores are done, then one thread releases them at device
  // scope (the XCD's L2 writes back what it holds) and counts the piece in, adding 1 to the
  // count and 1 to the field of the XCD it runs on.  The workgroup that brings the count to
  // nparts adds the slots in piece order (its own sums from registers, so the order, and the
  // result, do not depend on which piece finished last).  The schedule puts every piece of a
  // unit on one XCD (workgroups b and b + 8k are dispatched to the same XCD), so the slots meet
  // in that XCD's L2; if the fields show pieces on another XCD, the last piece first acquires at
  // device scope (invalidating stale lines of its L2) and counts the event in the stats word.
  if (nparts > 1) {
    const rsrc_t prs = make_rsrc(reinterpret_cast<unsigned char*>(H.partial) +
                                 (size_t)slot0 * H.slot_bytes);
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      if (!dreal[i]) continue;
      const unsigned o = (unsigned)part * H.slot_bytes +
                         (unsigned)a.wv[wave].tile[i] * (kRT * 1024) + (unsigned)lane * 16;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][rt]), prs,
                                               o + rt * 1024, 0, kDeviceCoherent);
    }
    SPLIT_VMCNT(0);
    __syncthreads();
    int* flag = reinterpret_cast<int*>(smem);
    if (tid == 0) {
      unsigned hw;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw));
      const unsigned x = hw & 7u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const unsigned long long old = __hip_atomic_fetch_add(
          H.counter + sid, 1ull + (1ull << (8 + 6 * x)), __ATOMIC_RELAXED,
          __HIP_MEMORY_SCOPE_AGENT);
      const bool last = (int)(old & 0xFFu) == nparts - 1;
      const bool elsewhere = ((old >> 8) & ~(0x3Full << (6 * x))) != 0ull;
      if (last && elsewhere) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_fetch_add(H.stats, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      flag[0] = last ? 1 : 0;
    }
    __syncthreads();
    if (flag[0] == 0) return;  // workgroup-uniform: another piece finishes this unit
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      if (!dreal[i]) continue;
      const unsigned o = (unsigned)a.wv[wave].tile[i] * (kRT * 1024) + (unsigned)lane * 16;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int pc = 0; pc < nparts; ++pc)
          v += pc == part ? acc[i][rt]
                          : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                prs, (unsigned)pc * H.slot_bytes + o + rt * 1024, 0,
                                kDeviceCoherent));
        acc[i][rt] = v;
      }
    }
  }

  // ---- epilogue: y = accumulators ---------------------------------------------------------------
  const bool vec_store = (d_out & 3) == 0;  // y rows start on 4-element boundaries
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int tr = 16 * a.wv[wave].tile[i] + j;  // relative token
    if (!dreal[i] || tr < lo_tok || tr >= hi_tok) continue;
    const size_t ybase = (size_t)(a.tok_base + tr) * d_out;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      const int orow = row0 + rt * 16 + 4 * g;
      const f32x4 v = acc[i][rt];
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
// A workgroup covers one 16-token block and 4 K steps of one linear, one wave per step; lane
// L = 16 g + j writes token j's 16-byte slot of every 1 KiB piece of that step (layouts above), so
// each piece is written whole by one wave.  Every token gets its bf16 pieces; a token of variant
// v also gets the two fp6 terms of x' = alpha_v * x for the 32 columns c = g (mod 4) of the step,
// with their block scales, and (lane group 0) the step's correction sum; a base-model token's
// correction sum is 0.  Lanes of tokens outside the launch write nothing.
constexpr int kActThreads = 256;
constexpr int kActSteps = kActThreads / 64;

// Exponent a with m <= 7.5 * 2^a < 2 m (m > 0, finite): the block scale that puts m in the top
// binade of e2m3.  m = 1.f * 2^E, and 7.5 = 1.875 * 2^2: a = E - 2 for 1.f <= 1.875, else E - 1.
__device__ __forceinline__ int e2m3_block_exp(float m) {
  const unsigned b = __float_as_uint(m);
  if ((b >> 23) == 0u) {  // subnormal m
    int E;
    const float f = frexpf(m, &E);  // m = f 2^E, f in [0.5, 1)
    return f <= 0.9375f ? E - 3 : E - 2;
  }
  const int E = (int)(b >> 23) - 127;
  return (b & 0x7FFFFFu) <= 0x700000u ? E - 2 : E - 1;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef int i32x6 __attribute__((ext_vector_type(6)));

// 32 values / scale as e2m3 codes, rounded to nearest even (saturating at 7.5): field 2i of the
// six dwords takes even[i], field 2i + 1 takes odd[i].  Written out rather than through the
// compiler's builtin: with the builtin the compiler gave the destination registers that overlap
// the last source registers, and the instruction then converted overwritten inputs (wrong codes
// in the last odd fields, seen on the GPU); an early-clobber output keeps them apart.
__device__ __forceinline__ i32x6 cvt_e2m3x32(const f32x16& even, const f32x16& odd, float scale) {
  i32x6 r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(even), "v"(odd), "v"(scale));
  return r;
}
// the 32 values of six dwords of e2m3 codes (field f -> element f), times scale
__device__ __forceinline__ f32x32 e2m3x32_values(const i32x6& codes, float scale) {
  f32x32 r;
  asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(r) : "v"(codes), "v"(scale));
  return r;
}

__device__ __forceinline__ float pow2f(int e) {  // 2^e for -126 <= e <= 127
  return __uint_as_float((unsigned)(e + 127) << 23);
}

__global__ __launch_bounds__(kActThreads) void split_act_kernel(const SplitActArgs a, int nsq) {
  if (blockIdx.x == 0 && blockIdx.y == 0)  // the split counters of the launch that follows
    for (int c = threadIdx.x; c < a.ncounter; c += kActThreads) a.counter[c] = 0;
  const int p = blockIdx.y;
  const int d_in = a.d_in[p], nsteps = d_in / 128;
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int s = (int)(blockIdx.x % nsq) * kActSteps + (int)(threadIdx.x >> 6);
  if (s >= nsteps) return;                   // wave-uniform
  const int tb = (a.tok_base + a.lo) / 16 + (int)(blockIdx.x / nsq);  // absolute 16-token block
  const int t = 16 * tb + j, tr = t - a.tok_base;
  if (tr < a.lo || tr >= a.hi) return;       // not a token of this launch (all 4 lanes of t)
  const int slot = a.token_slot[tr];
  const size_t nblk = (size_t)a.Mp / 16;
  const size_t ostep = nblk * 1024;          // bytes between consecutive pieces
  const size_t pbase = (size_t)tb * 1024 + (size_t)lane * 16;
  const uint16_t* __restrict__ x = a.x[p] + (size_t)t * d_in + (size_t)s * 128;

  // bf16 pieces (s, c): columns 32c + 8g .. +7 of the step; the four lanes of a token load its
  // whole 256-byte row of the step, which also goes to LDS (rows padded to 264 bytes, so the
  // column reads below hit 16 different banks) for the fp6 terms' strided columns
  __shared__ __attribute__((aligned(16))) uint16_t rows[kActSteps][16][132];
  uint16_t* row = rows[threadIdx.x >> 6][j];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + 32 * c + 8 * g);
    *reinterpret_cast<u32x4*>(a.xb[p] + ((size_t)s * 4 + c) * ostep + pbase) = v;
    *reinterpret_cast<u32x2*>(row + 32 * c + 8 * g) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(row + 32 * c + 8 * g + 4) = u32x2{v[2], v[3]};
  }
  float* corr = a.xc[p] + (size_t)s * a.Mp + t;
  if (slot < 0) {  // base-model token: no sign term, no correction
    if (g == 0) *corr = 0.f;
    return;
  }
  // the row of token j was written by lanes j, j+16, j+32, j+48 of this wave, all still here
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();

  // fp6 terms of lane group g: the 32 columns c = g (mod 4) of the step, field f <- column
  // 32 (f / 8) + 4 (f % 8) + g
  const float alpha = a.alpha[p][slot] ? *a.alpha[p][slot] : 1.0f;  // null: x' = x
  float xp[32];
  float m = 0.f;
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    const unsigned b = row[32 * (f >> 3) + 4 * (f & 7) + g];
    xp[f] = alpha * __uint_as_float(b << 16);
    m = fmaxf(m, fabsf(xp[f]));
  }
  int ea = m > 0.f ? e2m3_block_exp(m) : 0;
  ea = max(-126, min(125, ea));
  const float sa = pow2f(ea);
  f32x16 ev, od;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = xp[2 * i];
    od[i] = xp[2 * i + 1];
  }
  const i32x6 hi = cvt_e2m3x32(ev, od, sa);
  const f32x32 hv = e2m3x32_values(hi, sa);   // values of the hi term
  float rm = 0.f;
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    xp[f] -= hv[f];                          // remainder
    rm = fmaxf(rm, fabsf(xp[f]));
  }
  int eb = rm > 0.f ? e2m3_block_exp(rm) : ea;
  eb = max(-126, min(125, eb));
  const float sb = pow2f(eb);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = xp[2 * i];
    od[i] = xp[2 * i + 1];
  }
  const i32x6 lo = cvt_e2m3x32(ev, od, sb);
  const f32x32 lv = e2m3x32_values(lo, sb);
  float cs = 0.f;                            // sum of this lane's quantized x', in field order
#pragma unroll
  for (int f = 0; f < 32; ++f) cs += hv[f] + lv[f];
  unsigned char* q = a.xq[p] + pbase;
  const u32x4 q0 = {(unsigned)hi[0], (unsigned)hi[1], (unsigned)hi[2], (unsigned)hi[3]};
  const u32x4 q1 = {(unsigned)hi[4], (unsigned)hi[5], (unsigned)lo[0], (unsigned)lo[1]};
  const u32x4 q2 = {(unsigned)lo[2], (unsigned)lo[3], (unsigned)lo[4], (unsigned)lo[5]};
  *reinterpret_cast<u32x4*>(q + ((size_t)s * 3 + 0) * ostep) = q0;
  *reinterpret_cast<u32x4*>(q + ((size_t)s * 3 + 1) * ostep) = q1;
  *reinterpret_cast<u32x4*>(q + ((size_t)s * 3 + 2) * ostep) = q2;
  // Block scales with the lane group's operand factor: the sign operand of lane groups 0..2
  // holds the bit b = (s + 1) / 2 as 0.5 * 2^g, so their terms carry 2^(2-g) (the products are
  // 2 b x'); lane group 3 holds s as +-0.5, so its terms carry 2 (the products are s x').
  const int fe = g < 3 ? 2 - g : 1;
  *reinterpret_cast<unsigned*>(a.xs[p] + ((size_t)s * nblk + tb) * 256 + (size_t)lane * 4) =
      (unsigned)(ea + fe + 127) | ((unsigned)(eb + fe + 127) << 8);
  // correction: s x' = 2 b x' - x' on lane groups 0..2, so the token's products over this step
  // need sum(x') of those columns subtracted; lanes 16g + j with g = 0..3 hold token j
  if (g == 3) cs = 0.f;
  cs += __shfl_xor(cs, 16);
  cs += __shfl_xor(cs, 32);
  if (g == 0) *corr = cs;
}

// Dynamic LDS one workgroup may use on the current device, capped at one compute unit's.
int lds_limit() {
  static std::atomic<int> cached[64];  // per device, 0 = not queried yet
  const int v = device_attribute_cached(cached, hipDeviceAttributeMaxSharedMemoryPerBlock, 0);
  return v < (int)kLdsCap ? v : (int)kLdsCap;
}

template <int ND, int NG, int RA = kRowsNone>
hipError_t launch_nd_ng(const SplitArgs& a, int nblocks, unsigned stage, int nst,
                         hipStream_t stream) {
  static DeviceOnce once;
  hipError_t e = set_dynamic_lds_once(
      once, reinterpret_cast<const void*>(&split_kernel<ND, NG, RA>), lds_limit());
  if (e != hipSuccess) return e;
  clear_stale_error();
  hipLaunchKernelGGL((split_kernel<ND, NG, RA>), dim3(nblocks), dim3(kThreads),
                     nst * stage + (RA == kRowsStep ? kRowScaleBytes : 0u), stream, a, stage, nst);
  return hipGetLastError();
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

void split_workspace_parts(int64_t M, int64_t d_in, size_t* xb_bytes, size_t* xq_bytes,
                           size_t* xs_bytes, size_t* xc_bytes) {
  const size_t mp = (size_t)((M + 15) / 16) * 16;
  *xb_bytes = round256(mp * 2 * (size_t)d_in);       // bf16
  *xq_bytes = round256(mp * 3 * (size_t)d_in / 2);   // two fp6 terms: 12 bits per element
  *xs_bytes = round256(mp * (size_t)d_in / 8);       // 4 bytes per token and 32 columns
  *xc_bytes = round256(mp * (size_t)d_in / 32);      // 4 bytes per token and 128 columns
}

size_t split_slot_bytes(int64_t M) {
  return (size_t)((M + 15) / 16) * 16 * kSplitRows * 4;
}

size_t split_partial_bytes(int64_t M) {
  return round256((size_t)kSplitSlotsPerLinear * split_slot_bytes(M)) +
         round256(kSplitCounterBytes) + kSplitStatsBytes;
}

size_t split_workspace_bytes(int64_t M, int64_t d_in) {
  size_t b, q, c, k;
  split_workspace_parts(M, d_in, &b, &q, &c, &k);
  return b + q + c + k + split_partial_bytes(M);
}

hipError_t launch_split_act(const SplitActArgs& a, hipStream_t stream) {
  if (a.nprob <= 0 || a.nprob > kMaxProblems || a.lo < 0 || a.hi <= a.lo || a.hi > kSplitMaxM ||
      (a.tok_base & 15) != 0 || a.ncounter < 0 || (a.ncounter > 0 && !a.counter))
    return hipErrorInvalidValue;
  int max_steps = 0;
  for (int q = 0; q < a.nprob; ++q) max_steps = max(max_steps, a.d_in[q] / 128);
  const int nsq = (max_steps + kActSteps - 1) / kActSteps;
  const int ntb = (a.hi - 1) / 16 - a.lo / 16 + 1;
  if (nsq < 1) return hipErrorInvalidValue;
  clear_stale_error();
  hipLaunchKernelGGL(split_act_kernel, dim3(ntb * nsq, a.nprob), dim3(kActThreads), 0, stream, a,
                     nsq);
  return hipGetLastError();
}

hipError_t launch_split(const SplitArgs& a, int nd, int ng, hipStream_t stream) {
  if (a.hi < 1 || a.hi > kSplitMaxM || a.lo < 0 || a.lo >= a.hi || (a.tok_base & 15) != 0 ||
      a.nslots < 0 || a.nslots > kMaxSlots || a.nprob < 1 || a.nprob > kMaxProblems ||
      nd < 1 || nd > 2 || ng < 0 || ng > kSplitMaxGroups)
    return hipErrorInvalidValue;
  unsigned copy_shares = 0;
  for (int w = 0; w < kWaves; ++w) {
    const SplitWave& W = a.wv[w];
    if (W.copier < -1 || W.copier >= copy_waves(nd)) return hipErrorInvalidValue;
    if (W.copier >= 0) {
      if (copy_shares >> W.copier & 1u) return hipErrorInvalidValue;
      copy_shares |= 1u << W.copier;
    }
    for (int i = 0; i < 2; ++i)
      if (W.tile[i] >= kSplitMaxM / 16 || (i >= nd && W.tile[i] >= 0)) return hipErrorInvalidValue;
    for (int q = 0; q < kSplitMaxGroups; ++q)
      for (int i = 0; i < 2; ++i) {
        const int slot = W.slot[q][i];
        if (slot < -1 || slot >= a.nslots) return hipErrorInvalidValue;
        if (slot >= 0 && (q >= ng || i >= nd || W.tile[i] < 0)) return hipErrorInvalidValue;
      }
  }
  if (copy_shares != (1u << copy_waves(nd)) - 1u) return hipErrorInvalidValue;  // every copy issued
  // variants with one scale per output row: with two tiles per wave their scales take
  // kRowScaleBytes of LDS past the ring
  bool rows = false;
  for (int q = 0; q < a.nprob; ++q) {
    const SplitProblem& P = a.prob[q];
    for (int sl = 0; sl < a.nslots; ++sl)
      if (((P.alpha_rows >> sl) & 1u) && !P.alpha[sl]) return hipErrorInvalidValue;
    rows = rows || (P.alpha_rows & ((1u << a.nslots) - 1u)) != 0u;
  }
  const int lds = lds_limit() - (rows && nd == 2 ? (int)kRowScaleBytes : 0);
  const unsigned stage = kWStage + (unsigned)a.nslots * kSSlot;
  int nst = lds / (int)stage;
  nst = nst > 4 ? 4 : nst;
  if (nst < 2) return hipErrorInvalidConfiguration;
  // the schedule must describe the lists the kernel walks (see the piece map in the kernel): each
  // linear's row blocks tiled by the XCDs' runs in XCD order, every list's counts as its
  // parameters give them, counters and partial slots numbered XCD after XCD within what the
  // workspace holds (kSplitSlotsPerLinear of each per linear)
  const SplitSched& H = a.sch;
  int ns[kMaxProblems], pos[kMaxProblems];
  for (int q = 0; q < kMaxProblems; ++q) ns[q] = pos[q] = 0;
  for (int q = 0; q < a.nprob; ++q) {
    const SplitProblem& P = a.prob[q];
    if (P.nblocks < 1 || P.d_in < kKS || P.d_in % kKS != 0) return hipErrorInvalidValue;
    ns[q] = P.d_in / kKS;
  }
  int max_list = 0, split_end = 0, slot_end = 0;
  for (int x = 0; x < 8; ++x) {
    const SplitXcd& X = H.x[x];
    if (X.sigma < 1 || X.cut < 1 || X.pooled < 0) return hipErrorInvalidValue;
    for (int q = 0; q < kMaxProblems; ++q) {
      if (X.cnt[q] < 0 || (q >= a.nprob && X.cnt[q] != 0)) return hipErrorInvalidValue;
      if (X.cnt[q] > 0) {
        if (X.first[q] != pos[q]) return hipErrorInvalidValue;
        pos[q] += X.cnt[q];
      }
    }
    int nh, npl, nsp, nsl;
    const int max_parts = split_xcd_counts(X, a.nprob, ns, &nh, &npl, &nsp, &nsl);
    // a unit's counter has 6 bits per XCD field and 8 for the count
    if (max_parts > 63) return hipErrorInvalidValue;
    if (nh != X.nheads || npl != X.npool || nsp != X.nsplit || nsl != X.nslot)
      return hipErrorInvalidValue;
    if (X.split0 != split_end || X.slot0 != slot_end) return hipErrorInvalidValue;
    split_end += nsp;
    slot_end += nsl;
    max_list = max(max_list, nh + npl);
  }
  for (int q = 0; q < a.nprob; ++q)
    if (pos[q] != a.prob[q].nblocks) return hipErrorInvalidValue;
  if (split_end > a.nprob * kSplitSlotsPerLinear || slot_end > a.nprob * kSplitSlotsPerLinear)
    return hipErrorInvalidValue;
  if (slot_end > 0 && (!H.partial || !H.counter || !H.stats || H.slot_bytes < (unsigned)a.Mp * kRows * 4))
    return hipErrorInvalidValue;
  const int nblocks = 8 * max_list;
  if (rows) {
    if (nd == 1) {
      if (ng <= 1) return launch_nd_ng<1, 1, kRowsAcc>(a, nblocks, stage, nst, stream);
      if (ng <= 2) return launch_nd_ng<1, 2, kRowsAcc>(a, nblocks, stage, nst, stream);
      if (ng <= 4) return launch_nd_ng<1, 4, kRowsAcc>(a, nblocks, stage, nst, stream);
      return launch_nd_ng<1, 8, kRowsAcc>(a, nblocks, stage, nst, stream);
    }
    if (ng <= 1) return launch_nd_ng<2, 1, kRowsStep>(a, nblocks, stage, nst, stream);
    if (ng <= 2) return launch_nd_ng<2, 2, kRowsStep>(a, nblocks, stage, nst, stream);
    if (ng <= 4) return launch_nd_ng<2, 4, kRowsStep>(a, nblocks, stage, nst, stream);
    return launch_nd_ng<2, 8, kRowsStep>(a, nblocks, stage, nst, stream);
  }
  if (nd == 1) {
    if (ng <= 1) return launch_nd_ng<1, 1>(a, nblocks, stage, nst, stream);
    if (ng <= 2) return launch_nd_ng<1, 2>(a, nblocks, stage, nst, stream);
    if (ng <= 4) return launch_nd_ng<1, 4>(a, nblocks, stage, nst, stream);
    return launch_nd_ng<1, 8>(a, nblocks, stage, nst, stream);
  }
  if (ng <= 1) return launch_nd_ng<2, 1>(a, nblocks, stage, nst, stream);
  if (ng <= 2) return launch_nd_ng<2, 2>(a, nblocks, stage, nst, stream);
  if (ng <= 4) return launch_nd_ng<2, 4>(a, nblocks, stage, nst, stream);
  return launch_nd_ng<2, 8>(a, nblocks, stage, nst, stream);
}

}  // namespace bd
