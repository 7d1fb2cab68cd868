// Prefill-sized batches: the fused reconstruct-and-multiply of the BitDelta post ("Serving
// architecture": reconstruction in fast on-chip memory, fused with the matmul, W_eff never
// written to HBM) as a dense bf16 MFMA contraction per segment.
//
// A workgroup (8 waves, two per SIMD) computes a tile of 256 tokens (one segment, hence one
// variant) by 256 output rows, walking d_in in steps of 32 taken in pairs.  Wave w owns rows
// 32w .. 32w + 31 for all 256 tokens.  Per pair of steps:
//   * the 256x64 block of activations, which every wave needs, and wave w's own 32x64 block of
//     W_base go straight from memory into LDS (direct global->LDS loads of whole 128-byte lines,
//     16 bytes per lane, one pair ahead, double-buffered, issued between the matrix
//     instructions of the pair's first step); 16-byte units are XOR-swizzled by row so the
//     operand reads are conflict-free;
//   * each wave reads its raw weights back and rebuilds them in registers,
//         W_eff = bf16(fp32(w) + (bit ? +alpha : -alpha))   (round to nearest even),
//     one bf16 dot-product instruction per weight for the widening and the add,
//     with the sign words (one 16-byte load per row per 4 steps) in registers one quad ahead,
//     so each weight is rebuilt once, by the wave that multiplies it;
//   * v_mfma_f32_16x16x32_bf16 over 2 row tiles x 16 token tiles, fp32 accumulation.
// One barrier per pair (the activations).  Rounding W_eff to bf16 before the product is the one
// departure from an exact W_eff; the error it adds is below half a bf16 ulp of each weight and
// shows in y far inside the output tolerance.
//
// Tile order: workgroup b runs on XCD b % 8.  Each XCD takes groups of 32 tiles, 4 M tiles by 8
// N tiles, so the workgroups running side by side on it share 4 activation blocks and 8 weight
// blocks in its L2; the 8 XCDs take neighbouring groups (the same N tiles, other M tiles), so
// weight blocks also meet in the memory-side cache.
#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 512;
constexpr int kBK = 32;                            // K per step
constexpr unsigned kXPair = kPrefillBM * 2 * kBK * 2;   // 32 KiB of activations per pair
constexpr unsigned kWPair = kPrefillBN * 2 * kBK * 2;   // 32 KiB of W_base per pair
constexpr unsigned kPair = kXPair + kWPair;
constexpr unsigned kLds = 2 * kPair;                    // double-buffered
static_assert(kLds <= 160 * 1024, "the ring must fit in one compute unit's LDS");
constexpr int kGroupM = 4, kGroupN = 8;            // tiles per XCD group

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// 16 bytes per lane from base + voff straight into LDS at lds_base + 16 * lane
__device__ __forceinline__ void dma16(rsrc_t r, unsigned voff, unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding, n <= 63).
#define PREFILL_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Byte offset of row t's 16-byte unit u in a pair block (units 4 h + c: chunk c of step h of the
// pair, 8 bf16 each): each row's 128 bytes are contiguous, with the units XOR-swizzled by
// (t / 2) % 8 so that 16 consecutive rows reading the same unit hit 16 different banks.
__device__ __forceinline__ unsigned unit_off(int t, int u) {
  return (unsigned)(8 * t + (u ^ ((t >> 1) & 7))) * 16u;
}

// bit 31 of s, bits 0..30 of m (one v_bfi_b32)
__device__ __forceinline__ unsigned sign_into(unsigned s, unsigned m) {
  unsigned r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0x80000000u), "v"(s), "v"(m));
  return r;
}

// 8 bf16 weights (k = pos0 .. pos0+7 of word) -> 8 bf16 of w + (+-alpha).  The widening of each
// weight and the add are one bf16 dot product with one_lo = (1, 0) or one_hi = (0, 1) that
// accumulates onto +-alpha: w * 1 is exact, so the result is fp32(w + (+-alpha)) rounded once.
// nword = ~word: bit k clear gives the sign bit of -alpha.  one_lo and one_hi must come in
// registers: encoded in the instruction as a constant, (1, 0) and (0, 1) are not read as these
// bf16 pairs.
__device__ __forceinline__ u32x4 rebuild8(const u32x4& w, unsigned nword, unsigned pos0,
                                          unsigned abits, bf16x2 one_lo, bf16x2 one_hi) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // through a scalar: a bit cast of the vector element itself reads element 0
    const unsigned wd = w[d];
    const bf16x2 wp = __builtin_bit_cast(bf16x2, wd);
    const unsigned k0 = pos0 + 2 * d;
    const float a0 = __uint_as_float(sign_into(nword << (31u - k0), abits));
    const float a1 = __uint_as_float(sign_into(nword << (30u - k0), abits));
    f32x2 f;
    f[0] = __builtin_amdgcn_fdot2_f32_bf16(wp, one_lo, a0, false);
    f[1] = __builtin_amdgcn_fdot2_f32_bf16(wp, one_hi, a1, false);
    r[d] = __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
  }
  return r;
}

__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(const PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- tile of this workgroup ----------------------------------------------------------------
  // XCD x takes groups x, x + 8, ... of 32 tiles (4 M tiles by 8 N tiles); groups are numbered
  // M-group fastest, so the 8 XCDs work on the same 8 N tiles at a time.
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int ngm = (a.n_mtiles + kGroupM - 1) / kGroupM;
  const int grp = (kk / (kGroupM * kGroupN)) * 8 + xcd, within = kk % (kGroupM * kGroupN);
  const int gm = grp % ngm, gn = grp / ngm;
  const int mt = gm * kGroupM + within % kGroupM, nt = gn * kGroupN + within / kGroupM;
  if (mt >= a.n_mtiles || nt >= a.n_ntiles) return;  // workgroup-uniform

  const int d_in = a.d_in, d_out = a.d_out;
  const int xrow0 = a.mt_row[mt];
  const int nrows = a.mt_rows[mt];
  const int slot = a.mt_slot[mt];
  const int n0 = nt * kPrefillBN;
  const int wpr = d_in >> 5;  // sign words per row
  const int nsteps = d_in / kBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  // the scale of the two rows the lane rebuilds (32w + 16rt + j): the variant's one alpha or the
  // row's; base-model tiles rebuild with alpha = 0, which leaves every weight as it is
  unsigned abits[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int ri = ((a.alpha_rows >> (slot & 31)) & 1u) ? min(n0 + 32 * wave + 16 * rt + j, d_out - 1) : 0;
    abits[rt] = slot >= 0 ? __float_as_uint(a.alpha[slot][ri]) & 0x7FFFFFFFu : 0u;
  }

  // ---- copies of a pair: wave w moves tokens 32w .. 32w + 31 (4 x 1 KiB) and its own weight rows
  // 32w .. 32w + 31 (4 x 1 KiB), 8 rows of 128 bytes per copy: lane L fills stored unit L % 8 of
  // row 8i + L / 8 of the wave's 32, i.e. unit (L % 8) ^ ((row / 2) % 8) of that row ---------
  const rsrc_t xrs = make_rsrc(a.x + (size_t)xrow0 * d_in);
  const rsrc_t wrs = make_rsrc(a.w + (size_t)n0 * d_in);
  auto copy_pair = [&](int p, int i) {  // copy i (0..7) of pair p (past the end: clamped)
    const int r = 32 * wave + 8 * (i & 3) + (lane >> 3);
    const int u = (lane & 7) ^ ((r >> 1) & 7);
    const int sc = min(2 * p + (u >> 2), nsteps - 1);  // the step of this lane's unit
    unsigned char* dst = smem + (unsigned)(p & 1) * kPair + (unsigned)(32 * wave + 8 * (i & 3)) * 128u;
    if (i < 4)
      dma16(xrs, (unsigned)((min(r, nrows - 1) * d_in + sc * kBK + 8 * (u & 3)) * 2), dst);
    else
      dma16(wrs, (unsigned)(((min(n0 + r, d_out - 1) - n0) * d_in + sc * kBK + 8 * (u & 3)) * 2),
            dst + kXPair);
  };

  // ---- sign words: lane (j, g) of row tile rt holds the 4 words of row 32w + 16rt + j for a quad
  // row-major words: the tile's rows start at word n0 * wpr; tiled words (n0 is a multiple of
  // 256, so the tile starts a 128-row block): at word (n0 / 128) * (wpr / 4) * 512
  const bool tiled = slot >= 0 && ((a.tiled >> slot) & 1u);
  const rsrc_t srs = make_rsrc(
      slot >= 0 ? static_cast<const void*>(a.words[slot] + sign_quad_offset(tiled, n0, 0, wpr))
                : static_cast<const void*>(a.w));
  unsigned soff[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    soff[rt] = (unsigned)sign_quad_offset(tiled, min(n0 + 32 * wave + 16 * rt + j, d_out - 1) - n0,
                                          0, wpr) * 4u;
  // 16-byte quads of words: the slot's bit of vec_signs; base-model tiles read (and ignore) W_base
  // bytes, 16 at a time whenever d_in % 128 == 0
  const bool vec_signs = ((unsigned)a.vec_signs >> (slot >= 0 ? slot : 31)) & 1u;
  const unsigned quad_bytes = tiled ? 2048u : 16u;  // bytes between the words of two quads
  auto load_s = [&](u32x4* sw, int q0, int rt) {  // the quad starting at step q0 (clamped)
    if (vec_signs) {
      const int qc = min(q0, (nsteps - 1) & ~3);
      sw[rt] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, soff[rt] + (unsigned)(qc >> 2) * quad_bytes,
                                                        0, 0));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        sw[rt][t] = __builtin_amdgcn_raw_buffer_load_b32(
            srs, soff[rt] + (unsigned)min(q0 + t, nsteps - 1) * 4u, 0, 0);
    }
  };

  f32x4 acc[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand reads: unit 4h + g of token 16 tt + j (B) and of row 32w + 16 rt + j (A)
  const unsigned b_lane[2] = {unit_off(j, g), unit_off(j, 4 + g)};  // + tt * 16 rows * 128 bytes
  const unsigned a_lane[2] = {unit_off(32 * wave + j, g) + kXPair,
                              unit_off(32 * wave + j, 4 + g) + kXPair};  // + rt * 16 * 128

  // the bf16 pairs (1, 0) and (0, 1) of the rebuild, kept in registers the compiler cannot fold
  unsigned one_bits[2] = {0x00003F80u, 0x3F800000u};
  asm volatile("" : "+v"(one_bits[0]), "+v"(one_bits[1]));
  const bf16x2 one_lo = __builtin_bit_cast(bf16x2, one_bits[0]);
  const bf16x2 one_hi = __builtin_bit_cast(bf16x2, one_bits[1]);

  // Step s (h = s % 2 of its pair): rebuild the two weight fragments, multiply by the 16 token
  // tiles.
  // With cp >= 0 the wave also issues its 8 copies of pair cp, one after every second token
  // tile: spread between the matrix instructions they keep the memory queue from filling up
  // and stalling the wave's issue.
  auto mma_step = [&](const u32x4* sw, int s, int cp) {
    const int h = s & 1;
    const unsigned char* pb = smem + (unsigned)((s >> 1) & 1) * kPair;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(pb + a_lane[h]);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(pb + a_lane[h] + 16 * 128);
    const u32x4 A0 = rebuild8(w0, ~sw[0][s & 3], 8u * g, abits[0], one_lo, one_hi);
    const u32x4 A1 = rebuild8(w1, ~sw[1][s & 3], 8u * g, abits[1], one_lo, one_hi);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const u32x4 B = *reinterpret_cast<const u32x4*>(pb + b_lane[h] + tt * 16 * 128);
      acc[0][tt] = mfma(A0, B, acc[0][tt]);
      acc[1][tt] = mfma(A1, B, acc[1][tt]);
      if (cp >= 0 && (tt & 1) == 1) copy_pair(cp, tt >> 1);
    }
  };
  // A quad (two pairs): steps q0 .. q0 + 3 with the sign words cur, while the next pair's copies
  // go out between the matrix instructions of each pair's first step and the next quad's sign
  // words into nxt; everything a pair issued is waited for before the barrier that ends it.
  auto quad = [&](const u32x4* cur, u32x4* nxt, int q0) {
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const int p = (q0 >> 1) + hp;
      load_s(nxt, q0 + 4, hp);
      if (2 * p < nsteps) {
        mma_step(cur, 2 * p, p + 1);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) copy_pair(p + 1, i);
      }
      if (2 * p + 1 < nsteps) mma_step(cur, 2 * p + 1, -1);
      PREFILL_VMCNT(0);
      __syncthreads();
    }
  };

  // ---- prologue: pair 0 and the sign words of quad 0 -------------------------------------------
  u32x4 sa[2], sb[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) copy_pair(0, i);
  load_s(sa, 0, 0);
  load_s(sa, 0, 1);
  PREFILL_VMCNT(0);
  __syncthreads();

  int q0 = 0;
  for (; q0 + 4 < nsteps; q0 += 8) {
    quad(sa, sb, q0);
    quad(sb, sa, q0 + 4);
  }
  if (q0 < nsteps) quad(sa, sb, q0);

  // ---- epilogue: lane holds rows 4g..4g+3 of each row tile for token j of each token tile ----
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    const int tok = tt * 16 + j;
    if (tok < nrows) {
      const size_t ybase = (size_t)(xrow0 + tok) * d_out;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int orow = n0 + 32 * wave + rt * 16 + 4 * g;
        const f32x4 v = acc[rt][tt];
        if (a.y_f32) {
          float* y = reinterpret_cast<float*>(a.y) + ybase;
          if (orow + 3 < d_out && (d_out & 3) == 0) {
            *reinterpret_cast<f32x4*>(y + orow) = v;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (orow + r < d_out) y[orow + r] = v[r];
          }
        } else {
          uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + ybase;
          if (orow + 3 < d_out && (d_out & 3) == 0) {
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
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.n_mtiles < 1 || a.n_mtiles > kPrefillMaxMTiles || a.n_ntiles < 1 || a.d_in < kBK ||
      a.d_in % kBK != 0 || a.d_out < 1)
    return hipErrorInvalidValue;
  // 31-bit buffer offsets within one tile's activations, weights and sign words
  if ((int64_t)kPrefillBM * a.d_in * 2 >= (int64_t(1) << 31) ||
      (int64_t)kPrefillBN * a.d_in * 2 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  for (int m = 0; m < a.n_mtiles; ++m)
    if (a.mt_rows[m] < 1 || a.mt_rows[m] > kPrefillBM) return hipErrorInvalidValue;
  static DeviceOnce once;
  hipError_t e = set_dynamic_lds_once(once, reinterpret_cast<const void*>(&prefill_kernel), (int)kLds);
  if (e != hipSuccess) return e;
  // grid: 8 XCD lists of whole 32-tile groups
  const int ngroups = ((a.n_mtiles + kGroupM - 1) / kGroupM) * ((a.n_ntiles + kGroupN - 1) / kGroupN);
  const int nblocks = ((ngroups + 7) / 8) * 8 * kGroupM * kGroupN;
  clear_stale_error();
  hipLaunchKernelGGL(prefill_kernel, dim3(nblocks), dim3(kThreads), kLds, stream, a);
  return hipGetLastError();
}

}  // namespace bd
