// Prefill-sized batches: the fused reconstruct-and-multiply of the BitDelta post ("Serving
// architecture": reconstruction in fast on-chip memory, fused with the matmul, W_eff never
// written to HBM) as a dense bf16 MFMA contraction per segment.
//
// A workgroup (8 waves, two per SIMD) computes a tile of 256 tokens (one segment, hence one
// variant) by 256 output rows, walking d_in in steps of 32 grouped in quads of 4 steps.  Wave w
// owns rows 32w .. 32w + 31 for all 256 tokens:
//   * its W_base rows (16 bytes per lane: exactly the bf16 MFMA operand of one row tile) and
//     their sign words (one 16-byte load per row covers the quad) go straight from memory into
//     registers one quad ahead, and each weight is rebuilt in registers by the wave that
//     multiplies it,
//         W_eff = bf16(fp32(w) + (bit ? +alpha : -alpha))   (round to nearest even),
//     so no weight passes through LDS and no other wave waits for it;
//   * the quad's 256x128 block of activations, which every wave needs, goes straight from
//     memory into an 8-step LDS ring (direct global->LDS loads, 16 bytes per lane, one quad
//     ahead, one eighth per wave); 16-byte chunks are XOR-swizzled by token so the operand reads
//     are conflict-free;
//   * v_mfma_f32_16x16x32_bf16 over 2 row tiles x 16 token tiles, fp32 accumulation.
// The next quad's loads are spread over the first steps of the quad, between the MFMAs; one
// barrier per quad.  Rounding W_eff to bf16 before the product is the one departure from an
// exact W_eff; the error it adds is below half a bf16 ulp of each weight and shows in y far
// inside the output tolerance.
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
constexpr int kStages = 8;                         // activation ring
constexpr int kAhead = kStages - 1;                // copies issued this many steps ahead
constexpr unsigned kXBytes = kPrefillBM * kBK * 2;  // 16 KiB of activations per stage
constexpr unsigned kLds = kStages * kXBytes;
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

// Byte offset in a stage of token r's 16-byte chunk c (4 chunks of 8 bf16 per token).
__device__ __forceinline__ unsigned chunk_off(int r, int c) {
  return (unsigned)(4 * r + (c ^ ((r >> 2) & 3))) * 16u;
}

// +alpha where bit `pos` of word is set, -alpha where it is clear (alpha_bits: |alpha|)
__device__ __forceinline__ float signed_alpha(unsigned alpha_bits, unsigned word, unsigned pos) {
  return __uint_as_float(alpha_bits | ((~(word << (31u - pos))) & 0x80000000u));
}

// 8 bf16 weights (k = pos0 .. pos0+7 of word) -> 8 bf16 of w + (+-alpha)
__device__ __forceinline__ u32x4 rebuild8(const u32x4& w, unsigned word, unsigned pos0,
                                          unsigned abits) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f32x2 f;
    f[0] = bf16lo_to_f32(w[d]) + signed_alpha(abits, word, pos0 + 2 * d);
    f[1] = bf16hi_to_f32(w[d]) + signed_alpha(abits, word, pos0 + 2 * d + 1);
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
  // base-model tiles rebuild with alpha = 0, which leaves every weight as it is
  const unsigned abits = slot >= 0 ? __float_as_uint(*a.alpha[slot]) & 0x7FFFFFFFu : 0u;
  const int n0 = nt * kPrefillBN;
  const int wpr = d_in >> 5;  // sign words per row
  const int nsteps = d_in / kBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;

  // ---- activation copies: wave w moves tokens 32w .. 32w + 31 of each step (2 x 1 KiB) --------
  const rsrc_t xrs = make_rsrc(a.x + (size_t)xrow0 * d_in);
  unsigned xoff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // block i = 2 wave + u covers tokens 16 i .. 16 i + 15; lane L fills stored chunk L % 4 of
    // token 16 i + L / 4, i.e. chunk (L % 4) ^ ((token >> 2) & 3) of that token
    const int tok = 16 * (2 * wave + u) + (lane >> 2);
    const int c = (lane & 3) ^ ((tok >> 2) & 3);
    xoff[u] = (unsigned)((min(tok, nrows - 1) * d_in + 8 * c) * 2);
  }
  auto copy_x = [&](int s, int u) {  // step s (clamped: past the end it reloads the last step)
    const int sc = min(s, nsteps - 1);
    dma16(xrs, xoff[u] + (unsigned)sc * (kBK * 2),
          smem + (unsigned)(s % kStages) * kXBytes + (2 * wave + u) * 1024);
  };

  // ---- weights: lane (j, g) of row tile rt holds row 32w + 16rt + j, columns 8g .. 8g + 7 ------
  const rsrc_t wrs = make_rsrc(a.w + (size_t)n0 * d_in);
  const rsrc_t srs = make_rsrc(slot >= 0 ? static_cast<const void*>(a.words[slot] + (size_t)n0 * wpr)
                                         : static_cast<const void*>(a.w));
  unsigned woff[2], soff[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = min(n0 + 32 * wave + 16 * rt + j, d_out - 1) - n0;
    woff[rt] = (unsigned)(r * d_in + 8 * g) * 2u;
    soff[rt] = (unsigned)(r * wpr) * 4u;
  }
  // Registers of one quad: raw weights [step][row tile] and the sign words [row tile] (word t of
  // the 16-byte load belongs to step t of the quad; with d_in % 128 != 0 the words are loaded one
  // by one).  Past the last step, loads are clamped to it (in-range data nobody uses).
  struct Quad {
    u32x4 w[4][2];
    u32x4 sw[2];
  };
  const bool vec_signs = a.vec_signs != 0;
  auto load_w = [&](Quad& Q, int s, int rt) {  // step s of the quad starting at (s & ~3)
    const int sc = min(s, nsteps - 1);
    Q.w[s & 3][rt] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, woff[rt] + (unsigned)sc * (kBK * 2), 0, 0));
  };
  auto load_s = [&](Quad& Q, int q0, int rt) {  // sign words of the quad starting at step q0
    if (vec_signs) {
      const int qc = min(q0, (nsteps - 1) & ~3);
      Q.sw[rt] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, soff[rt] + (unsigned)qc * 4u, 0, 0));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        Q.sw[rt][t] = __builtin_amdgcn_raw_buffer_load_b32(
            srs, soff[rt] + (unsigned)min(q0 + t, nsteps - 1) * 4u, 0, 0);
    }
  };

  f32x4 acc[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const unsigned b_lane = chunk_off(j, g);  // + tt * 16 tokens * 64 bytes

  // One step of a quad: rebuild this step's two weight fragments, multiply by the 16 token tiles
  // of the stage.
  auto mma_step = [&](const Quad& Q, int s) {
    const int t = s & 3;
    const u32x4 A0 = rebuild8(Q.w[t][0], Q.sw[0][t], 8u * g, abits);
    const u32x4 A1 = rebuild8(Q.w[t][1], Q.sw[1][t], 8u * g, abits);
    const unsigned char* st = smem + (unsigned)(s % kStages) * kXBytes + b_lane;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const u32x4 B = *reinterpret_cast<const u32x4*>(st + tt * 1024);
      acc[0][tt] = mfma(A0, B, acc[0][tt]);
      acc[1][tt] = mfma(A1, B, acc[1][tt]);
    }
  };
  // A quad: steps q0 .. q0 + 3 from registers cur, while the loads of the next quad (activations
  // into the other half of the ring, weights and signs into nxt) go out during its first two
  // steps; all of them must be in before the barrier that ends the quad.
  auto quad = [&](const Quad& cur, Quad& nxt, int q0) {
    const int q1 = q0 + 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 2) {
        copy_x(q1 + 2 * t, 0);
        copy_x(q1 + 2 * t, 1);
        copy_x(q1 + 2 * t + 1, 0);
        copy_x(q1 + 2 * t + 1, 1);
        load_w(nxt, q1 + 2 * t, 0);
        load_w(nxt, q1 + 2 * t, 1);
        load_w(nxt, q1 + 2 * t + 1, 0);
        load_w(nxt, q1 + 2 * t + 1, 1);
        load_s(nxt, q1, t);
      }
      if (q0 + t < nsteps) mma_step(cur, q0 + t);
    }
    PREFILL_VMCNT(0);
    __syncthreads();
  };

  // ---- prologue: the first quad --------------------------------------------------------------
  Quad qa, qb;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    copy_x(t, 0);
    copy_x(t, 1);
    load_w(qa, t, 0);
    load_w(qa, t, 1);
  }
  load_s(qa, 0, 0);
  load_s(qa, 0, 1);
  PREFILL_VMCNT(0);
  __syncthreads();

  int q0 = 0;
  for (; q0 + 4 < nsteps; q0 += 8) {
    quad(qa, qb, q0);
    quad(qb, qa, q0 + 4);
  }
  if (q0 < nsteps) quad(qa, qb, q0);

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
  static bool configured = false;  // benign race: every caller sets the same value
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  // grid: 8 XCD lists of whole 32-tile groups
  const int ngroups = ((a.n_mtiles + kGroupM - 1) / kGroupM) * ((a.n_ntiles + kGroupN - 1) / kGroupN);
  const int nblocks = ((ngroups + 7) / 8) * 8 * kGroupM * kGroupN;
  clear_stale_error();
  hipLaunchKernelGGL(prefill_kernel, dim3(nblocks), dim3(kThreads), kLds, stream, a);
  return hipGetLastError();
}

}  // namespace bd
