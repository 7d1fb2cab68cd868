// Decode GEMV for very small batches (M <= 4 tokens): the fused reconstruct-and-multiply of
// the BitDelta post ("Serving architecture", conceptual fused linear) with the reconstructed
// weight W_eff = W_base + alpha_v * sign_v formed in fp32 registers, element by element, and
// never stored.
//
// A wave owns kRows consecutive output rows.  Per 512-column chunk each lane loads 8 consecutive
// bf16 of every row (one 16-byte load per row; the wave covers 512 contiguous elements of each
// row) and the one sign word holding their bits (kU chunks' loads are issued together), widens the weights to fp32, applies +-alpha from
// the bit by inserting the sign into alpha's bit pattern, and multiply-adds with the lane's 8
// activations of each token (fp32 accumulation).  Tokens are in segment order, so a token
// either reuses the previous token's reconstructed value or rebuilds it for its own variant.
// A final wave reduction gives each (token, row) sum; the row's outputs are rounded to bf16
// (nearest-even) or stored as fp32.
#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;  // output rows per wave
// 512-column chunks whose loads are in flight together: more for fewer tokens, so the registers
// of the unrolled loads stay within two waves per SIMD
template <int M>
constexpr int chunks_in_flight() { return M == 1 ? 4 : (M == 2 ? 2 : 1); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// +alpha if bit `pos` of `word` is set, -alpha otherwise.
__device__ __forceinline__ float signed_alpha(unsigned alpha_bits, unsigned word, unsigned pos) {
  return __uint_as_float(alpha_bits | ((~(word << (31u - pos))) & 0x80000000u));
}

template <int M>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * (kThreads / 64) + wave) * kRows;
  if (row0 >= a.d_out) return;  // the whole wave is past the last row
  const int d_in = a.d_in;
  const int wpr = d_in >> 5;  // sign words per row

  int slot[M];
  bool fresh[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    slot[t] = a.tok_slot[t];
    fresh[t] = (t == 0) || (slot[t] != slot[t - 1]);
  }

  const uint16_t* wrow[kRows];
  int rowc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    rowc[r] = min(row0 + r, a.d_out - 1);  // rows past the end read the last row; not stored
    wrow[r] = a.w + (size_t)rowc[r] * d_in;
  }
  // the scale of each (row, token): the variant's one alpha, or its row's alpha
  unsigned abits[kRows][M];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int t = 0; t < M; ++t)
      abits[r][t] = slot[t] >= 0 ? __float_as_uint(a.alpha[slot[t]][((a.alpha_rows >> slot[t]) & 1u)
                                                                          ? rowc[r]
                                                                          : 0])
                                 : 0u;

  float acc[kRows][M];
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int t = 0; t < M; ++t) acc[r][t] = 0.f;

  const unsigned pos0 = 8u * (unsigned)(lane & 3);  // bit of the lane's first element in its word

  // Each iteration covers kU chunks of 512 columns: every load of the kU chunks is issued before
  // any is used, so a wave keeps kU * kRows 16-byte weight loads (plus their words and the
  // activations) in flight.  Columns past d_in read as zero activations and are skipped.
  constexpr int kU = chunks_in_flight<M>();
  for (int kb = lane * 8; kb < d_in; kb += 512 * kU) {
    u32x4 wv[kU][kRows];
    unsigned word[kU][kRows][M];
    u32x4 xv[kU][M];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k0 = kb + 512 * u;
      const bool in = k0 < d_in;
      const int wi = k0 >> 5;
#pragma unroll
      for (int t = 0; t < M; ++t)
        xv[u][t] = in ? *reinterpret_cast<const u32x4*>(a.x + (size_t)t * d_in + k0)
                      : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        wv[u][r] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + k0))
                      : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < M; ++t) {
          if (slot[t] >= 0 && fresh[t])
            word[u][r][t] = in ? a.words[slot[t]][sign_quad_offset((a.tiled >> slot[t]) & 1u, rowc[r],
                                                                   wi >> 2, wpr) + (wi & 3)]
                               : 0u;
          else
            word[u][r][t] = t > 0 ? word[u][r][t - 1] : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // activations of every token, widened to fp32
      float xf[M][8];
#pragma unroll
      for (int t = 0; t < M; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          xf[t][2 * d] = bf16lo_to_f32(xv[u][t][d]);
          xf[t][2 * d + 1] = bf16hi_to_f32(xv[u][t][d]);
        }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float wf = (e & 1) ? bf16hi_to_f32(wv[u][r][e >> 1]) : bf16lo_to_f32(wv[u][r][e >> 1]);
          float weff = wf;
#pragma unroll
          for (int t = 0; t < M; ++t) {
            if (fresh[t])
              weff = slot[t] >= 0 ? wf + signed_alpha(abits[r][t], word[u][r][t], pos0 + e) : wf;
            acc[r][t] = fmaf(weff, xf[t][e], acc[r][t]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int t = 0; t < M; ++t) acc[r][t] = wave_sum(acc[r][t]);

  // lane (r * M + t) stores y[t][row0 + r]
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int t = 0; t < M; ++t)
      if (lane == r * M + t && row0 + r < a.d_out) {
        const size_t o = (size_t)t * a.d_out + row0 + r;
        if (a.y_f32)
          reinterpret_cast<float*>(a.y)[o] = acc[r][t];
        else
          reinterpret_cast<uint16_t*>(a.y)[o] = (uint16_t)f32_to_bf16_rne(acc[r][t]);
      }
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int rows_per_block = kRows * (kThreads / 64);
  const dim3 grid((a.d_out + rows_per_block - 1) / rows_per_block);
  clear_stale_error();
  switch (a.M) {
    case 1: hipLaunchKernelGGL(gemv_kernel<1>, grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(gemv_kernel<2>, grid, dim3(kThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(gemv_kernel<3>, grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(gemv_kernel<4>, grid, dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bd
