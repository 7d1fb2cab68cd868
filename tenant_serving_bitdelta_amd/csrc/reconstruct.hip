// Two HBM-bound helpers around the fused path.
//
// reconstruct_kernel: the unfused form of the BitDelta post's reconstruction ("Serving
// architecture": W_eff = W_base + alpha * sign(Delta), which the post's fused kernel never
// writes to HBM).  It writes W_eff as a bf16 matrix, so a plain product with it measures what
// the fused kernels save.  Element by element: bf16_RNE(fp32(w) + (+-alpha)), one fp32 addition
// (the same rounding the prefill kernel's in-register rebuild applies).  A lane takes 8
// consecutive weights (16 bytes) and the byte of their sign bits; a wave covers 512 columns of
// one row, grid-stride over rows and column chunks.
//
// retile_kernel: row-major sign words -> the 128-row tiled layout the matmul kernels stream (the
// storage format of "Infrastructure details" is the row-major packing; the tiled one is how the
// words sit in HBM for the kernels).  A workgroup takes one 128-row block and 8 steps of 128
// columns: it reads each row's 128 contiguous bytes of those steps and writes the 8 chunks of
// 2 KiB, through LDS.  Rows past d_out are not written (the kernels never read them for a real
// output row).
#include <algorithm>

#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kRecThreads = 256;
constexpr int kRetileThreads = 256;
constexpr int kRetileSteps = 8;  // 128-column steps per workgroup

__global__ __launch_bounds__(kRecThreads) void reconstruct_kernel(
    const uint16_t* __restrict__ w, const uint32_t* __restrict__ words, int tiled,
    const float* __restrict__ alpha, int alpha_per_row, int d_out, int d_in,
    uint16_t* __restrict__ w_eff) {
  const int wpr = d_in >> 5;
  const int chunks = (d_in + 511) >> 9;  // 512-column chunks per row
  const int64_t units = (int64_t)d_out * chunks;
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (int64_t)blockIdx.x * (kRecThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kRecThreads / 64);
  for (int64_t u = wave0; u < units; u += nwaves) {
    const int r = (int)(u / chunks);
    const int k0 = (int)(u - (int64_t)r * chunks) * 512 + lane * 8;
    if (k0 >= d_in) continue;  // d_in % 32 == 0: a lane's 8 columns are all in or all out
    const unsigned ab = __float_as_uint(alpha[alpha_per_row ? r : 0]) & 0x7FFFFFFFu;
    const int c = k0 >> 5;
    const unsigned word = words[sign_quad_offset(tiled != 0, r, c >> 2, wpr) + (c & 3)];
    const unsigned byte = word >> (k0 & 31);
    const size_t e0 = (size_t)r * d_in + k0;
    const u32x4 wv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w + e0));
    u32x4 out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // bit 1 -> +alpha, bit 0 -> -alpha: the sign bit of alpha's pattern is the inverted bit
      const float a0 = __uint_as_float(ab | ((~byte << (31 - 2 * d)) & 0x80000000u));
      const float a1 = __uint_as_float(ab | ((~byte << (30 - 2 * d)) & 0x80000000u));
      const unsigned lo = f32_to_bf16_rne(bf16lo_to_f32(wv[d]) + a0);
      const unsigned hi = f32_to_bf16_rne(bf16hi_to_f32(wv[d]) + a1);
      out[d] = lo | (hi << 16);
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(w_eff + e0));
  }
}

__global__ __launch_bounds__(kRetileThreads) void retile_kernel(const uint32_t* __restrict__ src,
                                                                int d_out, int wpr,
                                                                uint32_t* __restrict__ dst) {
  __shared__ __align__(16) u32x4 buf[kRetileSteps][128];
  const int rb = blockIdx.x, q0 = blockIdx.y * kRetileSteps;
  const int nq = wpr >> 2;
  // read: item i = (row i / 8, step i % 8), 16 bytes each; 8 consecutive lanes read one row's
  // 128 contiguous bytes
  for (int i = threadIdx.x; i < 128 * kRetileSteps; i += kRetileThreads) {
    const int row = i / kRetileSteps, q = i % kRetileSteps;
    const int r = rb * 128 + row;
    if (r < d_out && q0 + q < nq)
      buf[q][row] = *reinterpret_cast<const u32x4*>(src + (size_t)r * wpr + 4 * (size_t)(q0 + q));
  }
  __syncthreads();
  // write: item i = (step i / 128, row i % 128): each step's chunk is 2 KiB contiguous
  for (int i = threadIdx.x; i < 128 * kRetileSteps; i += kRetileThreads) {
    const int q = i / 128, row = i % 128;
    const int r = rb * 128 + row;
    if (r < d_out && q0 + q < nq)
      *reinterpret_cast<u32x4*>(dst + sign_quad_offset(true, r, q0 + q, wpr)) = buf[q][row];
  }
}

}  // namespace

hipError_t launch_reconstruct(const uint16_t* w, const uint32_t* words, int tiled,
                              const float* alpha, int alpha_per_row, int64_t d_out, int64_t d_in,
                              uint16_t* w_eff, hipStream_t stream) {
  if (d_out < 1 || d_in < 32 || d_in % 32 != 0 || (tiled && d_in % 128 != 0))
    return hipErrorInvalidValue;
  const int64_t units = d_out * ((d_in + 511) / 512);
  const int64_t per_block = kRecThreads / 64;
  const int grid = (int)std::min<int64_t>((units + per_block - 1) / per_block, 8192);
  clear_stale_error();
  hipLaunchKernelGGL(reconstruct_kernel, dim3(grid), dim3(kRecThreads), 0, stream, w, words,
                     tiled, alpha, alpha_per_row, (int)d_out, (int)d_in, w_eff);
  return hipGetLastError();
}

hipError_t launch_retile(const uint32_t* src, int64_t d_out, int64_t d_in, uint32_t* dst,
                         hipStream_t stream) {
  if (d_out < 1 || d_in < 128 || d_in % 128 != 0) return hipErrorInvalidValue;
  const int nq = (int)(d_in / 128);
  const dim3 grid((unsigned)((d_out + 127) / 128), (unsigned)((nq + kRetileSteps - 1) / kRetileSteps));
  clear_stale_error();
  hipLaunchKernelGGL(retile_kernel, grid, dim3(kRetileThreads), 0, stream, src, (int)d_out,
                     (int)(d_in / 32), dst);
  return hipGetLastError();
}

}  // namespace bd
