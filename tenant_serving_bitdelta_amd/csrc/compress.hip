// Compression of one delta matrix (BitDelta post, "The mathematical foundation"):
//   alpha = ||Delta||_1 / n  (mean absolute value over every element), and
//   one sign bit per element, packed least-significant-bit first along d_in into uint32
//   words (bit 1 = +1), the byte image of the post's eight-bits-per-int8 storage format
//   ("Infrastructure details").
//
// Pass 1 streams Delta once with 16-byte loads.  A wave covers 256 consecutive elements per
// iteration: lane l holds elements 4l..4l+3, so the 32 elements of one output word live in the
// 8 lanes 8w..8w+7; their 4-bit groups are OR-combined across those lanes and one lane stores
// the word.  |Delta| is accumulated in fp64 per lane and reduced per workgroup into one fp64
// partial.  Pass 2 sums the partials in a fixed order and rounds sum/n once to float32, so the
// result is identical from run to run (no atomics anywhere).
//
// Optionally pass 1 also writes a second copy of the sign words in the tiled layout the
// split-activation decode kernel streams: for every block of 128 rows and every 128-column step,
// the 4 words of each of the 128 rows lie in one contiguous 2 KiB chunk,
//   tiled word ((r / 128) * (d_in / 128) + c / 4) * 512 + (r % 128) * 4 + c % 4  <-  word (r, c),
// so a block's sign words for one step are read as whole cache lines.  Rows past d_out in the
// last block are not written.
#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;        // float4 loads in flight per lane
constexpr int kMaxGrid = 2048;    // workgroups (= partials) at most

// 1 if v is strictly negative (negative zero is not); works on the bit pattern so negative
// subnormals count as negative whatever the denormal mode.
__device__ __forceinline__ unsigned is_negative(float v) {
  unsigned u = __float_as_uint(v);
  return (u >> 31) & (unsigned)((u & 0x7FFFFFFFu) != 0u);
}

__device__ __forceinline__ unsigned nonneg_nibble(f32x4 v) {
  return (is_negative(v[0]) ^ 1u) | ((is_negative(v[1]) ^ 1u) << 1) |
         ((is_negative(v[2]) ^ 1u) << 2) | ((is_negative(v[3]) ^ 1u) << 3);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kThreads) void compress_pass1(const f32x4* __restrict__ delta,
                                                          int64_t n4,
                                                          uint32_t* __restrict__ words,
                                                          uint32_t* __restrict__ tiled,
                                                          int64_t wpr,
                                                          double* __restrict__ partials) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64) * 64;   // float4 per sweep
  int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * 64;
  double acc = 0.0;
  const unsigned shift = 4u * (unsigned)(lane & 7);

  for (; base < n4; base += stride * kUnroll) {
    f32x4 v[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * stride + lane;
      ok[u] = i < n4;
      v[u] = ok[u] ? __builtin_nontemporal_load(delta + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * stride + lane;
      acc += fabs((double)v[u][0]);
      acc += fabs((double)v[u][1]);
      acc += fabs((double)v[u][2]);
      acc += fabs((double)v[u][3]);
      unsigned part = nonneg_nibble(v[u]) << shift;
      part |= __shfl_xor(part, 1);
      part |= __shfl_xor(part, 2);
      part |= __shfl_xor(part, 4);
      // n is a multiple of 32, so the 8 lanes of a word are all in range or all out of range.
      if ((lane & 7) == 0 && ok[u]) {
        const int64_t w = i >> 3;
        words[w] = part;
        if (tiled) {
          const int64_t r = w / wpr, c = w - r * wpr;
          tiled[((r >> 7) * (wpr >> 2) + (c >> 2)) * 512 + (r & 127) * 4 + (c & 3)] = part;
        }
      }
    }
  }

  __shared__ double wsum[kThreads / 64];
  acc = wave_sum(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += wsum[w];
    partials[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(kThreads) void compress_pass2(const double* __restrict__ partials,
                                                          int nparts, double n,
                                                          float* __restrict__ alpha) {
  double s = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) s += partials[i];
  __shared__ double red[kThreads];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int width = kThreads / 2; width >= 1; width >>= 1) {
    if ((int)threadIdx.x < width) red[threadIdx.x] += red[threadIdx.x + width];
    __syncthreads();
  }
  if (threadIdx.x == 0) alpha[0] = (float)(red[0] / n);
}

}  // namespace

int compress_grid(int64_t n) {
  const int64_t n4 = n / 4;
  const int64_t per_block = (int64_t)kThreads * kUnroll;  // float4 per workgroup per sweep
  int64_t g = (n4 + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > kMaxGrid) g = kMaxGrid;
  return (int)g;
}

hipError_t launch_compress(const float* delta, int64_t n, int64_t d_in, uint32_t* words,
                           uint32_t* tiled, float* alpha, double* partials, hipStream_t stream) {
  const int grid = compress_grid(n);
  clear_stale_error();
  hipLaunchKernelGGL(compress_pass1, dim3(grid), dim3(kThreads), 0, stream,
                     reinterpret_cast<const f32x4*>(delta), n / 4, words, tiled, d_in / 32,
                     partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_pass2, dim3(1), dim3(kThreads), 0, stream, partials, grid,
                     (double)n, alpha);
  return hipGetLastError();
}

}  // namespace bd
