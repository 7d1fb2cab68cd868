// Compression of one delta matrix (BitDelta post, "The mathematical foundation"):
//   alpha = ||Delta||_1 / n  (mean absolute value over every element), and
//   one sign bit per element, packed least-significant-bit first along d_in into uint32
//   words (bit 1 = +1), the byte image of the post's eight-bits-per-int8 storage format
//   ("Infrastructure details").
//
// Pass 1 streams Delta once with 16-byte loads; a lane holds 4 consecutive elements, so the 32
// elements of one output word live in 8 neighbouring lanes, whose 4-bit groups are OR-combined
// with three shuffles.  Two forms:
//  * row tiles (d_in a multiple of 128, word arrays 16-byte aligned): a workgroup of 8 waves
//    takes 8 rows x 1024 columns (32 KiB of Delta), one row per wave.  The 256 words of a tile
//    are gathered in LDS and written as whole 128-byte lines: one line per row of the plain
//    words, and, for the tiled copy below, one line per 4-word column group holding the tile's
//    8 rows.  Scattered 4-byte word stores interleave many small writes with the read stream,
//    which costs HBM far more than their byte count.
//  * flat (any d_in that is a multiple of 32): a grid-stride sweep in which one lane of each
//    8 stores the word (and its tiled copy) directly.
// |Delta| is accumulated in fp64 per lane (each lane's 4 elements are first added in fp32, a
// relative error below 2^-23 of that group) and reduced per workgroup into one fp64 partial.
// Pass 2 sums the partials in a fixed order and rounds sum/n once to float32, so the result is
// identical from run to run (no atomics anywhere).
//
// Pass 1 writes the row-major words, the tiled layout below, or both (either pointer may be
// null, not both).  The tiled layout is the one every matmul kernel streams: for every block of
// 128 rows and every 128-column step,
// the 4 words of each of the 128 rows lie in one contiguous 2 KiB chunk,
//   tiled word ((r / 128) * (d_in / 128) + c / 4) * 512 + (r % 128) * 4 + c % 4  <-  word (r, c),
// so a block's sign words for one step are read as whole cache lines.  Rows past d_out in the
// last block are not written.
#include <algorithm>

#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 256;        // flat pass 1 and pass 2
constexpr int kUnroll = 4;           // flat: float4 loads in flight per lane
constexpr int kMaxGrid = 2048;       // flat: workgroups (= partials) at most
constexpr int kTileWaves = 8;        // row tiles: one row per wave
constexpr int kTileCols = 1024;      // row tiles: columns per tile (4 float4 loads per lane)
constexpr int kMaxTileGrid = 16384;  // row tiles: workgroups (= partials) at most
constexpr int kPass2Threads = 1024;

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

// Flat form.  kSmall: fewer than 2^32 words, so word indices and their row / column split fit
// 32-bit math.
template <bool kSmall>
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
      acc += (double)((fabsf(v[u][0]) + fabsf(v[u][1])) + (fabsf(v[u][2]) + fabsf(v[u][3])));
      unsigned part = nonneg_nibble(v[u]) << shift;
      part |= __shfl_xor(part, 1);
      part |= __shfl_xor(part, 2);
      part |= __shfl_xor(part, 4);
      // n is a multiple of 32, so the 8 lanes of a word are all in range or all out of range.
      if ((lane & 7) == 0 && ok[u]) {
        const int64_t w = i >> 3;
        if (words) words[w] = part;
        if (tiled) {
          if (kSmall) {
            const unsigned w32 = (unsigned)w, wpr32 = (unsigned)wpr;
            const unsigned r = w32 / wpr32, c = w32 - r * wpr32;
            tiled[((size_t)(r >> 7) * (wpr32 >> 2) + (c >> 2)) * 512 + (r & 127) * 4 + (c & 3)] = part;
          } else {
            const int64_t r = w / wpr, c = w - r * wpr;
            tiled[((r >> 7) * (wpr >> 2) + (c >> 2)) * 512 + (r & 127) * 4 + (c & 3)] = part;
          }
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

// Row-tile form.  Tile t covers rows 8 (t / ncg) .. +7 and columns 1024 (t % ncg) .. +1023
// (ncg = ceil(d_in / 1024)); rows past d_out and columns past d_in are skipped.  Per-matrix
// scale (kRows = false): d_in % 128 == 0 and 16-byte aligned words, so a 4-word group is wholly
// inside or outside the row; one fp64 partial per workgroup.  Per-row scales (kRows = true): any
// d_in % 32 == 0 (words stored one by one unless vec), one fp64 partial per row and column
// group, partials[r * ncg + cg].
template <bool kRows>
__global__ __launch_bounds__(kTileWaves * 64) void compress_tiles(
    const float* __restrict__ delta, int64_t d_out, int64_t d_in, uint32_t* __restrict__ words,
    uint32_t* __restrict__ tiled, int vec_words, double* __restrict__ partials) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wpr = d_in >> 5;
  const int64_t ncg = (d_in + kTileCols - 1) / kTileCols;
  const int64_t ntiles = (d_out + kTileWaves - 1) / kTileWaves * ncg;
  const unsigned shift = 4u * (unsigned)(lane & 7);
  // sign words of the tile: [row][32 words], two buffers so one barrier per tile suffices
  __shared__ __align__(16) uint32_t tw[2][kTileWaves][kTileCols / 32];
  double acc = 0.0;
  int buf = 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x, buf ^= 1) {
    const int64_t rg = t / ncg, cg = t - rg * ncg;
    const int64_t r = rg * kTileWaves + wave;
    f32x4 v[kTileCols / 256];
#pragma unroll
    for (int u = 0; u < kTileCols / 256; ++u) {
      const int64_t c = cg * kTileCols + u * 256 + lane * 4;
      v[u] = (r < d_out && c < d_in)
                 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(delta + r * d_in + c))
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double tacc = 0.0;
#pragma unroll
    for (int u = 0; u < kTileCols / 256; ++u) {
      const double grp =
          (double)((fabsf(v[u][0]) + fabsf(v[u][1])) + (fabsf(v[u][2]) + fabsf(v[u][3])));
      if (kRows)
        tacc += grp;
      else
        acc += grp;
      unsigned part = nonneg_nibble(v[u]) << shift;
      part |= __shfl_xor(part, 1);
      part |= __shfl_xor(part, 2);
      part |= __shfl_xor(part, 4);
      if ((lane & 7) == 0) tw[buf][wave][u * 8 + (lane >> 3)] = part;
    }
    if (kRows) {
      tacc = wave_sum(tacc);
      if (lane == 0 && r < d_out) partials[r * ncg + cg] = tacc;
    }
    __syncthreads();
    if (wave == 0 && words) {
      // plain words: lane = (row, 4-word group); the 8 lanes of a row fill its 128-byte line
      const int row = lane >> 3, q = lane & 7;
      const int64_t rr = rg * kTileWaves + row, wc = cg * (kTileCols / 32) + q * 4;
      if (rr < d_out && wc < wpr) {
        if (!kRows || vec_words) {
          *reinterpret_cast<u32x4*>(words + rr * wpr + wc) =
              *reinterpret_cast<const u32x4*>(&tw[buf][row][q * 4]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (wc + e < wpr) words[rr * wpr + wc + e] = tw[buf][row][q * 4 + e];
        }
      }
    } else if (wave == kTileWaves - 1 && tiled) {
      // tiled copy: lane = (4-word group, row); the tile's 8 rows of a group are one line
      const int q = lane >> 3, row = lane & 7;
      const int64_t rr = rg * kTileWaves + row, wc = cg * (kTileCols / 32) + q * 4;
      if (rr < d_out && wc < wpr)
        *reinterpret_cast<u32x4*>(tiled + ((rr >> 7) * (wpr >> 2) + (wc >> 2)) * 512 +
                                  (rr & 127) * 4) =
            *reinterpret_cast<const u32x4*>(&tw[buf][row][q * 4]);
    }
  }

  if (kRows) return;
  __shared__ double wsum[kTileWaves];
  acc = wave_sum(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kTileWaves; ++w) sum += wsum[w];
    partials[blockIdx.x] = sum;
  }
}

// Compression of the task vector of a bf16 weight pair, Delta = W_ft - W_base, in the row-tile
// form: a workgroup of 8 waves takes 8 rows x 1024 columns, one row per wave; each lane loads 8
// consecutive weights of both matrices twice (two 1 KiB loads per matrix and wave), so 4 lanes
// hold the 32 elements of one word, one byte each.  Delta is the fp32 difference of the two
// weights (bf16 values widen exactly; the difference is exact unless their exponents are more
// than 16 apart, then rounded once, and it keeps the sign of the exact difference: zero only for
// equal weights, subnormals kept since fp32 denormals are not flushed); 4 consecutive |Delta| are
// added in fp32 and accumulated in fp64, as in the kernels above.
// Words and the tiled copy are gathered in LDS and written as whole lines when the word array is
// 16-byte aligned and d_in % 128 == 0, else word by word.
__global__ __launch_bounds__(kTileWaves * 64) void compress_pair_tiles(
    const uint16_t* __restrict__ w_ft, const uint16_t* __restrict__ w_base, int64_t d_out,
    int64_t d_in, uint32_t* __restrict__ words, uint32_t* __restrict__ tiled, int vec,
    double* __restrict__ partials) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wpr = d_in >> 5;
  const int64_t ncg = (d_in + kTileCols - 1) / kTileCols;
  const int64_t ntiles = (d_out + kTileWaves - 1) / kTileWaves * ncg;
  const unsigned shift = 8u * (unsigned)(lane & 3);
  __shared__ __align__(16) uint32_t tw[2][kTileWaves][kTileCols / 32];
  double acc = 0.0;
  int buf = 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x, buf ^= 1) {
    const int64_t rg = t / ncg, cg = t - rg * ncg;
    const int64_t r = rg * kTileWaves + wave;
    u32x4 a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t c = cg * kTileCols + u * 512 + lane * 8;
      const bool ok = r < d_out && c < d_in;
      a[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w_ft + r * d_in + c))
                : u32x4{0u, 0u, 0u, 0u};
      b[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w_base + r * d_in + c))
                : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      unsigned byte = 0u;
      float grp[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned wa = a[u][e >> 1], wb = b[u][e >> 1];
        const float fa = __uint_as_float((e & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
        const float fb = __uint_as_float((e & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
        const float d = fa - fb;
        byte |= (is_negative(d) ^ 1u) << e;
        grp[e >> 2] += fabsf(d);
      }
      acc += (double)grp[0];
      acc += (double)grp[1];
      unsigned part = byte << shift;
      part |= __shfl_xor(part, 1);
      part |= __shfl_xor(part, 2);
      if ((lane & 3) == 0) tw[buf][wave][u * 16 + (lane >> 2)] = part;
    }
    __syncthreads();
    if (wave == 0 && words) {
      const int row = lane >> 3, q = lane & 7;
      const int64_t rr = rg * kTileWaves + row, wc = cg * (kTileCols / 32) + q * 4;
      if (rr < d_out && wc < wpr) {
        if (vec) {
          *reinterpret_cast<u32x4*>(words + rr * wpr + wc) =
              *reinterpret_cast<const u32x4*>(&tw[buf][row][q * 4]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (wc + e < wpr) words[rr * wpr + wc + e] = tw[buf][row][q * 4 + e];
        }
      }
    } else if (wave == kTileWaves - 1 && tiled) {
      const int q = lane >> 3, row = lane & 7;
      const int64_t rr = rg * kTileWaves + row, wc = cg * (kTileCols / 32) + q * 4;
      if (rr < d_out && wc < wpr)
        *reinterpret_cast<u32x4*>(tiled + ((rr >> 7) * (wpr >> 2) + (wc >> 2)) * 512 +
                                  (rr & 127) * 4) =
            *reinterpret_cast<const u32x4*>(&tw[buf][row][q * 4]);
    }
  }

  __shared__ double wsum[kTileWaves];
  acc = wave_sum(acc);
  if (lane == 0) wsum[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kTileWaves; ++w) sum += wsum[w];
    partials[blockIdx.x] = sum;
  }
}

__global__ __launch_bounds__(kPass2Threads) void compress_pass2(const double* __restrict__ partials,
                                                               int nparts, double n,
                                                               float* __restrict__ alpha) {
  double s = 0.0;
#pragma unroll 4
  for (int i = threadIdx.x; i < nparts; i += kPass2Threads) s += partials[i];
  __shared__ double red[kPass2Threads];
  red[threadIdx.x] = s;
  __syncthreads();
#pragma unroll
  for (int width = kPass2Threads / 2; width >= 1; width >>= 1) {
    if ((int)threadIdx.x < width) red[threadIdx.x] += red[threadIdx.x + width];
    __syncthreads();
  }
  if (threadIdx.x == 0) alpha[0] = (float)(red[0] / n);
}

// Per-row scales: thread r adds row r's column-group partials in column order.
constexpr int kRowsPass2Threads = 256;
__global__ __launch_bounds__(kRowsPass2Threads) void compress_rows_pass2(
    const double* __restrict__ partials, int64_t d_out, int64_t ncg, double d_in,
    float* __restrict__ alpha) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPass2Threads + threadIdx.x;
  if (r >= d_out) return;
  double s = 0.0;
  for (int64_t c = 0; c < ncg; ++c) s += partials[r * ncg + c];
  alpha[r] = (float)(s / d_in);
}

int flat_grid(int64_t n) {
  const int64_t n4 = n / 4;
  const int64_t per_block = (int64_t)kThreads * kUnroll;  // float4 per workgroup per sweep
  int64_t g = (n4 + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > kMaxGrid) g = kMaxGrid;
  return (int)g;
}

int tile_grid(int64_t d_out, int64_t d_in) {
  const int64_t ntiles = (d_out + kTileWaves - 1) / kTileWaves * ((d_in + kTileCols - 1) / kTileCols);
  return (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, kMaxTileGrid));
}

}  // namespace

int64_t compress_partials(int64_t d_out, int64_t d_in) {
  // the row-tile forms (Delta, or a weight pair with any d_in) and the flat form
  return std::max<int64_t>(flat_grid(d_out * d_in), tile_grid(d_out, d_in));
}

hipError_t launch_compress(const float* delta, int64_t d_out, int64_t d_in, uint32_t* words,
                           uint32_t* tiled, float* alpha, double* partials, hipStream_t stream) {
  const int64_t n = d_out * d_in;
  const bool tiles = d_in % 128 == 0 && reinterpret_cast<uintptr_t>(words) % 16 == 0;
  const int grid = tiles ? tile_grid(d_out, d_in) : flat_grid(n);
  clear_stale_error();
  if (tiles)
    hipLaunchKernelGGL(compress_tiles<false>, dim3(grid), dim3(kTileWaves * 64), 0, stream, delta,
                       d_out, d_in, words, tiled, 1, partials);
  else if (n / 32 < (int64_t(1) << 32))
    hipLaunchKernelGGL(compress_pass1<true>, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const f32x4*>(delta), n / 4, words, tiled, d_in / 32,
                       partials);
  else
    hipLaunchKernelGGL(compress_pass1<false>, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const f32x4*>(delta), n / 4, words, tiled, d_in / 32,
                       partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_pass2, dim3(1), dim3(kPass2Threads), 0, stream, partials, grid,
                     (double)n, alpha);
  return hipGetLastError();
}

int64_t compress_rows_partials(int64_t d_out, int64_t d_in) {
  return d_out * ((d_in + kTileCols - 1) / kTileCols);
}

hipError_t launch_compress_rows(const float* delta, int64_t d_out, int64_t d_in, uint32_t* words,
                                uint32_t* tiled, float* alpha, double* partials,
                                hipStream_t stream) {
  const int grid = tile_grid(d_out, d_in);
  const int vec = d_in % 128 == 0 && reinterpret_cast<uintptr_t>(words) % 16 == 0;
  clear_stale_error();
  hipLaunchKernelGGL(compress_tiles<true>, dim3(grid), dim3(kTileWaves * 64), 0, stream, delta,
                     d_out, d_in, words, tiled, vec, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = (d_out + kRowsPass2Threads - 1) / kRowsPass2Threads;
  hipLaunchKernelGGL(compress_rows_pass2, dim3((unsigned)blocks), dim3(kRowsPass2Threads), 0,
                     stream, partials, d_out, (d_in + kTileCols - 1) / kTileCols, (double)d_in,
                     alpha);
  return hipGetLastError();
}

hipError_t launch_compress_pair(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                                int64_t d_in, uint32_t* words, uint32_t* tiled, float* alpha,
                                double* partials, hipStream_t stream) {
  const int grid = tile_grid(d_out, d_in);
  const int vec = d_in % 128 == 0 && reinterpret_cast<uintptr_t>(words) % 16 == 0;
  clear_stale_error();
  hipLaunchKernelGGL(compress_pair_tiles, dim3(grid), dim3(kTileWaves * 64), 0, stream, w_ft,
                     w_base, d_out, d_in, words, tiled, vec, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_pass2, dim3(1), dim3(kPass2Threads), 0, stream, partials, grid,
                     (double)d_out * (double)d_in, alpha);
  return hipGetLastError();
}

}  // namespace bd
