// Multi-variant decode: the fused reconstruct-and-multiply of the BitDelta post ("Serving
// architecture") for a token batch grouped by variant, with W_base read from HBM once for the
// whole batch and each active variant's sign bits read once.
//
// For a token t of variant v and output row r,
//     y[t][r] = sum_k x[t][k] * w[r][k]  +  alpha_v * sum_k x[t][k] * s_v[r][k],   s = +-1,
// which is x * (W_base + alpha_v * sign_v)^T with the product split in two: the base part and
// the sign part are both exact bf16 x bf16 products accumulated in fp32 by MFMA, and alpha_v is
// applied once in fp32 at the end.  W_eff is never formed in memory.
//
// Work split.  A workgroup (8 waves, two per SIMD) owns 64 output rows of one linear; the
// batch is cut into 16-token tiles that never straddle a segment (one variant per tile), and
// wave w owns tiles [w*NTW, w*NTW+NTW).  For each of its tiles and each of the 4 row tiles it
// keeps two 16x16 fp32 accumulators (base and sign).  The K loop walks d_in in steps of 64 (two
// 32-wide chunks of v_mfma_f32_16x16x32_bf16):
//   * a wave loads its own tiles' activations straight from global memory into B-operand
//     registers (16 bytes per lane, one step ahead): activations are never staged in LDS, and no
//     wave reads another wave's tokens;
//   * the 64x64 block of W_base and the sign words of every active variant for the 64 rows
//     (16 bytes = 4 steps per row and variant at a time) are loaded two steps ahead into
//     registers and committed to double-buffered LDS, where all 8 waves read them; one
//     workgroup barrier per step, which does not wait for outstanding global loads;
//   * per chunk, tile and row tile the variant's 32-bit sign word of each row is expanded in
//     registers into a bf16 +-1 A operand: a byte permute puts the lane's 8 bits in both 16-bit
//     halves, a packed 16-bit shift moves bit pair (2d, 2d+1) to the two bf16 sign positions,
//     and one 3-input bit operation merges them with the constant 1.0 (2 VALU ops per 2
//     weights); consecutive tiles of the same variant reuse the expansion;
//   * acc_base += W * X_tile and acc_sign += S_v * X_tile.
// Epilogue: y = acc_base + alpha_v * acc_sign, rounded to bf16 (nearest-even) or stored fp32.
#include <type_traits>

#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kKS = 64;                     // k per step
constexpr int kRows = kStreamRowsPerBlock;  // 64 output rows per workgroup
constexpr int kRT = kRows / 16;             // row tiles
constexpr int kRowBytes = kKS * 2;          // bytes of one staged 64-wide bf16 row
constexpr int kBitsRowBytes = 32;           // 8 sign words (4 steps) per row and variant
constexpr unsigned kWBytes = kRows * kRowBytes;

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Expand the 8 sign bits k = 8g..8g+7 (byte g of `word`) into 8 bf16 of +-1.0, in the order the
// A operand holds them (dword d = elements 8g+2d (low half) and 8g+2d+1 (high half)).
__device__ __forceinline__ u32x4 expand_signs(unsigned word, unsigned byte_sel) {
  const unsigned t = __builtin_amdgcn_perm(0u, word, byte_sel);  // [b, 0, b, 0]
  const u16x2 tv = __builtin_bit_cast(u16x2, t);
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u16x2 sh = {(unsigned short)(15 - 2 * d), (unsigned short)(14 - 2 * d)};
    const unsigned m = __builtin_bit_cast(unsigned, (u16x2)(tv << sh));
    r[d] = 0x3F803F80u | (~m & 0x80008000u);  // bit 1 -> +1.0, bit 0 -> -1.0
  }
  return r;
}

// Workgroup barrier ordering LDS traffic only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename T>
__device__ __forceinline__ T* lds_at(unsigned char* base, unsigned off) {
  return reinterpret_cast<T*>(base + off);
}

// NTW: token tiles per wave (the batch has at most 8*NTW tiles).
template <int NTW>
__global__ __launch_bounds__(kThreads, 1) void stream_kernel(const StreamArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // ---- which linear and which 64-row block (all wave-uniform) --------------------------------
  const int bid = blockIdx.x;
  int p = 0;
#pragma unroll
  for (int q = 1; q < kMaxProblems; ++q)
    if (q < a.nprob && bid >= a.prob[q].block_begin) p = q;
  const uint16_t* __restrict__ xg = a.prob[p].x;
  const uint16_t* __restrict__ wg = a.prob[p].w;
  const int d_in = a.prob[p].d_in, d_out = a.prob[p].d_out;
  const int row0 = (bid - a.prob[p].block_begin) * kRows;
  const int T = a.ntiles;   // 1..8*NTW
  const int NS = a.nslots;  // >= 1 (the host supplies a readable dummy when no variant is used)
  const int wpr = d_in >> 5;
  const int nsteps = d_in / kKS;  // even: d_in is a multiple of 128 on this path

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const unsigned byte_sel = (unsigned)g | 0x0C00u | ((unsigned)g << 16) | 0x0C000000u;

  const unsigned bs_bytes = (unsigned)NS * kRows * kBitsRowBytes;
  unsigned char* WS = smem;                 // [2][64 rows][128 B], 16-byte columns swizzled
  unsigned char* BS = smem + 2 * kWBytes;   // [2][NS][64 rows][32 B]

  // ---- this wave's tiles ------------------------------------------------------------------------
  int xoff[NTW];           // element offset of this lane's activation row (+ its 8-wide k group)
  unsigned tslot[NTW];     // byte offset of the tile's variant inside a sign-word buffer
  bool treal[NTW];         // tile exists (wave-uniform)
  bool tnew[NTW];          // tile's variant differs from the previous tile's (wave-uniform)
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int ti_raw = wave * NTW + i;
    const int ti = min(ti_raw, T - 1);
    const int valid = a.tile_valid[ti];
    xoff[i] = (a.tile_src[ti] + min(j, valid - 1)) * d_in + 8 * g;
    const int s = a.tile_slot[ti];
    tslot[i] = __builtin_amdgcn_readfirstlane((unsigned)((s < 0 ? 0 : s) * kRows * kBitsRowBytes));
    treal[i] = ti_raw < T;
    tnew[i] = i == 0 || a.tile_slot[min(ti_raw - 1, T - 1)] != s;
  }

  // ---- staging of W_base and sign words (all threads) ---------------------------------------
  const int wr_row = tid >> 3, wr_col = tid & 7;  // one 16-byte piece per thread per step
  const int wsrc = min(row0 + wr_row, d_out - 1) * d_in + (wr_col ^ (wr_row & 7)) * 8;
  const unsigned wdst = (unsigned)(wr_row * kRowBytes + wr_col * 16);
  // sign words: per 4-step group NS x 64 rows x 2 pieces of 16 B; at each step a thread moves
  // piece id = tid + 512 * (step % 4): slot id / 128 (wave-uniform), row (id / 2) % 64,
  // half id % 2.  Rows 8..15 of every 16 swap halves (bank spread on reads).
  const int brow = (tid >> 1) & 63, bhalf = tid & 1;
  const int bgrow = min(row0 + brow, d_out - 1);
  const unsigned bdst = (unsigned)(brow * kBitsRowBytes + ((bhalf ^ ((brow >> 3) & 1)) * 16));
  const int bslot_base = wave >> 1;

  // ---- per-lane LDS read offsets ----------------------------------------------------------------
  unsigned aoff[2];  // + rt * 16 * kRowBytes
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) aoff[cc] = (unsigned)(j * kRowBytes + (((cc * 4 + g) ^ (j & 7)) * 16));
  const unsigned bw_lane = (unsigned)(j * kBitsRowBytes);  // + rt * 16 * kBitsRowBytes
  const unsigned bw_swz = ((j >> 3) & 1) * 4;               // word-index xor of this lane's rows

  // ---- registers ----------------------------------------------------------------------------------
  u32x4 xv[2][NTW][2];  // [set][tile][chunk] activation B operands
  u32x4 wr[2];
  u32x4 br[2];

  auto load_x = [&](int ks, int set) {
    const int kc = min(ks, nsteps - 1) * kKS;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        xv[set][i][cc] = *reinterpret_cast<const u32x4*>(xg + xoff[i] + kc + cc * 32);
  };
  auto load_w = [&](int ks, int set) {
    const int kc = min(ks, nsteps - 1) * kKS;
    wr[set] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wg + wsrc + kc));
  };
  auto store_w = [&](int buf, int set) { *lds_at<u32x4>(WS, buf * kWBytes + wdst) = wr[set]; };
  // the sign-word piece moved at step `ks` belongs to group ks / 4 + 1, quarter ks % 4
  auto bits_slot = [&](int ks) { return min(bslot_base + 4 * (ks & 3), NS - 1); };
  auto load_bits = [&](int ks, int set) {
    const int grp = min((ks >> 2) + 1, (nsteps - 1) >> 2);
    const int widx = min(grp * 8 + bhalf * 4, wpr - 4);
    const int sl = bits_slot(ks);
    br[set] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        a.prob[p].words[sl] + sign_quad_offset((a.prob[p].tiled >> sl) & 1u, bgrow, widx >> 2, wpr)));
  };
  auto store_bits = [&](int ks, int set) {
    const int grp = (ks >> 2) + 1;
    *lds_at<u32x4>(BS, (grp & 1) * bs_bytes + bits_slot(ks) * kRows * kBitsRowBytes + bdst) =
        br[set];
  };

  f32x4 accb[NTW][kRT], accd[NTW][kRT];
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      accb[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accd[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // ---- prologue ------------------------------------------------------------------------------------
#pragma unroll
  for (int quarter = 0; quarter < 4; ++quarter) {  // sign-word group 0 straight into BS[0]
    const int slot = bits_slot(quarter);
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        a.prob[p].words[slot] + sign_quad_offset((a.prob[p].tiled >> slot) & 1u, bgrow,
                                                 min(bhalf * 4, wpr - 4) >> 2, wpr)));
    *lds_at<u32x4>(BS, slot * kRows * kBitsRowBytes + bdst) = v;
  }
  load_x(0, 0);
  load_x(1, 1);
  load_w(0, 0);
  store_w(0, 0);
  load_w(1, 1);
  load_w(2, 0);
  load_bits(0, 0);
  load_bits(1, 1);
  lds_barrier();

  // ---- main loop: two steps per iteration so each register set is fixed at compile time -------
  auto step = [&](int ks, auto set_c) {
    constexpr int set = decltype(set_c)::value;  // == ks & 1
    const unsigned wbuf = (unsigned)set * kWBytes;
    const unsigned bbuf = (unsigned)((ks >> 2) & 1) * bs_bytes;
    const int quarter = ks & 3;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 A[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        A[rt] = *lds_at<const u32x4>(WS, wbuf + aoff[cc] + rt * 16 * kRowBytes);
      const unsigned wsel = bbuf + bw_lane + (unsigned)((2 * quarter + cc) ^ bw_swz) * 4;
      u32x4 S[kRT];
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        if (!treal[i]) break;  // the wave's remaining tiles are past the batch
        if (tnew[i]) {
          unsigned word[kRT];
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt)
            word[rt] = *lds_at<const unsigned>(BS, wsel + tslot[i] + rt * 16 * kBitsRowBytes);
#pragma unroll
          for (int rt = 0; rt < kRT; ++rt) S[rt] = expand_signs(word[rt], byte_sel);
        }
        const u32x4 B = xv[set][i][cc];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          accb[i][rt] = mfma(A[rt], B, accb[i][rt]);
          accd[i][rt] = mfma(S[rt], B, accd[i][rt]);
        }
      }
    }
    // commit what the next step needs (loaded two steps ago) into the other buffers
    store_w(set ^ 1, set ^ 1);
    store_bits(ks, set);
    lds_barrier();
    // issue loads: activations for step ks+2 into the set just consumed, weights and sign
    // words two steps ahead of their commit
    load_x(ks + 2, set);
    load_w(ks + 3, set ^ 1);
    load_bits(ks + 2, set);
  };
  for (int ks = 0; ks < nsteps; ks += 2) {
    step(ks, std::integral_constant<int, 0>{});
    step(ks + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: lane holds rows 4g..4g+3 of each row tile for token j of each tile ----------
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int ti = wave * NTW + i;
    if (ti < T) {
      const int s = a.tile_slot[ti];
      const float* ap = s >= 0 ? a.prob[p].alpha[s] : nullptr;
      const bool per_row = s >= 0 && ((a.prob[p].alpha_rows >> s) & 1u);
      const float al = s >= 0 ? ap[0] : 0.f;
      if (j < (int)a.tile_valid[ti]) {
        const size_t ybase = (size_t)(a.tile_src[ti] + j) * d_out;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
          const int orow = row0 + rt * 16 + 4 * g;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = per_row ? ap[min(orow + r, d_out - 1)] : al;
            v[r] = accb[i][rt][r] + ar * accd[i][rt][r];
          }
          if (a.y_f32) {
            float* y = reinterpret_cast<float*>(a.prob[p].y) + ybase;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (orow + r < d_out) y[orow + r] = v[r];
          } else {
            uint16_t* y = reinterpret_cast<uint16_t*>(a.prob[p].y) + ybase;
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
}

template <int NTW>
hipError_t launch_ntw(const StreamArgs& a, int nblocks, hipStream_t stream) {
  const size_t lds = stream_lds_bytes(a.ntiles, a.nslots);
  static DeviceOnce once;
  hipError_t e = set_dynamic_lds_once(once, reinterpret_cast<const void*>(&stream_kernel<NTW>),
                                      160 * 1024);
  if (e != hipSuccess) return e;
  clear_stale_error();
  hipLaunchKernelGGL(stream_kernel<NTW>, dim3(nblocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

size_t stream_lds_bytes(int ntiles, int nslots) {
  (void)ntiles;
  return 2 * (size_t)kWBytes + 2 * (size_t)nslots * kRows * kBitsRowBytes;
}

hipError_t launch_stream(const StreamArgs& a, int nblocks, hipStream_t stream) {
  if (a.ntiles < 1 || a.ntiles > kStreamMaxTiles || a.nslots < 1 || a.nslots > kMaxSlots)
    return hipErrorInvalidValue;
  if (a.ntiles <= kWaves) return launch_ntw<1>(a, nblocks, stream);
  if (a.ntiles <= 2 * kWaves) return launch_ntw<2>(a, nblocks, stream);
  return launch_ntw<3>(a, nblocks, stream);
}

}  // namespace bd
