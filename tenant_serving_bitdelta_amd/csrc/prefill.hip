// Prefill-sized batches: the fused reconstruct-and-multiply of the BitDelta post ("Serving
// architecture": reconstruction in fast on-chip memory, fused with the matmul, W_eff never
// written to HBM) as a dense bf16 MFMA contraction per segment.
//
// A workgroup (8 waves, two per SIMD) computes a tile of 256 tokens (one segment, hence one
// variant) by 256 output rows, walking d_in in steps of 32 taken in pairs.  Wave w owns rows
// 32w .. 32w + 31 for all 256 tokens (2 row tiles x 16 token tiles of fp32 accumulators).
// Two kinds of work per step:
//   * rebuild: the wave reads its raw weights from LDS and turns them into the bf16 operand
//         W_eff = bf16(fp32(w) + (bit ? +alpha : -alpha))   (round to nearest even),
//     with the sign words (one 16-byte load per row per 4 steps) in registers one quad ahead,
//     so each weight is rebuilt once, by the wave that multiplies it;
//   * multiply: v_mfma_f32_16x16x32_bf16 over the 2 x 16 tiles, the activation operand read
//     from LDS a few token tiles ahead.
// The two waves that share a SIMD (w and w + 4) take turns, in four phases per pair separated
// by barriers: while one multiplies, the other rebuilds and issues the copies, so that no copy
// sits in the instruction stream of a multiplying wave.
//
// Data: the activations of a pair (256 x 64) go from memory straight into LDS (direct
// global->LDS loads of whole 128-byte rows, 16 bytes per lane) into a ring of 3 pair slots,
// two pairs ahead, copied by waves 4..7; each wave copies its own weight rows (32 x 64) into a
// ring of 2 slots, two pairs ahead, over the slot it has just finished reading.  16-byte units
// are XOR-swizzled by row so the operand reads are conflict-free.  Rounding W_eff to bf16
// before the product is the one departure from an exact W_eff; the error it adds is below half
// a bf16 ulp of each weight and shows in y far inside the output tolerance.
//
// Tile order: workgroup b runs on XCD b % 8.  Each XCD takes groups of 32 tiles, 4 M tiles by 8
// N tiles, so the workgroups running side by side on it share 4 activation blocks and 8 weight
// blocks in its L2; the 8 XCDs take neighbouring groups (the same N tiles, other M tiles), so
// weight blocks also meet in the memory-side cache.
#include <type_traits>

#include "bd_internal.h"

namespace bd {

namespace {

constexpr int kThreads = 512;
constexpr int kBK = 32;                            // K per step
constexpr unsigned kXPair = kPrefillBM * 2 * kBK * 2;   // 32 KiB of activations per pair
constexpr unsigned kWPair = kPrefillBN * 2 * kBK * 2;   // 32 KiB of W_base per pair
constexpr unsigned kWBase = 3 * kXPair;                 // activations: 3 pair slots
constexpr unsigned kLds = kWBase + 2 * kWPair;          // weights: 2 pair slots
static_assert(kLds <= 160 * 1024, "the ring must fit in one compute unit's LDS");
constexpr int kGroupM = 4, kGroupN = 8;            // tiles per XCD group
constexpr int kBDepth = 4;                         // activation reads in flight per multiply

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

// s_waitcnt lgkmcnt(0) (the wave's LDS reads returned), leaving the other counters alone
#define LDS_DRAIN() __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14))
// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding, n <= 63).
#define PREFILL_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Byte offset of row t's 16-byte unit u in a pair block (units 4 h + c: chunk c of step h of the
// pair, 8 bf16 each): each row's 128 bytes are contiguous, with the units XOR-swizzled by
// (t / 2) % 8 so that 16 consecutive rows reading the same unit hit 16 different banks
// (measured conflict-free; unswizzled rows cost 12 conflict cycles per read).
__device__ __forceinline__ unsigned unit_off(int t, int u) {
  return (unsigned)(8 * t + (u ^ ((t >> 1) & 7))) * 16u;
}

// bit 31 of s, bits 0..30 of m (one v_bfi_b32)
__device__ __forceinline__ unsigned sign_into(unsigned s, unsigned m) {
  unsigned r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0x80000000u), "v"(s), "v"(m));
  return r;
}

// 8 bf16 weights (k = pos0 .. pos0+7 of word) -> 8 bf16 of w + (+-alpha).  A bf16 widens to
// fp32 exactly (a shift or a mask), so one fp32 addition gives fp32(w + (+-alpha)) rounded once,
// then rounded to bf16 (nearest even).  nword = ~word: bit k clear gives the sign bit of -alpha.
// (Plain fp32 adds rather than bf16 dot products: the kernel measured 12% slower on those.)
__device__ __forceinline__ u32x4 rebuild8(const u32x4& w, unsigned nword, unsigned pos0,
                                          unsigned abits) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // through a scalar: a bit cast of the vector element itself reads element 0
    const unsigned wd = w[d];
    const unsigned k0 = pos0 + 2 * d;
    const float a0 = __uint_as_float(sign_into(nword << (31u - k0), abits));
    const float a1 = __uint_as_float(sign_into(nword << (30u - k0), abits));
    f32x2 f;
    f[0] = __uint_as_float(wd << 16) + a0;
    f[1] = __uint_as_float(wd & 0xFFFF0000u) + a1;
    r[d] = __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
  }
  return r;
}

// kVec: every slot's sign words (and the base-model tiles' stand-in) are read 16 bytes, one
// quad of steps, at a time; otherwise one word at a time
template <bool kVec>
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

  const rsrc_t xrs = make_rsrc(a.x + (size_t)xrow0 * d_in);
  const rsrc_t wrs = make_rsrc(a.w + (size_t)n0 * d_in);
  // ---- copies (past the end: clamped).  Activations: the second wave of each SIMD (w >= 4) moves
  // tokens 64 (w - 4) .. + 63, copy i (0..7) taking 8 of them; weights: each wave moves its own
  // rows 32w .. 32w + 31, copy i (0..3) taking 8.  A copy moves 8 rows of 128 bytes: lane L
  // fills stored unit L % 8 of row r0 + L / 8, i.e. unit (L % 8) ^ ((row / 2) % 8) of that row.
  auto copy_x = [&](int p, int i) {
    const int r = 64 * (wave & 3) + 8 * i + (lane >> 3);
    const int u = (lane & 7) ^ ((r >> 1) & 7);
    const int sc = min(2 * p + (u >> 2), nsteps - 1);  // the step of this lane's unit
    dma16(xrs, (unsigned)((min(r, nrows - 1) * d_in + sc * kBK + 8 * (u & 3)) * 2),
          smem + (unsigned)(p % 3) * kXPair + (unsigned)(64 * (wave & 3) + 8 * i) * 128u);
  };
  auto copy_w = [&](int p, int i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int u = (lane & 7) ^ ((r >> 1) & 7);
    const int sc = min(2 * p + (u >> 2), nsteps - 1);
    dma16(wrs, (unsigned)(((min(n0 + r, d_out - 1) - n0) * d_in + sc * kBK + 8 * (u & 3)) * 2),
          smem + kWBase + (unsigned)(p & 1) * kWPair + (unsigned)(32 * wave + 8 * i) * 128u);
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
  // kVec: 16-byte quads of words; base-model tiles then read (and ignore) W_base bytes
  const unsigned quad_bytes = tiled ? 2048u : 16u;  // bytes between the words of two quads
  auto load_s = [&](u32x4* sw, int q0, int rt) {  // the quad starting at step q0 (clamped)
    if constexpr (kVec) {
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
  const unsigned a_lane[2] = {kWBase + unit_off(32 * wave + j, g),
                              kWBase + unit_off(32 * wave + j, 4 + g)};  // + W slot + rt * 16 * 128

  u32x4 af[2];  // the wave's two weight fragments for its next multiply
  // fragments of step s from its raw weights (LDS slot of pair s / 2) and the quad's words sw
  auto rebuild = [&](int s, const u32x4* sw) {
    const unsigned char* pb = smem + (unsigned)((s >> 1) & 1) * kWPair;
    const int h = s & 1;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(pb + a_lane[h]);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(pb + a_lane[h] + 16 * 128);
    af[0] = rebuild8(w0, ~sw[0][s & 3], 8u * g, abits[0]);
    af[1] = rebuild8(w1, ~sw[1][s & 3], 8u * g, abits[1]);
  };
  // the fragments times the 16 token tiles of step s
  auto multiply = [&](int s) {
    const unsigned char* pb = smem + (unsigned)((s >> 1) % 3) * kXPair + b_lane[s & 1];
    // kBDepth operand reads in flight ahead of the matrix instructions: this wave is the only
    // one of its SIMD issuing them, so nothing else hides the LDS latency
    u32x4 bq[kBDepth];
#pragma unroll
    for (int i = 0; i < kBDepth; ++i) bq[i] = *reinterpret_cast<const u32x4*>(pb + i * 16 * 128);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const u32x4 B = bq[tt % kBDepth];
      if (tt + kBDepth < 16)
        bq[tt % kBDepth] = *reinterpret_cast<const u32x4*>(pb + (tt + kBDepth) * 16 * 128);
      acc[0][tt] = mfma(af[0], B, acc[0][tt]);
      acc[1][tt] = mfma(af[1], B, acc[1][tt]);
    }
    // keep the order (the scheduler would otherwise sink the reads to their uses): kBDepth
    // reads, then 2 matrix instructions per further read
    __builtin_amdgcn_sched_group_barrier(0x100, kBDepth, 0);
#pragma unroll
    for (int i = 0; i < 16 - kBDepth; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kBDepth, 0);
  };
  // a barrier that only keeps the two roles in step (no memory ordering is needed at it)
  auto phase = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // a barrier after which pair p + 1's activations, waited for by every wave, are visible
  // (the weights are per wave: each rebuilds from rows it copied itself)
  auto pair_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Pair p (steps s0 = 2p, s1 = 2p + 1) in four phases:
  //            leading wave (w < 4)                 other wave (w >= 4)
  //   1   multiply s0                            rebuild s0, pair p + 2's activations
  //   2   rebuild s1, pair p + 2's weights       multiply s0
  //   3   multiply s1                            rebuild s1, pair p + 2's weights
  //   4   rebuild s0 of pair p + 1               multiply s1
  // so that no copy sits in the instruction stream of a multiplying wave.  Activations sit in
  // 3 slots, copied two pairs ahead; weights in 2, each wave copying pair p + 2's rows over pair
  // p's once it has read them (its LDS reads drained first).  Memory operations complete in
  // issue order.  Leading wave: before its phase-4 rebuild (pair p + 1's weights, issued the
  // pair before) at most the next quad's 2 sign loads and this pair's 4 weight copies are
  // newer.  Other wave: before its phase-1 rebuild (pair p's weights) at most 12 newer
  // operations (the next pair's 8 activation and 4 weight copies; sign loads make the wait
  // only longer); at the end of the pair pair p + 1's activations, after which come at most 4
  // weight copies, 2 sign loads, 8 activation copies and 4 weight copies: wait for 16 (pair
  // p + 1's activations are then in place, from every wave after the barrier).
  // sw: words of s0 and s1; swn: words of 2p + 2.
  auto pair = [&](auto role, int p, const u32x4* sw, const u32x4* swn) {
    constexpr bool kLead = decltype(role)::value;
    const int s0 = 2 * p, s1 = 2 * p + 1;
    const bool has1 = s1 < nsteps, more = s1 + 1 < nsteps;
    if constexpr (kLead) {
      multiply(s0);
    } else {
      PREFILL_VMCNT(12);
      rebuild(s0, sw);
#pragma unroll
      for (int i = 0; i < 8; ++i) copy_x(p + 2, i);
    }
    phase();
    if constexpr (kLead) {
      if (has1) rebuild(s1, sw);
      LDS_DRAIN();
#pragma unroll
      for (int i = 0; i < 4; ++i) copy_w(p + 2, i);
    } else {
      multiply(s0);
    }
    phase();
    if constexpr (kLead) {
      if (has1) multiply(s1);
    } else {
      if (has1) rebuild(s1, sw);
      LDS_DRAIN();
#pragma unroll
      for (int i = 0; i < 4; ++i) copy_w(p + 2, i);
    }
    phase();
    if constexpr (kLead) {
      if (more) {
        PREFILL_VMCNT(4);
        rebuild(s1 + 1, swn);
      }
    } else {
      if (has1) multiply(s1);
      PREFILL_VMCNT(16);
    }
    pair_barrier();
  };
  // A quad (two pairs) with the sign words cur; the next quad's words go into nxt during the
  // first pair (the second pair's phase 4 rebuilds from them).
  auto quad = [&](auto role, const u32x4* cur, u32x4* nxt, int q0) {
    load_s(nxt, q0 + 4, 0);
    load_s(nxt, q0 + 4, 1);
    pair(role, q0 >> 1, cur, cur);
    if (q0 + 2 < nsteps) pair(role, (q0 >> 1) + 1, cur, nxt);
  };
  auto run = [&](auto role, u32x4* sa, u32x4* sb) {
    int q0 = 0;
    for (; q0 + 4 < nsteps; q0 += 8) {
      quad(role, sa, sb, q0);
      quad(role, sb, sa, q0 + 4);
    }
    if (q0 < nsteps) quad(role, sa, sb, q0);
  };

  // ---- prologue: the sign words of quad 0, pairs 0 and 1's activations and weights ------
  u32x4 sa[2], sb[2];
  load_s(sa, 0, 0);
  load_s(sa, 0, 1);
  if (wave >= 4) {
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_x(0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) copy_x(1, i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) copy_w(0, i);
#pragma unroll
  for (int i = 0; i < 4; ++i) copy_w(1, i);
  PREFILL_VMCNT(4);
  pair_barrier();
  // waves w and w + 4 share a SIMD (as the hardware places the 8 waves of a workgroup; another
  // placement would only cost speed): w leads, i.e. multiplies first
  if (wave < 4) {
    rebuild(0, sa);
    run(std::true_type{}, sa, sb);
  } else {
    run(std::false_type{}, sa, sb);
  }
  PREFILL_VMCNT(0);

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
  // 16-byte sign quads when every slot of the launch (and the base-model tiles) allows them
  const bool vec = a.vec_signs == -1;
  const void* fn = vec ? reinterpret_cast<const void*>(&prefill_kernel<true>)
                       : reinterpret_cast<const void*>(&prefill_kernel<false>);
  static DeviceOnce once[2];
  hipError_t e = set_dynamic_lds_once(once[vec ? 1 : 0], fn, (int)kLds);
  if (e != hipSuccess) return e;
  // grid: 8 XCD lists of whole 32-tile groups
  const int ngroups = ((a.n_mtiles + kGroupM - 1) / kGroupM) * ((a.n_ntiles + kGroupN - 1) / kGroupN);
  const int nblocks = ((ngroups + 7) / 8) * 8 * kGroupM * kGroupN;
  clear_stale_error();
  if (vec)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(nblocks), dim3(kThreads), kLds, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(nblocks), dim3(kThreads), kLds, stream, a);
  return hipGetLastError();
}

}  // namespace bd
