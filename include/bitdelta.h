/*
 * bitdelta.h — C ABI of the MI355X (gfx950) BitDelta hot path.
 *
 * Method: the hanzo blog post "BitDelta: serving 14 Zen models from one GPU cluster"
 * (2026-02-28; "the BitDelta post" below).  A fine-tuned variant of a base model is stored per
 * weight matrix as one float32 scale alpha = mean|Delta| and one sign bit per element
 * ("The mathematical foundation"); at serving time each token's output is
 * y = x * (W_base + alpha_v * sign(Delta_v))^T for the variant v the token's request names,
 * computed without ever writing W_base + alpha_v * sign(Delta_v) to memory ("Serving
 * architecture": reconstruction fused with the multiply).
 *
 * Conventions shared by every entry point
 *   - Pointers marked [dev] are device (HBM) pointers; [host] are host pointers.
 *   - The caller owns every buffer.  The library never allocates device memory, keeps no
 *     state between calls, and is safe to call from several host threads.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *     A call returns as soon as its kernels are enqueued.
 *   - Argument errors are detected on the host BEFORE anything is enqueued and are reported
 *     as a status; no device memory is touched in that case.  Launch failures report
 *     BITDELTA_ERR_HIP.
 *   - Sign bits: element (r, k) of a d_out x d_in matrix is bit (k % 32) of the uint32 word
 *     r * (d_in / 32) + k / 32, least-significant bit first; bit 1 means +1, bit 0 means -1.
 *     The byte image of these words equals the BitDelta post's packing of eight sign bits per
 *     int8 ("Infrastructure details", delta storage format).  sign(+0) = sign(-0) = +1.
 *   - Tiled sign words (the layout the matmul kernels stream; needs d_in % 128 == 0): rows are
 *     grouped in blocks of 128 and columns in steps of 128; the 4 words of one row and one step
 *     sit at word ((r / 128) * (d_in / 128) + c / 4) * 512 + (r % 128) * 4 + c % 4 for
 *     row-major word (r, c), so each (block, step) is one contiguous 2 KiB chunk.  The last
 *     block is padded to 128 rows; padding words are never read for output rows < d_out.
 *     A variant needs its bits resident in ONE layout: the tiled one whenever d_in % 128 == 0
 *     (every kernel family reads it), the row-major one otherwise.  The row-major form is the
 *     storage and upload format; bitdelta_upload_variant converts it on the way in.
 *   - bf16 tensors are passed as `const void*` holding IEEE bfloat16 values, row-major.
 *   - d_in must be a multiple of 32 (one word per 32 elements of a row).
 */
#ifndef BITDELTA_H_
#define BITDELTA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITDELTA_ABI_VERSION 7
#define BITDELTA_MAX_VARIANTS 64   /* variant ids 0..63 per matmul call                      */
#define BITDELTA_MAX_SEGMENTS 65   /* base (-1) plus every variant                            */
#define BITDELTA_MAX_PROBLEMS 8    /* linears per grouped matmul call                         */

typedef enum {
  BITDELTA_OK = 0,
  BITDELTA_ERR_INVALID_ARG = 1, /* null pointer, negative size, unknown enum value            */
  BITDELTA_ERR_SHAPE = 2,       /* d_in not a multiple of 32, inconsistent segments           */
  BITDELTA_ERR_ALIGNMENT = 3,   /* a tensor pointer is not 16-byte aligned (words: 4-byte)    */
  BITDELTA_ERR_WORKSPACE = 4,   /* workspace smaller than the matching *_workspace_bytes query */
  BITDELTA_ERR_UNSUPPORTED = 5, /* a size beyond what the kernels handle                      */
  BITDELTA_ERR_HIP = 6          /* the HIP runtime reported an error while enqueueing         */
} bitdelta_status;

typedef void* bitdelta_stream; /* hipStream_t */
typedef void* bitdelta_event;  /* hipEvent_t */

typedef enum { BITDELTA_OUT_BF16 = 0, BITDELTA_OUT_F32 = 1 } bitdelta_out_dtype;

/* Which kernel family runs a matmul.  AUTO picks by batch shape; the others force one (for
 * tests and measurement).  Every path computes the same y within the documented tolerance. */
typedef enum {
  BITDELTA_PATH_AUTO = 0,
  BITDELTA_PATH_GEMV = 1,    /* fp32 reconstruction in registers, VALU; M <= 4                 */
  BITDELTA_PATH_STREAM = 2,  /* decode: base and sign sums both as bf16 MFMA; no workspace;
                              * d_in % 128 == 0                                               */
  BITDELTA_PATH_PREFILL = 3, /* prefill: per-segment tiles, bf16 W_eff rebuilt in registers   */
  BITDELTA_PATH_SPLIT = 4    /* decode: base sum bf16 MFMA, sign sum fp4 x fp6 MFMA on a
                              * two-term fp6 split of alpha * x (per-32-column power-of-two
                              * scales; for a per-row-alpha variant of x, with each step's
                              * sums times alpha_r in fp32); needs workspace and tiled sign
                              * words                                                        */
} bitdelta_path;

/* One compressed variant of one weight matrix: the output of bitdelta_compress.  At least one of
 * the two word pointers is set; when both are, they hold the same bits and the kernels read the
 * tiled one.  (ABI 7: either may be NULL.) */
typedef struct {
  const uint32_t* sign_words;      /* [dev] d_out * d_in / 32 words, row-major, 4-byte aligned
                                    * (16-byte aligned for the STREAM path), or NULL           */
  const uint32_t* sign_words_t128; /* [dev] the tiled layout above, 16-byte aligned (d_in % 128
                                    * == 0, else SHAPE), or NULL; needed by the SPLIT path     */
  const float* alpha;              /* [dev] the scale: one float32, or d_out (alpha_per_row)   */
  int32_t alpha_per_row;           /* 0: one scale per matrix (bitdelta_compress); 1: one per
                                    * output row, alpha[r] for row r (bitdelta_compress_rows);
                                    * other values: INVALID_ARG.  ABI 5.                      */
} bitdelta_variant;

/* One linear layer of a grouped matmul: every problem of a call sees the same token batch
 * segmentation (same M, same segments), with its own activations, weights and variants. */
typedef struct {
  const void* x;                    /* [dev] bf16 [M][d_in], rows in segment order, 16B-aligned */
  const void* w_base;               /* [dev] bf16 [d_out][d_in], 16-byte aligned                */
  void* y;                          /* [dev] [M][d_out] bf16 or f32 (y_dtype), 16-byte aligned  */
  int64_t d_out;
  int64_t d_in;                     /* multiple of 32                                           */
  const bitdelta_variant* variants; /* [host] num_variants entries (may be NULL if 0)           */
  int32_t num_variants;
} bitdelta_problem;

/* ABI version of the loaded library (BITDELTA_ABI_VERSION). */
int bitdelta_abi_version(void);

/* Static string naming a status code. */
const char* bitdelta_status_string(int status);

/* The hipError_t code behind the most recent BITDELTA_ERR_HIP returned on the calling thread
 * (0 if there was none), and the HIP runtime's static string for it. */
int32_t bitdelta_last_hip_error(void);
const char* bitdelta_last_hip_error_string(void);

/* Number of uint32 sign words of a d_out x d_in matrix (d_out * d_in / 32), or -1 if d_in is
 * not a positive multiple of 32 or d_out is negative. */
int64_t bitdelta_sign_words(int64_t d_out, int64_t d_in);

/* Number of uint32 words of the tiled sign copy of a d_out x d_in matrix
 * (ceil(d_out / 128) * 128 * d_in / 32), or -1 if d_in is not a positive multiple of 128. */
int64_t bitdelta_sign_words_t128(int64_t d_out, int64_t d_in);

/* Device workspace bytes bitdelta_compress needs for this shape (fp64 partial sums). */
size_t bitdelta_compress_workspace_bytes(int64_t d_out, int64_t d_in);

/*
 * bitdelta_compress — the compression step of the BitDelta post ("The mathematical
 * foundation"): alpha = ||Delta||_1 / n, the mean absolute value over all n = d_out * d_in
 * elements (exact zeros included), and sign(Delta) packed one bit per element.
 *
 *   delta       [dev] float32 [d_out][d_in], 16-byte aligned, finite values.  Read only.
 *   sign_words  [dev] out, optional when sign_words_t128 is given (NULL = not written):
 *               uint32 [d_out][d_in/32] (layout above), 4-byte aligned; with d_in % 128 == 0
 *               and 16-byte alignment the words are written as whole lines (the faster form),
 *               otherwise word by word.
 *   sign_words_t128 [dev] out, optional when sign_words is given (NULL = not written): the same
 *               bits in the tiled layout above, bitdelta_sign_words_t128 words, 16-byte
 *               aligned; needs d_in % 128 == 0 (else SHAPE).
 *   alpha       [dev] out: one float32, the sum of |Delta| (each 4 consecutive elements added
 *               in fp32, those sums in fp64, in a fixed order, so repeated calls are
 *               bit-identical) divided by n and rounded once to float32.
 *   workspace   [dev] at least bitdelta_compress_workspace_bytes(d_out, d_in) bytes,
 *               8-byte aligned; scratch only, contents on return unspecified.
 * Errors: INVALID_ARG (null pointer, both word pointers null, d_out <= 0), SHAPE (d_in not a
 * positive multiple of 32), ALIGNMENT, WORKSPACE (workspace_bytes too small), HIP.
 * The buffers must not overlap.
 */
bitdelta_status bitdelta_compress(const float* delta, int64_t d_out, int64_t d_in,
                                  uint32_t* sign_words, uint32_t* sign_words_t128, float* alpha,
                                  void* workspace, size_t workspace_bytes, bitdelta_stream stream);

/*
 * bitdelta_compress_from_weights — the same compression of the task vector of a bf16 weight pair,
 * Delta = W_ft - W_base (BitDelta post, "The mathematical foundation": the fine-tune's delta
 * from the base), without materialising Delta.  The sign of each element is that of the exact
 * difference (zero, i.e. equal weights, gives +1); alpha sums |Delta| formed in fp32 (exact
 * unless the two exponents are more than 16 apart, then rounded once), 4 consecutive elements
 * in fp32 and those sums in fp64 (weights below 4e37 in magnitude keep every sum finite).
 *
 *   w_ft, w_base [dev] bf16 [d_out][d_in], 16-byte aligned, finite values.  Read only.
 *   sign_words, sign_words_t128, alpha, workspace: as for bitdelta_compress (the same workspace
 *               size; the words are written as whole lines when 16-byte aligned and
 *               d_in % 128 == 0, else word by word).
 * Errors: as for bitdelta_compress.  The buffers must not overlap.
 * ABI 4.
 */
bitdelta_status bitdelta_compress_from_weights(const void* w_ft, const void* w_base, int64_t d_out,
                                               int64_t d_in, uint32_t* sign_words,
                                               uint32_t* sign_words_t128, float* alpha,
                                               void* workspace, size_t workspace_bytes,
                                               bitdelta_stream stream);

/* Device workspace bytes bitdelta_compress_rows needs for this shape (one fp64 partial sum per
 * row and 1024-column group), 0 for an invalid shape. */
size_t bitdelta_compress_rows_workspace_bytes(int64_t d_out, int64_t d_in);

/*
 * bitdelta_compress_rows — compression with one scale per output row, the other granularity the
 * post allows (BitDelta post, "Serving architecture": the conceptual fused kernel takes alpha of
 * shape [d_out] or a scalar; "Infrastructure details": alpha kept as float32, one per output
 * dimension): alpha[r] = the mean of |Delta| over the d_in elements of row r.  The sign bits are
 * those of bitdelta_compress.  Use the result with alpha_per_row = 1 in bitdelta_variant.
 *
 *   delta, sign_words, sign_words_t128: as for bitdelta_compress (any 4-byte-aligned word array;
 *               whole lines when 16-byte aligned and d_in % 128 == 0, else word by word).
 *   alpha       [dev] out: float32 [d_out], 4-byte aligned: row r's sum of |Delta| (4
 *               consecutive elements added in fp32, those sums in fp64, the row's 1024-column
 *               groups in column order, so repeated calls are bit-identical) divided by d_in and
 *               rounded once to float32.
 *   workspace   [dev] at least bitdelta_compress_rows_workspace_bytes(d_out, d_in) bytes,
 *               8-byte aligned; scratch only.
 * Errors: as for bitdelta_compress.  The buffers must not overlap.  ABI 5.
 */
bitdelta_status bitdelta_compress_rows(const float* delta, int64_t d_out, int64_t d_in,
                                       uint32_t* sign_words, uint32_t* sign_words_t128,
                                       float* alpha, void* workspace, size_t workspace_bytes,
                                       bitdelta_stream stream);

/*
 * bitdelta_plan_segments — group a token batch by variant (host only, O(M), no device work).
 * The BitDelta post's router sends each request to its variant while the base weights are one
 * shared read ("Serving architecture"); this groups tokens so one matmul call serves them all.
 * Stable counting sort by variant id: the base model (-1) first, then 0..num_variants-1;
 * empty groups are dropped.
 *
 *   token_variant [host] int32 [M], each in [-1, num_variants).
 *   perm          [host] out int32 [M]: sorted position p holds original token perm[p].
 *   seg_offsets   [host] out int32 [num_variants + 2]: segment s covers sorted positions
 *                 [seg_offsets[s], seg_offsets[s+1]); seg_offsets[0] = 0.
 *   seg_variant   [host] out int32 [num_variants + 1]: variant of segment s (-1 = base).
 *   num_segments  [host] out: number of non-empty segments.
 * Errors: INVALID_ARG (null pointer, M < 0, num_variants outside [0, BITDELTA_MAX_VARIANTS],
 * a variant id out of range; nothing is written then).  M = 0 yields zero segments.
 */
bitdelta_status bitdelta_plan_segments(const int32_t* token_variant, int64_t M,
                                       int32_t num_variants, int32_t* perm,
                                       int32_t* seg_offsets, int32_t* seg_variant,
                                       int32_t* num_segments);

/*
 * bitdelta_matmul_workspace_bytes — device workspace one linear (one problem) of a matmul call
 * on `path` needs, for a batch of M tokens and input width d_in (a multiple of 256 bytes; 0 when
 * the path needs none).  AUTO reports what the path AUTO would pick for M needs.  A grouped call
 * needs the sum over its problems.  The SPLIT path keeps there, per token (M rounded up to 16),
 * a bf16 copy of its activations in operand order (2 * d_in bytes), the two fp6 terms of
 * alpha * x (1.5 * d_in bytes), one scale word per 32 columns (d_in / 8 bytes) and one fp32
 * correction sum per 128 columns (d_in / 32 bytes), each rounded up to 256 bytes, and, per
 * linear, 128 fp32 partial-sum slots of 128 rows (512 bytes per token each), 128 counters of
 * 8 bytes, which the launch uses when it splits a 128-row block's K range over several compute
 * units, and a 256-byte statistics block.  In a call's workspace the slots of all its linears
 * come first after the activation parts, then all counters, then all statistics blocks; the first
 * uint32 of the first statistics block counts the split K ranges whose pieces ran on more than
 * one XCD (the launch intends one XCD per row block; such a handoff is then made coherent with
 * a device-scope acquire).  The library only ever adds to that word.
 * M = 0 or invalid arguments give 0.
 */
size_t bitdelta_matmul_workspace_bytes(int64_t M, int64_t d_in, int32_t path);

/*
 * bitdelta_matmul — the fused reconstruct-and-multiply of the BitDelta post ("Serving
 * architecture", conceptual fused linear): for every token t in segment s with variant
 * v = seg_variant[s],
 *     y[t][r] = sum_k x[t][k] * (w_base[r][k] + alpha_v * sign_v[r][k])
 * and for v = -1 (the base model) y[t][r] = sum_k x[t][k] * w_base[r][k].
 * W_base is read once per call for the whole batch and each variant's bits once; the
 * reconstructed weight is never written to memory.  Accumulation is fp32.
 *
 *   x            [dev] bf16 [M][d_in], rows grouped by segment (see bitdelta_plan_segments).
 *   w_base       [dev] bf16 [d_out][d_in].
 *   variants     [host] array of num_variants compressed variants of this matrix.
 *   seg_offsets  [host] int32 [num_segments + 1], 0 = first <= ... <= last = M.
 *   seg_variant  [host] int32 [num_segments], each in [-1, num_variants).
 *   y            [dev] out [M][d_out], bf16 (round-to-nearest-even) or float32 per y_dtype.
 *   workspace    [dev] at least bitdelta_matmul_workspace_bytes(M, d_in, BITDELTA_PATH_AUTO)
 *                bytes, 256-byte aligned (may be NULL when that is 0); scratch owned by the
 *                caller, used by the kernels this call enqueues, contents afterwards unspecified.
 *                Calls in flight at the same time need separate workspaces.
 * M = 0 is a no-op (x, y and workspace may then be NULL).  Errors: INVALID_ARG, SHAPE,
 * ALIGNMENT, WORKSPACE, UNSUPPORTED, HIP.  y must not alias any input or the workspace.
 */
bitdelta_status bitdelta_matmul(const void* x, const void* w_base, int64_t M, int64_t d_out,
                                int64_t d_in, const bitdelta_variant* variants,
                                int32_t num_variants, const int32_t* seg_offsets,
                                const int32_t* seg_variant, int32_t num_segments, void* y,
                                int32_t y_dtype, void* workspace, size_t workspace_bytes,
                                bitdelta_stream stream);

/*
 * bitdelta_matmul_grouped — bitdelta_matmul over up to BITDELTA_MAX_PROBLEMS independent
 * linears that share one token segmentation (e.g. the seven linears of a decoder block for
 * one decode batch), enqueued as few launches as possible so small matrices share the GPU.
 * `path` selects the kernel family (bitdelta_path); AUTO picks by M (GEMV for M <= 4, SPLIT
 * for M <= 256, PREFILL above).  SPLIT needs d_in % 128 == 0 and the tiled sign words of every
 * variant the batch uses; STREAM needs d_in % 128 == 0 and, for a variant without the tiled
 * words, 16-byte aligned row-major words.  When
 * AUTO's choice does not apply it falls back SPLIT -> STREAM -> PREFILL; a forced path that does
 * not apply reports UNSUPPORTED.  `workspace` must hold the sum over the problems of
 * bitdelta_matmul_workspace_bytes(M, d_in_p, path), 256-byte aligned.
 * Errors as bitdelta_matmul, checked for every problem before anything is enqueued.
 */
bitdelta_status bitdelta_matmul_grouped(const bitdelta_problem* problems, int32_t num_problems,
                                        int64_t M, const int32_t* seg_offsets,
                                        const int32_t* seg_variant, int32_t num_segments,
                                        int32_t y_dtype, int32_t path, void* workspace,
                                        size_t workspace_bytes, bitdelta_stream stream);

/*
 * bitdelta_matmul_grouped_noalloc — bitdelta_matmul_grouped for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the SPLIT decode path (the one whose kernels use a workspace) with that workspace
 * in a scratch array the library holds, BITDELTA_NOALLOC_SCRATCH_BYTES per device, from the first
 * call on a device until the process ends.  It calls no allocation routine.  The caller passes
 * inputs and outputs as for bitdelta_matmul_grouped.
 *
 *   path  AUTO or SPLIT; a batch the SPLIT path does not serve (AUTO would pick GEMV or PREFILL
 *         for this M, a variant lacks the tiled words, d_in % 128 != 0)
 *         gives UNSUPPORTED: use bitdelta_matmul_grouped for those (they need no workspace).
 * Errors: as bitdelta_matmul_grouped, plus WORKSPACE when the batch needs more than
 * BITDELTA_NOALLOC_SCRATCH_BYTES (the sum over the problems of
 * bitdelta_matmul_workspace_bytes(M, d_in, BITDELTA_PATH_SPLIT)), checked before anything is
 * enqueued.  All calls on one device share its scratch: calls that overlap in time on one device
 * (on different streams, or from several threads) race and must not be made.  ABI 7.
 */
#define BITDELTA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
bitdelta_status bitdelta_matmul_grouped_noalloc(const bitdelta_problem* problems,
                                                int32_t num_problems, int64_t M,
                                                const int32_t* seg_offsets,
                                                const int32_t* seg_variant, int32_t num_segments,
                                                int32_t y_dtype, int32_t path,
                                                bitdelta_stream stream);

/* The kernel family bitdelta_matmul_grouped's AUTO picks for this batch shape (a bitdelta_path
 * value), or -1 for invalid segments.  Host only.  It sees the shape, not the variants: where it
 * answers SPLIT, a call whose variants lack the tiled sign words or d_in % 128 runs STREAM
 * instead (PREFILL when streaming does not apply either). */
int32_t bitdelta_auto_path(int64_t M, const int32_t* seg_offsets, const int32_t* seg_variant,
                           int32_t num_segments);

/*
 * bitdelta_reconstruct — the reconstruction of the BitDelta post written out to memory ("Serving
 * architecture": W_eff = W_base + alpha * sign(Delta), the step the fused kernels keep in
 * registers).  It exists for the unfused comparison: W_eff materialised in HBM, then a plain
 * product with it (bitdelta_matmul with the base-model segment, variant -1), against the fused
 * bitdelta_matmul.
 *     w_eff[r][k] = bf16_RNE(fp32(w_base[r][k]) + (bit ? +a : -a)),  a = alpha[0] or alpha[r]
 * with one fp32 addition, as the prefill kernel rebuilds its operands.
 *
 *   w_base   [dev] bf16 [d_out][d_in], 16-byte aligned.
 *   variant  [host] one compressed variant (either word layout; per-matrix or per-row alpha).
 *   w_eff    [dev] out: bf16 [d_out][d_in], 16-byte aligned, not overlapping the inputs.
 * Errors: INVALID_ARG (null pointer, d_out <= 0, both word pointers null), SHAPE (d_in not a
 * positive multiple of 32; tiled words with d_in % 128 != 0), ALIGNMENT, HIP.  ABI 7.
 */
bitdelta_status bitdelta_reconstruct(const void* w_base, int64_t d_out, int64_t d_in,
                                     const bitdelta_variant* variant, void* w_eff,
                                     bitdelta_stream stream);

/*
 * bitdelta_upload_variant — move one compressed matrix of a variant from host memory into the
 * device layout the kernels read (BitDelta post, "Infrastructure details": a variant's delta is
 * loaded into the GPU's delta cache on its first request; its storage format is the row-major
 * packing of eight sign bits per byte plus float32 scales).  Enqueued on `stream`: a host-to-
 * device copy of the row-major words, then (for the tiled layout) one pass that re-lays them
 * out, and a copy of the scales.  Host buffers in pinned memory (hipHostMalloc) make the copies
 * asynchronous; pageable ones are copied before the call returns.  Record an event on `stream`
 * after the call to learn when the variant is usable (see bitdelta_residency_load_enqueued).
 *
 *   host_words      [host] uint32 [d_out][d_in/32], row-major (the storage format).
 *   host_alpha      [host] alpha_count float32 (1, or d_out for per-row scales).
 *   sign_words      [dev] out, optional: the row-major words (4-byte aligned; 16-byte aligned
 *                   when the tiled layout is also written, which then reads from it).
 *   sign_words_t128 [dev] out, optional (d_in % 128 == 0): the tiled layout, 16-byte aligned.
 *                   At least one of the two is given.
 *   alpha           [dev] out: alpha_count float32, 4-byte aligned.
 *   staging         [dev] needed only when sign_words_t128 is given without sign_words: at least
 *                   d_out * d_in / 8 bytes, 16-byte aligned, scratch; it must not be reused
 *                   until the work this call enqueues has run (same stream: at once).
 * Errors: INVALID_ARG (null pointer, sizes <= 0, alpha_count not 1 or d_out, no destination),
 * SHAPE (d_in % 32, or d_in % 128 for the tiled layout), ALIGNMENT, WORKSPACE (staging missing
 * or too small), HIP.  ABI 7.
 */
bitdelta_status bitdelta_upload_variant(const uint32_t* host_words, const float* host_alpha,
                                        int64_t alpha_count, int64_t d_out, int64_t d_in,
                                        uint32_t* sign_words, uint32_t* sign_words_t128,
                                        float* alpha, void* staging, size_t staging_bytes,
                                        bitdelta_stream stream);

/* ---- Delta residency (host only, ABI 6; holds and events ABI 7) ---------------------------
 * Which variants' compressed deltas (sign words and alpha) stay in device memory, after the
 * BitDelta post, "Infrastructure details": the variants with the most requests stay pinned (the
 * top few by volume always resident), the rest share the remaining capacity with least-recently-
 * used eviction; a request for a variant that is not resident starts a load; requests for a
 * variant whose load is in flight wait for it rather than starting another.  Request rate is the
 * count of requests so far; pinned = the num_pinned highest counts (ties to the smaller id) among
 * variants requested at least once, the current request included.  Pinned and loading variants
 * are never evicted; nor are variants held by requests in flight (see `hold` below); eviction
 * takes the least recently requested evictable variant first (ties to the smaller id) until the
 * new delta fits.  The caller moves the bytes (bitdelta_upload_variant) and either calls
 * load_done or attaches the upload's completion event (load_enqueued) for poll to find.
 * Each call locks the manager, so calls from several threads are serialised. */
typedef struct bitdelta_residency bitdelta_residency;

enum {
  BITDELTA_RESIDENCY_HIT = 0,     /* resident: serve now                                      */
  BITDELTA_RESIDENCY_LOAD = 1,    /* start loading it (after dropping the evicted variants)   */
  BITDELTA_RESIDENCY_QUEUED = 2,  /* its load is in flight: wait for that load                 */
  BITDELTA_RESIDENCY_NO_ROOM = 3  /* cannot fit now (the rest is pinned or loading); nothing
                                   * changed but the request counts                           */
};
enum { BITDELTA_VARIANT_ABSENT = 0, BITDELTA_VARIANT_LOADING = 1, BITDELTA_VARIANT_RESIDENT = 2 };

/* num_variants in 1..4096; variant_bytes [host] num_variants sizes > 0 (copied); capacity_bytes
 * > 0; num_pinned >= 0.  *out receives the manager (NULL on error).  Errors: INVALID_ARG. */
bitdelta_status bitdelta_residency_create(int32_t num_variants, const int64_t* variant_bytes,
                                          int64_t capacity_bytes, int32_t num_pinned,
                                          bitdelta_residency** out);
void bitdelta_residency_destroy(bitdelta_residency* r);
/* One request for `variant`: *action = BITDELTA_RESIDENCY_*; evicted [host] room for
 * num_variants ids receives the variants dropped, in eviction order, *num_evicted their count
 * (their memory may be reused once the work that read them has drained).  hold = 1: an answer
 * HIT, LOAD or QUEUED also makes this request a holder of the variant, which is then never
 * evicted until every holder has called bitdelta_residency_release (so memory that queued
 * kernels still read is never handed to another upload, and the variants of one batch, requested
 * one by one, cannot evict each other); NO_ROOM holds nothing.  hold = 0: no hold.
 * Errors: INVALID_ARG (null pointer, variant out of range, hold not 0 or 1).  ABI 7 (hold). */
bitdelta_status bitdelta_residency_request(bitdelta_residency* r, int32_t variant, int32_t hold,
                                           int32_t* action, int32_t* evicted,
                                           int32_t* num_evicted);
/* Drop one hold of `variant` (after the streams that read it have finished the work of the
 * holding request).  INVALID_ARG if it has no holder.  ABI 7. */
bitdelta_status bitdelta_residency_release(bitdelta_residency* r, int32_t variant);
/* Current number of holders of `variant`, or -1 for a bad argument.  ABI 7. */
int64_t bitdelta_residency_holds(bitdelta_residency* r, int32_t variant);
/* Attach the event recorded after `variant`'s upload (on the upload's stream) to its load:
 * bitdelta_residency_poll then makes the variant resident once the event has completed.  The
 * manager does not own the event; keep it alive until poll has reported the variant (or until
 * load_done).  INVALID_ARG unless the variant is loading.  ABI 7. */
bitdelta_status bitdelta_residency_load_enqueued(bitdelta_residency* r, int32_t variant,
                                                 bitdelta_event event);
/* Query the events of loading variants; each whose upload has completed becomes resident and is
 * listed in completed [host, room for num_variants ids] (*num_completed of them): the requests
 * that were answered QUEUED for it may go ahead.  Never waits.  HIP if an event query fails.
 * ABI 7. */
bitdelta_status bitdelta_residency_poll(bitdelta_residency* r, int32_t* completed,
                                        int32_t* num_completed);
/* The load of `variant` has finished: it becomes resident.  INVALID_ARG unless it was loading. */
bitdelta_status bitdelta_residency_load_done(bitdelta_residency* r, int32_t variant);
/* BITDELTA_VARIANT_* of `variant`, or -1 for a bad argument. */
int32_t bitdelta_residency_state(bitdelta_residency* r, int32_t variant);
/* Bytes held by resident and loading variants, or -1 for a null manager. */
int64_t bitdelta_residency_used_bytes(bitdelta_residency* r);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_H_ */
