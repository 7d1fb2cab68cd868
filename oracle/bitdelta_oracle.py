"""Plain, slow, fp64 reference of the BitDelta hot path — TEST INFRASTRUCTURE ONLY.

Nothing in the product library may import or call this module; only tests, the smoke check
and the CPU-baseline leg of the benchmark do.  It shares no code with the HIP path.

What is computed, and where the BitDelta post ("BitDelta: serving 14 Zen models from one GPU
cluster", hanzo blog, 2026-02-28) defines it:

* compress — "The mathematical foundation": the 1-bit approximation W_ft ~ W_base + alpha*sign(Delta)
  (Delta = W_ft - W_base, also taken from a bf16 weight pair),
  the per-matrix scale alpha = ||Delta||_1 / n (the mean absolute delta over all n elements), and
  one bit per element for the sign.  "Infrastructure details" (delta storage format): sign
  matrices packed eight bits per byte along the input dimension; alpha kept as float32.
* reconstruct + multiply — "Serving architecture", the conceptual ``fused_bitdelta_linear``
  listing: unpack the bits to {-1,+1}, form W_eff = W_base + alpha*sign, return x @ W_eff^T.
* token batch segmented by variant — "Serving architecture" (each request names its variant;
  the base weights are one shared read for all variants).

Readings taken where the post is silent (each is listed in the design notes):

* alpha is one scalar per matrix (the formula averages over all n elements); the per-row form
  (``alpha_rows_ref``: the same mean taken over each output row) is offered beside it.
* alpha = float32 round-to-nearest-even of (exact sum of |Delta|) / n.  The sum is exact
  (``math.fsum``) up to ``FSUM_MAX`` elements and numpy's pairwise fp64 sum above that.
* sign(0) = +1, including -0.0; negative subnormals are negative.
* bit value 1 means +1, bit value 0 means -1; bits are packed least-significant-bit first along
  d_in into little-endian uint32 words, row-major by output row, d_in/32 words per row.  The
  byte image of those words is the post's int8 packing, eight bits per byte.
* variant id -1 selects the base model alone (W_eff = W_base).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants, special cases and brute force) — none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# Above this many elements the alpha sum uses numpy's pairwise fp64 summation (relative error
# <= ~log2(n) * 2^-53, far below the 1e-6 tolerance) instead of the exact math.fsum.  That branch
# is pinned separately, at n = 2^23, by closed forms whose fp64 partial sums are all exact.
FSUM_MAX = 1 << 22


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as their uint16 bit patterns (bf16 is the top half of
    an IEEE float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Compress  (BitDelta post, "The mathematical foundation"; "Infrastructure details")
# ----------------------------------------------------------------------------------------------

def alpha_ref(delta: np.ndarray) -> np.float32:
    """alpha = ||Delta||_1 / n: the mean of |Delta_ij| over every element of the matrix (exact
    zeros included), rounded once to float32 (the post stores alpha as float32)."""
    a = np.abs(np.asarray(delta, dtype=np.float64)).ravel()
    n = a.size
    if n == 0:
        raise ValueError("alpha of an empty matrix is undefined")
    total = math.fsum(a.tolist()) if n <= FSUM_MAX else float(np.sum(a, dtype=np.float64))
    return np.float32(total / n)


def alpha_rows_ref(delta: np.ndarray) -> np.ndarray:
    """Per-output-row scales, the other granularity the post allows (its conceptual fused kernel
    in "Serving architecture" takes alpha of shape [d_out] or a scalar; "Infrastructure details"
    stores one float32 per output dimension): alpha_r = mean over the d_in elements of row r of
    |Delta_rc|, the exact row sum divided by d_in and rounded once to float32."""
    a = np.abs(np.asarray(delta, dtype=np.float64))
    if a.ndim != 2 or a.shape[1] == 0:
        raise ValueError("alpha rows need a [d_out, d_in] matrix with d_in > 0")
    d_in = a.shape[1]
    return np.array([np.float32(math.fsum(row.tolist()) / d_in) for row in a], dtype=np.float32)


def signs_ref(delta: np.ndarray) -> np.ndarray:
    """sign(Delta) as int8 in {-1,+1}.  The post reduces each delta to "positive or negative";
    zero (either sign of zero) maps to +1 by convention; a value is negative only if it is
    strictly below zero."""
    d = np.asarray(delta)
    return np.where(d < 0, np.int8(-1), np.int8(1)).astype(np.int8)


def pack_signs_ref(signs: np.ndarray) -> np.ndarray:
    """Pack a {-1,+1} matrix [d_out, d_in] into uint32 words [d_out, d_in/32]: element (i, j)
    sits in word (i, j // 32) at bit (j % 32); bit 1 means +1."""
    s = np.asarray(signs)
    d_out, d_in = s.shape
    if d_in % 32:
        raise ValueError("d_in must be a multiple of 32")
    bits = (s > 0).astype(np.uint64).reshape(d_out, d_in // 32, 32)
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def unpack_signs_ref(words: np.ndarray, d_in: int) -> np.ndarray:
    """Inverse of ``pack_signs_ref``: uint32 words [d_out, d_in/32] -> int8 {-1,+1} [d_out, d_in]."""
    w = np.asarray(words, dtype=np.uint32)
    d_out = w.shape[0]
    if w.shape[1] * 32 != d_in:
        raise ValueError("word count does not match d_in")
    bit = (w[:, :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return (bit.astype(np.int8) * 2 - 1).reshape(d_out, d_in)


def compress_ref(delta: np.ndarray):
    """The compression step: (packed sign words, alpha)."""
    return pack_signs_ref(signs_ref(delta)), alpha_ref(delta)


def compress_rows_ref(delta: np.ndarray):
    """The compression step with per-output-row scales: (packed sign words, alpha [d_out])."""
    return pack_signs_ref(signs_ref(delta)), alpha_rows_ref(delta)


def task_vector_ref(w_ft_bits: np.ndarray, w_base_bits: np.ndarray) -> np.ndarray:
    """Delta = W_ft - W_base for bf16 weights given as uint16 bit patterns ("The mathematical
    foundation": the fine-tune's delta from the base).  Computed in fp64: exact whenever the two
    exponents differ by less than 45, otherwise correctly rounded; its sign is always exact and
    it is zero exactly when the two weights are equal."""
    return bf16_bits_to_f64(w_ft_bits) - bf16_bits_to_f64(w_base_bits)


def compress_from_weights_ref(w_ft_bits: np.ndarray, w_base_bits: np.ndarray):
    """The compression step applied to the task vector of a (fine-tuned, base) weight pair."""
    return compress_ref(task_vector_ref(w_ft_bits, w_base_bits))


def packed_nbytes_ref(d_out: int, d_in: int) -> int:
    """Bytes of one compressed matrix: one bit per element plus one float32 alpha."""
    return d_out * d_in // 8 + 4


# ----------------------------------------------------------------------------------------------
# Reconstruct + multiply  (BitDelta post, "Serving architecture", conceptual fused kernel)
# ----------------------------------------------------------------------------------------------

def reconstruct_ref(w_base: np.ndarray, words: np.ndarray, alpha) -> np.ndarray:
    """W_eff = W_base + alpha * sign(Delta) in fp64, with alpha the stored float32 value (one
    scalar, or one per output row: W_eff[r] = W_base[r] + alpha[r] * sign(Delta[r])) and the
    signs unpacked from the stored bits."""
    wb = np.asarray(w_base, dtype=np.float64)
    s = unpack_signs_ref(words, wb.shape[1]).astype(np.float64)
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64)
    if a.ndim == 1:
        if a.shape[0] != wb.shape[0]:
            raise ValueError("alpha rows must have one entry per output row")
        a = a[:, None]
    elif a.ndim != 0:
        raise ValueError("alpha is a scalar or a [d_out] vector")
    return wb + a * s


def fused_linear_ref(x: np.ndarray, w_base: np.ndarray, words: np.ndarray, alpha) -> np.ndarray:
    """One variant: y = x @ W_eff^T (the conceptual fused linear), exact fp64 product."""
    xf = np.asarray(x, dtype=np.float64)
    return xf @ reconstruct_ref(w_base, words, alpha).T


def plan_segments_ref(token_variant, num_variants: int):
    """Group a batch by variant: a stable sort of tokens by variant id, base (-1) first, then
    0..num_variants-1, empty groups dropped.  Returns (perm, seg_offsets, seg_variant) where
    sorted position p holds original token perm[p] and segment s covers sorted positions
    [seg_offsets[s], seg_offsets[s+1]) for variant seg_variant[s]."""
    ids = [int(v) for v in token_variant]
    for v in ids:
        if v < -1 or v >= num_variants:
            raise ValueError(f"variant id {v} out of range")
    perm, offsets, seg_var = [], [0], []
    for v in range(-1, num_variants):
        members = [t for t, tv in enumerate(ids) if tv == v]
        if members:
            perm.extend(members)
            offsets.append(len(perm))
            seg_var.append(v)
    return (np.asarray(perm, dtype=np.int32), np.asarray(offsets, dtype=np.int32),
            np.asarray(seg_var, dtype=np.int32))


def matmul_ref(x: np.ndarray, w_base: np.ndarray, variants, seg_offsets, seg_variant) -> np.ndarray:
    """Variant-segmented batch: rows of x are in segment order; segment s uses variant
    seg_variant[s] (its (words, alpha) pair in ``variants``) or the base model for -1.
    Returns y [M, d_out] in fp64."""
    xf = np.asarray(x, dtype=np.float64)
    wb = np.asarray(w_base, dtype=np.float64)
    y = np.zeros((xf.shape[0], wb.shape[0]), dtype=np.float64)
    for s in range(len(seg_variant)):
        lo, hi = int(seg_offsets[s]), int(seg_offsets[s + 1])
        if hi <= lo:
            continue
        v = int(seg_variant[s])
        w_eff = wb if v < 0 else reconstruct_ref(wb, variants[v][0], variants[v][1])
        y[lo:hi] = xf[lo:hi] @ w_eff.T
    return y


def matmul_bruteforce(x, w_base, variants, token_variant):
    """Pure-Python loops, no numpy products: y[t][r] = sum_k x[t][k] * (w[r][k] + alpha*s[r][k])
    with s read bit by bit from the packed words.  For tiny shapes only."""
    x = [[float(v) for v in row] for row in np.asarray(x, dtype=np.float64)]
    w = [[float(v) for v in row] for row in np.asarray(w_base, dtype=np.float64)]
    d_out, d_in = len(w), len(w[0])
    y = []
    for t, xt in enumerate(x):
        v = int(token_variant[t])
        row_out = []
        for r in range(d_out):
            acc = 0.0
            for k in range(d_in):
                weff = w[r][k]
                if v >= 0:
                    words, alpha = variants[v]
                    bit = (int(words[r][k // 32]) >> (k % 32)) & 1
                    a = np.asarray(alpha, dtype=np.float32)
                    scale = float(a) if a.ndim == 0 else float(a[r])
                    weff += scale * (1.0 if bit else -1.0)
                acc += xt[k] * weff
            row_out.append(acc)
        y.append(row_out)
    return np.asarray(y, dtype=np.float64)
