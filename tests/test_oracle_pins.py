"""Pins of the CPU oracle against what the BitDelta post and mathematics fix, independently of
the oracle's own formulas: hand-derived worked examples (tests/golden), printed storage
figures, closed forms, least-squares optimality, an energy identity, Laplace statistics,
special cases that reduce to plain integer products, and brute force on tiny shapes.

The ``check_*`` functions take the oracle module so the mutation tests at the bottom can plant
a plausible mistake in the oracle (on the CPU) and show that some pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.bitdelta_oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------------
# Pin checks
# ----------------------------------------------------------------------------------------------

def check_bit_order_golden(o):
    g = _load("bit_order.json")
    d = np.zeros((2, 64), dtype=np.float32)
    d[0] = np.where(np.arange(64) % 2 == 0, 1.0, -1.0)
    d[1, 0] = np.float32(-0.0)
    d[1, 1] = np.float32(-1e-40)
    d[1, 31] = -2.0
    d[1, 40] = 5.0
    d[1, 63] = -3.0
    assert np.signbit(d[1, 0]) and d[1, 1] < 0 and d[1, 1] > -1e-38  # -0.0 and a subnormal
    words, alpha = o.compress_ref(d)
    np.testing.assert_array_equal(words, np.asarray(g["words"], dtype=np.uint32))
    assert float(alpha) == g["alpha"]


def check_tiny_linear_golden(o):
    g = _load("tiny_linear.json")
    k = np.arange(32)
    w = np.stack([np.full(32, 0.5), np.where(k % 2 == 0, 0.25, -0.25)])
    d = np.stack([np.full(32, 0.125), np.where(k < 16, -0.125, 0.375)]).astype(np.float32)
    words, alpha = o.compress_ref(d)
    np.testing.assert_array_equal(words, np.asarray(g["words"], dtype=np.uint32))
    assert float(alpha) == g["alpha"]
    x = np.stack([np.ones(32), (k % 2 == 0).astype(float), (k < 16).astype(float), np.ones(32)])
    ids = np.asarray(g["token_variant"])
    perm, offs, segv = o.plan_segments_ref(ids, 1)
    y_sorted = o.matmul_ref(x[perm], w, [(words, alpha)], offs, segv)
    y = np.empty_like(y_sorted)
    y[perm] = y_sorted
    np.testing.assert_array_equal(y, np.asarray(g["y"]))
    np.testing.assert_array_equal(o.matmul_bruteforce(x, w, [(words, alpha)], ids), np.asarray(g["y"]))


def check_storage_arithmetic(o):
    g = _load("storage_arithmetic.json")
    ex = g["packed_example"]
    # bytes of the packed sign matrix alone (drop the one float32 alpha)
    assert o.packed_nbytes_ref(ex["d_out"], ex["d_in"]) - 4 == ex["packed_rows"] * ex["packed_cols_bytes"]
    n = 1 << 20
    assert (o.packed_nbytes_ref(1024, 1024) - 4) / (4 * n) == g["ratio_vs_fp32"]
    # 70B bits = 8.75 GB; 14 variants vs the naive layout
    assert g["params_70b"] // 8 == g["delta_bytes_70b"]
    total = g["base_bytes_70b_bf16"] + g["variants"] * g["delta_bytes_70b"]
    assert abs(total - g["bitdelta_bytes_approx"]) / g["bitdelta_bytes_approx"] < 0.01
    assert g["variants"] * g["base_bytes_70b_bf16"] == g["naive_bytes"]
    assert round(100 * (1 - total / g["naive_bytes"])) == g["reduction_percent_approx"]


def check_alpha_closed_forms(o):
    # constant magnitude: alpha is that magnitude exactly, whatever the signs
    rng = np.random.default_rng(1)
    d = (np.where(rng.random((8, 64)) < 0.5, -1, 1) * 0.375).astype(np.float32)
    assert float(o.alpha_ref(d)) == 0.375
    # a single nonzero element c in an n-element matrix: alpha = |c| / n
    d = np.zeros((4, 32), dtype=np.float32)
    d[2, 7] = -12.0
    assert float(o.alpha_ref(d)) == 12.0 / 128
    # all zero
    assert float(o.alpha_ref(np.zeros((3, 32), np.float32))) == 0.0


def check_alpha_large_matrices(o):
    """Matrices above the oracle's exact-summation limit (n = 4096 x 2048 = 2^23 elements, the
    branch every full-size alpha check of the 70B shapes goes through), against values the
    mathematics fixes: a constant magnitude with random signs gives that magnitude; a single
    nonzero c gives |c| / n; the ramp Delta_i = (i - n/4) h over the flattened matrix gives
    h (m (m + 1) + (n - m - 1)(n - m)) / (2 n) with m = n/4, evaluated here in integers (every
    partial sum of the ramp is an integer multiple of h below 2^53 h, so an exact fp64 sum is
    reachable and the expected float32 is the correctly rounded closed form)."""
    d_out, d_in = 4096, 2048
    n = d_out * d_in
    assert n > getattr(o, "FSUM_MAX", 0)
    rng = np.random.default_rng(3)
    c = 1.5 * 2.0 ** -12
    d = (np.where(rng.random((d_out, d_in)) < 0.5, -c, c)).astype(np.float32)
    assert float(o.alpha_ref(d)) == c
    d = np.zeros((d_out, d_in), dtype=np.float32)
    d[1234, 567] = -0.75
    assert float(o.alpha_ref(d)) == 0.75 / n
    h, m = 2.0 ** -30, n // 4
    ramp = ((np.arange(n, dtype=np.int64) - m).astype(np.float64) * h).astype(np.float32)
    total_over_h = (m * (m + 1) + (n - m - 1) * (n - m)) // 2      # sum of |i - m|, exact integer
    want = np.float32(total_over_h * 2.0 ** -53)                     # h / n = 2^-53: exact in fp64
    assert o.alpha_ref(ramp.reshape(d_out, d_in)) == want


def check_alpha_least_squares(o):
    """For fixed signs S the best scale minimises ||Delta - a S||_F^2; its minimiser is
    <Delta, S>/n = sum|Delta|/n.  The energy identity ||Delta - alpha S||^2 = ||Delta||^2 - n alpha^2
    must hold (to rounding of the float32 alpha)."""
    rng = np.random.default_rng(2)
    d = rng.laplace(0, 3e-4, size=(64, 96)).astype(np.float32)
    words, alpha = o.compress_ref(d)
    s = o.unpack_signs_ref(words, d.shape[1]).astype(np.float64)
    df = d.astype(np.float64)

    def err(a):
        return float(np.sum((df - a * s) ** 2))

    a = float(alpha)
    for eps in (1e-2, 1e-3):
        assert err(a) < err(a * (1 + eps)) and err(a) < err(a * (1 - eps))
    n = d.size
    lhs = err(a)
    rhs = float(np.sum(df ** 2)) - n * a * a
    assert abs(lhs - rhs) <= 1e-6 * float(np.sum(df ** 2))


def check_laplace_statistics(o):
    """E|Delta| = b for Laplace(0, b) (the post's model); with 1% exact zeros alpha ~ 0.99 b.
    Config 1 has n = 131072, so the standard error of alpha/b is about 1/sqrt(n) = 0.0028."""
    c = WL.config1()
    a = float(o.alpha_ref(c["deltas"][0]))
    assert abs(a / 1e-3 - 0.99) < 5 / math.sqrt(c["deltas"][0].size)


def check_signs_and_roundtrip(o):
    rng = np.random.default_rng(3)
    d = rng.normal(size=(16, 128)).astype(np.float32)
    d[rng.random(d.shape) < 0.1] = 0.0
    d[0, :4] = [np.float32(-0.0), np.float32(0.0), np.float32(-1e-45), np.float32(1e-45)]
    words, _ = o.compress_ref(d)
    s = o.unpack_signs_ref(words, 128)
    expect = np.array([[1 if (v > 0 or v == 0) else -1 for v in row] for row in d.tolist()])
    np.testing.assert_array_equal(s, expect)
    assert list(s[0, :4]) == [1, 1, -1, 1]
    # popcount of the words = number of elements that are not strictly negative
    pop = sum(bin(int(wd)).count("1") for wd in words.ravel())
    assert pop == int(np.sum(~(d < 0)))
    np.testing.assert_array_equal(o.pack_signs_ref(s), words)


def _int_case(rng, m, d_out, d_in):
    x = rng.integers(-3, 4, size=(m, d_in))
    w = rng.integers(-4, 5, size=(d_out, d_in))
    return x, w


def check_zero_delta_is_plain_product(o):
    """Delta = 0: alpha = 0, every bit 1, and y is the plain product x W^T (checked against exact
    integer arithmetic)."""
    rng = np.random.default_rng(4)
    x, w = _int_case(rng, 5, 7, 64)
    words, alpha = o.compress_ref(np.zeros((7, 64), np.float32))
    assert float(alpha) == 0.0 and np.all(words == np.uint32(0xFFFFFFFF))
    y = o.matmul_ref(x, w, [(words, alpha)], [0, 5], [0])
    exact = np.array([[sum(int(a) * int(b) for a, b in zip(xr, wr)) for wr in w] for xr in x])
    np.testing.assert_array_equal(y, exact.astype(np.float64))


def check_zero_base_isolates_delta(o):
    """W_base = 0: y = alpha * x S^T, so every output is alpha times an integer that exact integer
    arithmetic gives (sign and transposition errors show up directly)."""
    rng = np.random.default_rng(5)
    x, _ = _int_case(rng, 3, 5, 64)
    d = rng.laplace(0, 1e-3, size=(5, 64)).astype(np.float32)
    words, alpha = o.compress_ref(d)
    sgn = [[-1 if v < 0 else 1 for v in row] for row in d.tolist()]
    y = o.matmul_ref(x, np.zeros((5, 64)), [(words, alpha)], [0, 3], [0])
    exact = np.array([[sum(int(a) * b for a, b in zip(xr, sr)) for sr in sgn] for xr in x], dtype=np.float64)
    np.testing.assert_allclose(y, float(alpha) * exact, rtol=0, atol=1e-12)


def check_identity_readback(o):
    """x = I (one-hot tokens) reads W_eff back: y[k, r] = W_base[r, k] + alpha * s[r, k]."""
    rng = np.random.default_rng(6)
    d_out, d_in = 6, 32
    w = rng.normal(0, 0.02, size=(d_out, d_in))
    d = rng.laplace(0, 2e-4, size=(d_out, d_in)).astype(np.float32)
    words, alpha = o.compress_ref(d)
    y = o.matmul_ref(np.eye(d_in), w, [(words, alpha)], [0, d_in], [0])
    a = float(alpha)
    for kk in range(d_in):
        for r in range(d_out):
            assert y[kk, r] == w[r, kk] + (a if d[r, kk] >= 0 else -a)


def check_bruteforce_agrees(o):
    rng = np.random.default_rng(7)
    for (m, d_out, d_in, nv) in [(5, 3, 32, 2), (7, 9, 64, 3), (4, 2, 96, 1)]:
        w = rng.normal(0, 0.02, size=(d_out, d_in))
        variants = []
        for _ in range(nv):
            variants.append(o.compress_ref(rng.laplace(0, 1e-3, size=(d_out, d_in)).astype(np.float32)))
        x = rng.normal(size=(m, d_in))
        ids = rng.integers(-1, nv, size=m)
        perm, offs, segv = o.plan_segments_ref(ids, nv)
        ys = o.matmul_ref(x[perm], w, variants, offs, segv)
        y = np.empty_like(ys)
        y[perm] = ys
        np.testing.assert_allclose(y, o.matmul_bruteforce(x, w, variants, ids), rtol=1e-12, atol=1e-12)


def check_plan_is_stable_sort(o):
    rng = np.random.default_rng(8)
    for m in (0, 1, 17, 64):
        ids = rng.integers(-1, 5, size=m)
        perm, offs, segv = o.plan_segments_ref(ids, 5)
        expect = sorted(range(m), key=lambda t: int(ids[t]))  # Python's sort is stable
        assert list(perm) == expect
        assert offs[0] == 0 and offs[-1] == m and len(offs) == len(segv) + 1
        assert all(offs[i] < offs[i + 1] for i in range(len(segv)))
        for s, v in enumerate(segv):
            assert all(int(ids[perm[p]]) == v for p in range(offs[s], offs[s + 1]))
        assert list(segv) == sorted(set(int(v) for v in ids))


def check_batch_invariance(o):
    """A mixed batch equals separate single-variant calls of the fused linear."""
    rng = np.random.default_rng(9)
    d_out, d_in, nv = 8, 64, 3
    w = rng.normal(0, 0.02, size=(d_out, d_in))
    variants = [o.compress_ref(rng.laplace(0, 5e-4, size=(d_out, d_in)).astype(np.float32)) for _ in range(nv)]
    x = rng.normal(size=(12, d_in))
    ids = np.array([2, 0, 1, 1, -1, 0, 2, 2, 0, -1, 1, 0])
    perm, offs, segv = o.plan_segments_ref(ids, nv)
    ys = o.matmul_ref(x[perm], w, variants, offs, segv)
    for p, t in enumerate(perm):
        v = ids[t]
        single = x[t:t + 1] @ w.T if v < 0 else o.fused_linear_ref(x[t:t + 1], w, *variants[v])
        np.testing.assert_allclose(ys[p], single[0], rtol=1e-13, atol=1e-15)


def check_task_vector(o):
    """Compress from a (fine-tuned, base) bf16 pair: a hand-derived example, equal weights
    (Delta = 0: every bit +1, alpha 0), and a zero base (the fine-tuned weights themselves)."""
    g = _load("task_vector.json")
    k = np.arange(32)
    w_base = WL.f32_to_bf16_bits(np.stack([np.ones(32), 0.5 + k / 64]).astype(np.float32))
    w_ft = WL.f32_to_bf16_bits(np.stack([1 + (2 * (k % 4) - 3) / 128, 0.5 + k / 64]).astype(np.float32))
    words, alpha = o.compress_from_weights_ref(w_ft, w_base)
    np.testing.assert_array_equal(words, np.asarray(g["words"], dtype=np.uint32))
    assert float(alpha) == g["alpha"]
    rng = np.random.default_rng(10)
    w = WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(6, 96)).astype(np.float32))
    words, alpha = o.compress_from_weights_ref(w, w)
    assert np.all(words == 0xFFFFFFFF) and float(alpha) == 0.0
    zero = np.zeros_like(w)
    words, alpha = o.compress_from_weights_ref(w, zero)
    ref_words, ref_alpha = o.compress_ref(o.bf16_bits_to_f64(w))
    np.testing.assert_array_equal(words, ref_words)
    assert float(alpha) == float(ref_alpha)


def check_alpha_rows(o):
    """Per-output-row scales: hand-derived closed forms, one row equals the per-matrix scale,
    each alpha_r is the least-squares scale of its row for the row's signs (numpy's lstsq on the
    one-column system), the mean of equal-length rows' scales is the matrix scale, and the signs
    do not depend on the granularity."""
    k = np.arange(32)
    d = np.zeros((3, 32), dtype=np.float32)
    d[0] = np.where(k % 3 == 0, -0.5, 0.5)        # constant magnitude: 0.5
    d[1] = np.where(k % 2 == 0, 1, -1) * k / 32   # |d| = k/32: sum 496/32 over 32 -> 0.484375
    d[2, 9] = -3.0                                # one element: 3/32
    a = o.alpha_rows_ref(d)
    assert a.shape == (3,) and a.dtype == np.float32
    assert [float(v) for v in a] == [0.5, 0.484375, 0.09375]
    rng = np.random.default_rng(21)
    one = rng.laplace(0, 1e-3, size=(1, 160)).astype(np.float32)
    assert float(o.alpha_rows_ref(one)[0]) == float(o.alpha_ref(one))
    d = rng.laplace(0, 3e-4, size=(12, 96)).astype(np.float32)
    d[3] *= 40.0                                  # rows of very different scale
    words, a = o.compress_rows_ref(d)
    s = o.unpack_signs_ref(words, d.shape[1]).astype(np.float64)
    for r in range(d.shape[0]):
        best = np.linalg.lstsq(s[r][:, None], d[r].astype(np.float64), rcond=None)[0][0]
        assert abs(float(a[r]) - best) <= 1e-6 * abs(best)
    assert abs(float(np.mean(a.astype(np.float64))) - float(o.alpha_ref(d))) <= 1e-6 * float(o.alpha_ref(d))
    np.testing.assert_array_equal(words, o.compress_ref(d)[0])


def check_alpha_rows_linear(o):
    """The fused linear with per-row scales: with W_base = 0 and x = the unit vector e_j,
    y[r] = alpha_r * sign(Delta[r][j]) (hand-checkable); equal row scales reduce to the scalar
    form; the pure-loop brute force agrees on a mixed batch of per-row and per-matrix variants."""
    d = np.array([[0.5] * 32, [-1.0] * 32, [0.25 if c % 2 else -0.25 for c in range(32)]],
                 dtype=np.float32)
    words, a = o.compress_rows_ref(d)
    w0 = np.zeros((3, 32))
    for j in (0, 1):
        x = np.zeros((1, 32))
        x[0, j] = 1.0
        y = o.fused_linear_ref(x, w0, words, a)
        want = [0.5, -1.0, 0.25 if j % 2 else -0.25]
        assert [float(v) for v in y[0]] == want
    rng = np.random.default_rng(22)
    w = rng.normal(0, 0.02, size=(5, 64))
    dd = rng.laplace(0, 1e-3, size=(5, 64)).astype(np.float32)
    words, _ = o.compress_ref(dd)
    x = rng.normal(size=(4, 64))
    same = np.full(5, np.float32(7e-4), dtype=np.float32)
    np.testing.assert_allclose(o.fused_linear_ref(x, w, words, same),
                               o.fused_linear_ref(x, w, words, np.float32(7e-4)), rtol=0, atol=1e-15)
    variants = [o.compress_rows_ref(rng.laplace(0, 1e-3, size=(5, 64)).astype(np.float32)),
                o.compress_ref(rng.laplace(0, 1e-3, size=(5, 64)).astype(np.float32))]
    x = rng.normal(size=(7, 64))
    ids = np.array([1, 0, -1, 0, 1, 0, 0])
    perm, offs, segv = o.plan_segments_ref(ids, 2)
    ys = o.matmul_ref(x[perm], w, variants, offs, segv)
    y = np.empty_like(ys)
    y[perm] = ys
    np.testing.assert_allclose(y, o.matmul_bruteforce(x, w, variants, ids), rtol=1e-12, atol=1e-12)


ALL_CHECKS = [
    check_bit_order_golden, check_tiny_linear_golden, check_storage_arithmetic,
    check_alpha_closed_forms, check_alpha_large_matrices, check_alpha_least_squares, check_laplace_statistics,
    check_signs_and_roundtrip, check_zero_delta_is_plain_product, check_zero_base_isolates_delta,
    check_identity_readback, check_bruteforce_agrees, check_plan_is_stable_sort,
    check_batch_invariance, check_task_vector, check_alpha_rows, check_alpha_rows_linear,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)


def test_bf16_helpers_roundtrip():
    a = np.array([1.0, -2.5, 0.1, 3.0e-3, 1 + 2 ** -8, 1 + 3 * 2 ** -9], dtype=np.float32)
    bits = WL.f32_to_bf16_bits(a)
    back = O.bf16_bits_to_f64(bits)
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[4] == 1.0  # tie rounds to even
    assert back[5] == 1 + 2 ** -7  # 1.5 ulp rounds up to 2 ulp
    assert np.all(np.abs(back - a) <= np.abs(a) * 2 ** -8)  # half an ulp of an 8-bit significand


# ----------------------------------------------------------------------------------------------
# Mutation tests: plant a plausible mistake in the oracle and show a pin fails.
# ----------------------------------------------------------------------------------------------

def _signs_le(delta):  # zero mapped to -1
    return np.where(np.asarray(delta) <= 0, np.int8(-1), np.int8(1)).astype(np.int8)


def _signs_float_compare_ftz(delta):  # negative subnormals flushed to zero -> +1
    d = np.asarray(delta, dtype=np.float32)
    d = np.where(np.abs(d) < np.float32(1.1754944e-38), np.float32(0), d)
    return np.where(d < 0, np.int8(-1), np.int8(1)).astype(np.int8)


def _pack_msb_first(signs):
    s = np.asarray(signs)
    d_out, d_in = s.shape
    bits = (s > 0).astype(np.uint64).reshape(d_out, d_in // 32, 32)
    weights = np.left_shift(np.uint64(1), np.arange(31, -1, -1, dtype=np.uint64))
    return (bits * weights).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def _unpack_msb_first(words, d_in):
    w = np.asarray(words, dtype=np.uint32)
    bit = (w[:, :, None] >> np.arange(31, -1, -1, dtype=np.uint32)) & np.uint32(1)
    return (bit.astype(np.int8) * 2 - 1).reshape(w.shape[0], d_in)


def _alpha_row_mean_of_first_row(delta):  # mean over one row instead of the matrix
    return np.float32(np.mean(np.abs(np.asarray(delta, dtype=np.float64))[0]))


def _alpha_rms(delta):  # RMS instead of mean absolute value
    return np.float32(np.sqrt(np.mean(np.asarray(delta, dtype=np.float64) ** 2)))


def _alpha_large_f32_sum(delta):  # above the exact-summation limit, a float32 accumulation
    a = np.abs(np.asarray(delta, dtype=np.float64)).ravel()
    if a.size <= O.FSUM_MAX:
        return _REAL_ALPHA(delta)
    return np.float32(float(np.sum(a.astype(np.float32), dtype=np.float32)) / a.size)


def _alpha_large_n_minus_one(delta):  # above the limit, the sum divided by n - 1
    a = np.abs(np.asarray(delta, dtype=np.float64)).ravel()
    if a.size <= O.FSUM_MAX:
        return _REAL_ALPHA(delta)
    return np.float32(float(np.sum(a)) / (a.size - 1))


def _reconstruct_minus(w_base, words, alpha):  # wrong sign of the delta term
    wb = np.asarray(w_base, dtype=np.float64)
    return wb - np.float64(np.float32(alpha)) * O.unpack_signs_ref(words, wb.shape[1])


def _reconstruct_no_delta(w_base, words, alpha):  # dropped delta term
    return np.asarray(w_base, dtype=np.float64)


def _reconstruct_transposed_bits(w_base, words, alpha):  # signs read with rows/cols swapped
    wb = np.asarray(w_base, dtype=np.float64)
    s = O.unpack_signs_ref(words, wb.shape[1]).astype(np.float64)
    if s.shape[0] == s.shape[1]:
        s = s.T
    else:
        s = np.resize(s.T.ravel(), s.shape)
    return wb + np.float64(np.float32(alpha)) * s


def _matmul_wrong_segment(x, w_base, variants, seg_offsets, seg_variant):  # off-by-one variant
    segv = [(v + 1) % len(variants) if v >= 0 and len(variants) > 1 else v for v in seg_variant]
    return _REAL_MATMUL(x, w_base, variants, seg_offsets, segv)


def _plan_unstable(token_variant, num_variants):  # reverses order inside each group
    perm, offs, segv = _REAL_PLAN(token_variant, num_variants)
    perm = perm.copy()
    for s in range(len(segv)):
        perm[offs[s]:offs[s + 1]] = perm[offs[s]:offs[s + 1]][::-1]
    return perm, offs, segv


def _task_vector_reversed(w_ft_bits, w_base_bits):  # W_base - W_ft
    return O.bf16_bits_to_f64(w_base_bits) - O.bf16_bits_to_f64(w_ft_bits)


def _alpha_rows_of_columns(delta):  # means over columns instead of rows
    return np.abs(np.asarray(delta, dtype=np.float64)).mean(axis=0).astype(np.float32)


def _alpha_rows_divide_by_n(delta):  # row sums divided by the matrix size
    a = np.abs(np.asarray(delta, dtype=np.float64))
    return (a.sum(axis=1) / a.size).astype(np.float32)


def _reconstruct_first_row_alpha(w_base, words, alpha):  # alpha[0] used for every row
    a = np.asarray(alpha, dtype=np.float32)
    return _REAL_RECONSTRUCT(w_base, words, a if a.ndim == 0 else a[0])


_REAL_RECONSTRUCT = O.reconstruct_ref
_REAL_ALPHA = O.alpha_ref
_REAL_MATMUL = O.matmul_ref
_REAL_PLAN = O.plan_segments_ref

MUTANTS = [
    ("signs_ref", _signs_le),
    ("signs_ref", _signs_float_compare_ftz),
    ("pack_signs_ref", _pack_msb_first),
    ("unpack_signs_ref", _unpack_msb_first),
    ("alpha_ref", _alpha_row_mean_of_first_row),
    ("alpha_ref", _alpha_rms),
    ("alpha_ref", _alpha_large_f32_sum),
    ("alpha_ref", _alpha_large_n_minus_one),
    ("reconstruct_ref", _reconstruct_minus),
    ("reconstruct_ref", _reconstruct_no_delta),
    ("reconstruct_ref", _reconstruct_transposed_bits),
    ("matmul_ref", _matmul_wrong_segment),
    ("plan_segments_ref", _plan_unstable),
    ("task_vector_ref", _task_vector_reversed),
    ("alpha_rows_ref", _alpha_rows_of_columns),
    ("alpha_rows_ref", _alpha_rows_divide_by_n),
    ("reconstruct_ref", _reconstruct_first_row_alpha),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    failures = 0
    for check in ALL_CHECKS:
        try:
            check(O)
        except Exception:  # noqa: BLE001 - any failure of a pin counts as a catch
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake in {name}"
