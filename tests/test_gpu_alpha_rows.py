"""GPU parity of per-output-row scales: bitdelta_compress_rows against the oracle (bits exact,
every alpha_r within 1e-6 relative), and the fused matmul with per-row variants, mixed with
per-matrix ones, on the GEMV, streaming, split and prefill kernels and under the automatic
choice (the split kernel for 5..256 tokens, where per-row pairs take their own accumulators and
each piece applies alpha_r before its sums leave the registers)."""
import numpy as np
import pytest

import oracle.bitdelta_oracle as O
import workloads as WL
from parity import (DELTA_RESIDUAL_TOL_BF16, ROW_L2_TOL, bf16_dev, delta_residual, f32_dev,
                    gpu_compress, oracle_delta_term, row_rel_l2, tile_words_128, words_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bd = pytest.importorskip("tenant_serving_bitdelta_amd")


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def gpu_compress_rows(delta, offset_words=False):
    d_out, d_in = delta.shape
    nw = d_out * d_in // 32
    if offset_words:  # a word array that is only 4-byte aligned
        buf = torch.empty(nw + 4, dtype=torch.int32, device="cuda")
        words = buf[1:1 + nw].view(d_out, d_in // 32)
    else:
        words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
    alpha = torch.empty(d_out, dtype=torch.float32, device="cuda")
    nt = bd.sign_words_t128(d_out, d_in)
    tiled = torch.empty(nt, dtype=torch.int32, device="cuda") if nt > 0 else None
    bd.compress_rows(f32_dev(delta), words, alpha, tiled=tiled)
    return words, alpha, tiled


def check_compress_rows(delta, offset_words=False):
    words, alpha, tiled = gpu_compress_rows(delta, offset_words)
    torch.cuda.synchronize()
    ref_words, ref_alpha = O.compress_rows_ref(delta)
    np.testing.assert_array_equal(words_host(words), ref_words)
    got = alpha.cpu().numpy().astype(np.float64)
    ref = ref_alpha.astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-6 * np.abs(ref)), np.max(np.abs(got - ref) / np.maximum(ref, 1e-300))
    if tiled is not None:
        d_out, d_in = delta.shape
        real = tile_words_128(np.ones_like(ref_words), d_out, d_in) == 1
        np.testing.assert_array_equal(tiled.cpu().numpy().view(np.uint32)[real],
                                      tile_words_128(ref_words, d_out, d_in)[real])
    return words, alpha


def _deltas(rng, d_out, d_in):
    d = rng.laplace(0, 3e-4, size=(d_out, d_in)) * rng.uniform(0.1, 10.0, size=(d_out, 1))
    d = d.astype(np.float32)
    d[rng.random(d.shape) < 0.02] = 0.0
    return d


# whole lines for d_in % 128 == 0, word by word otherwise; ragged rows and column groups
@pytest.mark.parametrize("d_out,d_in,seed", [(1, 32, 41), (3, 64, 42), (17, 96, 43), (64, 1056, 44),
                                             (255, 512, 45), (130, 3200, 46), (9, 1152, 47),
                                             (33, 8192, 48), (1000, 4096, 49)])
def test_compress_rows_shapes(d_out, d_in, seed):
    rng = np.random.default_rng(seed)
    d = _deltas(rng, d_out, d_in)
    if d_out > 2:
        d[1] = 0.0     # a row with no change: alpha 0, every bit +1
        d[2] = -2e-3   # a row of constant magnitude: alpha exactly 2e-3 in float32
    check_compress_rows(d)


def test_compress_rows_unaligned_words_and_repeatable():
    rng = np.random.default_rng(50)
    d = _deltas(rng, 77, 2048)
    w1, a1 = check_compress_rows(d, offset_words=True)
    w2, a2 = check_compress_rows(d)
    assert torch.equal(w1, w2) and torch.equal(a1, a2)


def run_rows_matmul(m, d_out, d_in, rows_mask, path, out_dtype, seed):
    rng = np.random.default_rng(seed)
    w_bits = WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32))
    x_bits = WL.f32_to_bf16_bits(rng.normal(0, 1, size=(m, d_in)).astype(np.float32))
    var_gpu, var_ref = [], []
    for per_row in rows_mask:
        d = (rng.laplace(0, 1e-3, size=(d_out, d_in)) *
             rng.uniform(0.2, 5.0, size=(d_out, 1))).astype(np.float32)
        if per_row:
            words, alpha, tiled = gpu_compress_rows(d)
            var_ref.append(O.compress_rows_ref(d))
        else:
            (words, alpha, tiled), = gpu_compress([d])
            var_ref.append(O.compress_ref(d))
        var_gpu.append((words, alpha, tiled))
    nv = len(rows_mask)
    ids = rng.integers(-1, nv, size=m)
    ids[:nv] = np.arange(nv)[: min(nv, m)]  # every variant has tokens when m allows
    perm, offs, segv = bd.plan_segments(ids, nv)
    x = bf16_dev(x_bits[perm])
    y = bd.matmul(x, bf16_dev(w_bits), var_gpu, offs, segv, out_dtype=out_dtype, path=path)
    torch.cuda.synchronize()
    xf = O.bf16_bits_to_f64(x_bits)[perm]
    y_ref = O.matmul_ref(xf, O.bf16_bits_to_f64(w_bits), var_ref, offs, segv)
    y_got = y.float().cpu().numpy().astype(np.float64)
    rel = row_rel_l2(y_got, y_ref)
    assert rel.max() <= ROW_L2_TOL, f"row rel L2 {rel.max():.3e}"
    dres = delta_residual(y_got, y_ref, oracle_delta_term(xf, var_ref, offs, segv, d_out, d_in))
    if out_dtype == "f32":
        # the prefill kernel (also the automatic choice above 256 tokens) rounds W_eff to bf16;
        # the split kernel (the automatic choice for 5..256 tokens) takes x' as two fp6 terms
        eff = path if path != "auto" else {1: "gemv", 2: "stream", 3: "prefill", 4: "split"}[
            bd.auto_path(m, offs, segv)]
        lim = {"prefill": (5e-3, 0.75), "split": (5e-3, 1e-2)}.get(eff, (1e-5, 1e-2))
        assert rel.max() <= lim[0], f"f32 row rel L2 {rel.max():.3e}"
        assert dres.max() <= lim[1], f"delta residual {dres.max():.3e}"
    else:
        assert dres.max() <= DELTA_RESIDUAL_TOL_BF16, f"delta residual {dres.max():.3e}"


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,d_out,d_in,rows_mask,path,seed", [
    (1, 130, 1056, (1,), "gemv", 60),
    (3, 257, 512, (1, 0), "gemv", 61),
    (4, 64, 96, (0, 1, 1), "gemv", 62),
    (5, 200, 1024, (1, 0, 1), "stream", 63),
    (40, 130, 2048, (1, 1), "stream", 64),
    (300, 300, 640, (1, 0), "prefill", 65),
    (260, 129, 1056, (1, 1, 0), "prefill", 66),
    (64, 384, 1024, (1, 0, 1, 0), "auto", 67),
    (512, 256, 512, (0, 1), "auto", 68),
    (17, 130, 640, (1,), "split", 69),
    (200, 136, 2048, (1, 0, 1, 1, 0), "split", 72),
    (256, 257, 1024, (1, 1, 0), "split", 73),
    (40, 1000, 16384, (1, 0, 1), "split", 74),   # few row blocks, many K steps: K-split pieces
])
def test_matmul_alpha_rows(m, d_out, d_in, rows_mask, path, seed, out_dtype):
    run_rows_matmul(m, d_out, d_in, rows_mask, path, out_dtype, seed)


def test_equal_row_scales_match_the_scalar_form():
    """Per-row scales that are all the same value give exactly the per-matrix result."""
    rng = np.random.default_rng(70)
    d_out, d_in, m = 256, 1024, 24
    w = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)))
    x = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 1, size=(m, d_in)).astype(np.float32)))
    (words, alpha, tiled), = gpu_compress([rng.laplace(0, 1e-3, size=(d_out, d_in)).astype(np.float32)])
    rows = alpha.expand(d_out).contiguous()
    offs, segv = np.array([0, m], dtype=np.int32), np.array([0], dtype=np.int32)
    for path in ("stream", "prefill"):
        y1 = bd.matmul(x, w, [(words, alpha, tiled)], offs, segv, out_dtype="f32", path=path)
        y2 = bd.matmul(x, w, [(words, rows, tiled)], offs, segv, out_dtype="f32", path=path)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), path
    y1 = bd.matmul(x[:2], w, [(words, alpha, tiled)], np.array([0, 2], dtype=np.int32), segv,
                   out_dtype="f32", path="gemv")
    y2 = bd.matmul(x[:2], w, [(words, rows, tiled)], np.array([0, 2], dtype=np.int32), segv,
                   out_dtype="f32", path="gemv")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_split_per_row_variants_grouped_and_repeatable():
    """Per-row variants on the split kernel in a grouped launch with linears of different K
    (long ones cut into K pieces that meet in partial slots), mixed with per-matrix variants and
    base-model tokens: each linear against the oracle, the same result from single calls, and
    bit-identical repeats; equal row scales agree with the per-matrix form to the split path's
    precision."""
    rng = np.random.default_rng(71)
    m, nv = 48, 4
    ids = rng.integers(-1, nv, size=m).astype(np.int32)
    perm, offs, segv = bd.plan_segments(ids, nv)
    probs, refs = [], []
    for d_out, d_in in [(384, 2048), (256, 12288), (130, 4096)]:
        w_bits = WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32))
        x_bits = WL.f32_to_bf16_bits(rng.normal(size=(m, d_in)).astype(np.float32))
        var_gpu, var_ref = [], []
        for v in range(nv):
            d = (rng.laplace(0, 4e-4, size=(d_out, d_in)) *
                 rng.uniform(0.2, 5.0, size=(d_out, 1))).astype(np.float32)
            if v % 2 == 0:
                var_gpu.append(gpu_compress_rows(d))
                var_ref.append(O.compress_rows_ref(d))
            else:
                var_gpu.append(gpu_compress([d])[0])
                var_ref.append(O.compress_ref(d))
        y = torch.empty((m, d_out), dtype=torch.float32, device="cuda")
        probs.append((bf16_dev(x_bits[perm]), bf16_dev(w_bits), y, var_gpu))
        refs.append(O.matmul_ref(O.bf16_bits_to_f64(x_bits)[perm], O.bf16_bits_to_f64(w_bits),
                                 var_ref, offs, segv))
    bd.matmul_grouped(probs, offs, segv, path="split", out_dtype="f32")
    torch.cuda.synchronize()
    for (x, w, y, var), y_ref in zip(probs, refs):
        assert row_rel_l2(y.cpu().numpy().astype(np.float64), y_ref).max() <= 5e-3
        y1 = bd.matmul(x, w, var, offs, segv, out_dtype="f32", path="split")
        y2 = bd.matmul(x, w, var, offs, segv, out_dtype="f32", path="split")
        assert torch.equal(y1, y2)
        assert row_rel_l2(y1.cpu().numpy().astype(np.float64), y_ref).max() <= 5e-3
    # equal row scales: the same sums as the per-matrix form, quantised from x instead of alpha x
    d_out, d_in = 256, 1024
    w = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)))
    x = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 1, size=(24, d_in)).astype(np.float32)))
    (words, alpha, tiled), = gpu_compress([rng.laplace(0, 1e-3, size=(d_out, d_in)).astype(np.float32)])
    rows = alpha.expand(d_out).contiguous()
    o, sv = np.array([0, 24], dtype=np.int32), np.array([0], dtype=np.int32)
    y1 = bd.matmul(x, w, [(None, alpha, tiled)], o, sv, out_dtype="f32", path="split")
    y2 = bd.matmul(x, w, [(None, rows, tiled)], o, sv, out_dtype="f32", path="split")
    y0 = bd.matmul(x, w, [(words, alpha, None)], o, sv, out_dtype="f32", path="stream")  # exact
    torch.cuda.synchronize()
    ref = y0.cpu().numpy().astype(np.float64)
    for y in (y1, y2):
        assert row_rel_l2(y.cpu().numpy().astype(np.float64), ref).max() <= 5e-3


def test_per_row_alpha_size_checked():
    rng = np.random.default_rng(75)
    d_out, d_in, m = 128, 256, 16
    words, alpha, tiled = gpu_compress_rows(rng.laplace(0, 1e-3, size=(d_out, d_in)).astype(np.float32))
    w = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)))
    x = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 1, size=(m, d_in)).astype(np.float32)))
    with pytest.raises(ValueError):
        bd.matmul(x, w, [(words, alpha[:3], tiled)], np.array([0, m], dtype=np.int32),
                  np.array([0], dtype=np.int32))
