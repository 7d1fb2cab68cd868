"""GPU parity of the single resident sign layout, the unfused reconstruction and the delta upload:

* variants held only in the 128-row tiled layout (no row-major copy) give the oracle's result on
  every kernel path, and the same bits as row-major-only variants on the paths that read either;
* compress writes the tiled layout alone;
* bitdelta_reconstruct writes W_eff = bf16(fp32(w) + (+-alpha)) bit for bit, and the unfused
  product with it equals the fused prefill kernel bit for bit;
* bitdelta_upload_variant turns the row-major storage format into the kernels' layout, and a
  variant loaded through the residency manager (request, evict, upload, event, poll) serves
  tokens that match the oracle.
"""
import zlib

import numpy as np
import pytest

import oracle.bitdelta_oracle as O
import workloads as WL
from parity import (DELTA_RESIDUAL_TOL_BF16, ROW_L2_TOL, bf16_dev, delta_residual, f32_dev,
                    oracle_delta_term, row_rel_l2, tile_words_128, words_host)

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


def compress_layout(delta, layout, per_row=False):
    """Compress on the device into 'rowmajor', 'tiled' or 'both' layouts: (words, alpha, tiled)."""
    d_out, d_in = delta.shape
    words = (torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
             if layout in ("rowmajor", "both") else None)
    tiled = (torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
             if layout in ("tiled", "both") else None)
    alpha = torch.empty(d_out if per_row else 1, dtype=torch.float32, device="cuda")
    (bd.compress_rows if per_row else bd.compress)(f32_dev(delta), words, alpha, tiled=tiled)
    return words, alpha, tiled


LAYOUT_CASES = [
    # (name, d_out, d_in, M, variants, paths)
    ("m3", 200, 1024, 3, 3, ("gemv", "stream", "split", "prefill")),
    ("m17", 130, 640, 17, 5, ("stream", "split", "prefill")),
    ("m64-14v", 192, 1024, 64, 14, ("auto", "stream", "split", "prefill")),
    ("m300", 72, 2048, 300, 4, ("auto", "stream", "split", "prefill")),
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=lambda c: c[0])
def test_tiled_only_variants(case):
    name, d_out, d_in, m, nv, paths = case
    c = WL.linear_case(seed=zlib.crc32(name.encode()) % 1000 + 500, d_out=d_out, d_in=d_in, m=m,
                       num_variants=nv, base_frac=0.1, zero_frac=0.01)
    perm, offs, segv = bd.plan_segments(c["token_variant"], nv)
    w, x = bf16_dev(c["w"]), bf16_dev(c["x"][perm])
    tiled_only = [compress_layout(d, "tiled") for d in c["deltas"]]
    rowmajor_only = [compress_layout(d, "rowmajor") for d in c["deltas"]]
    var_ref = [O.compress_ref(d) for d in c["deltas"]]
    for (wd, _, td), (wr, _, _), (rw, _) in zip(tiled_only, rowmajor_only, var_ref):
        assert wd is None and td is not None
        np.testing.assert_array_equal(words_host(wr), rw)
        real = tile_words_128(np.ones_like(rw), d_out, d_in) == 1
        np.testing.assert_array_equal(td.cpu().numpy().view(np.uint32)[real],
                                      tile_words_128(rw, d_out, d_in)[real])
    xf = O.bf16_bits_to_f64(c["x"])[perm]
    y_ref = O.matmul_ref(xf, O.bf16_bits_to_f64(c["w"]), var_ref, offs, segv)
    y_delta = oracle_delta_term(xf, var_ref, offs, segv, d_out, d_in)
    for path in paths:
        # the kernel family that runs (AUTO picks by batch size)
        eff = path if path != "auto" else {1: "gemv", 2: "stream", 3: "prefill", 4: "split"}[
            bd.auto_path(m, offs, segv)]
        for out in ("bf16", "f32"):
            y_t = bd.matmul(x, w, tiled_only, offs, segv, out_dtype=out, path=path)
            got = y_t.float().cpu().numpy().astype(np.float64)
            assert row_rel_l2(got, y_ref).max() <= ROW_L2_TOL, (path, out)
            dres = delta_residual(got, y_ref, y_delta)
            # fp32 output: prefill rounds W_eff to bf16 (the delta term then carries that
            # rounding); the other paths keep it to fp32 or 8 significant bits
            lim = DELTA_RESIDUAL_TOL_BF16 if out == "bf16" else (0.75 if eff == "prefill" else 1e-2)
            assert dres.max() <= lim, (path, out, float(dres.max()))
            if path in ("gemv", "stream", "prefill"):
                # the layout changes only where the words are read from: the same bits
                y_r = bd.matmul(x, w, rowmajor_only, offs, segv, out_dtype=out, path=path)
                assert torch.equal(y_t, y_r), (path, out)


def test_mixed_layouts_in_one_batch():
    """Variants of one call in different layouts (tiled only, row-major only, both)."""
    d_out, d_in, m = 160, 1024, 40
    c = WL.linear_case(seed=611, d_out=d_out, d_in=d_in, m=m, num_variants=3, base_frac=0.1)
    perm, offs, segv = bd.plan_segments(c["token_variant"], 3)
    w, x = bf16_dev(c["w"]), bf16_dev(c["x"][perm])
    mixed = [compress_layout(c["deltas"][0], "tiled"), compress_layout(c["deltas"][1], "rowmajor"),
             compress_layout(c["deltas"][2], "both")]
    both = [compress_layout(d, "both") for d in c["deltas"]]
    for path in ("stream", "prefill"):
        assert torch.equal(bd.matmul(x, w, mixed, offs, segv, out_dtype="f32", path=path),
                           bd.matmul(x, w, both, offs, segv, out_dtype="f32", path=path)), path
    # split needs the tiled words of every variant it serves
    with pytest.raises(bd.BitDeltaError) as err:
        bd.matmul(x, w, mixed, offs, segv, path="split")
    assert err.value.status == 5
    ids = c["token_variant"][:4]
    p4, o4, s4 = bd.plan_segments(ids, 3)
    x4 = bf16_dev(c["x"][p4])
    assert torch.equal(bd.matmul(x4, w, mixed, o4, s4, out_dtype="f32", path="gemv"),
                       bd.matmul(x4, w, both, o4, s4, out_dtype="f32", path="gemv"))


@pytest.mark.parametrize("per_row", [False, True])
def test_compress_tiled_only(per_row):
    rng = np.random.default_rng(612 + per_row)
    d_out, d_in = 300, 2176
    d = rng.laplace(0, 3e-4, size=(d_out, d_in)).astype(np.float32)
    d[rng.random(d.shape) < 0.02] = 0.0
    words, alpha, tiled = compress_layout(d, "tiled", per_row=per_row)
    torch.cuda.synchronize()
    ref_words = O.pack_signs_ref(O.signs_ref(d))
    real = tile_words_128(np.ones_like(ref_words), d_out, d_in) == 1
    np.testing.assert_array_equal(tiled.cpu().numpy().view(np.uint32)[real],
                                  tile_words_128(ref_words, d_out, d_in)[real])
    ref_a = (O.alpha_rows_ref(d) if per_row else np.array([O.alpha_ref(d)])).astype(np.float64)
    got_a = alpha.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got_a - ref_a) <= 1e-6 * ref_a)


def test_compress_from_weights_tiled_only():
    rng = np.random.default_rng(613)
    d_out, d_in = 136, 1024
    base = rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)
    ft = base + rng.laplace(0, 3e-4, size=(d_out, d_in)).astype(np.float32)
    fb, bb = WL.f32_to_bf16_bits(ft), WL.f32_to_bf16_bits(base)
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    bd.compress_from_weights(bf16_dev(fb), bf16_dev(bb), None, alpha, tiled=tiled)
    torch.cuda.synchronize()
    ref_words, ref_alpha = O.compress_from_weights_ref(fb, bb)
    real = tile_words_128(np.ones_like(ref_words), d_out, d_in) == 1
    np.testing.assert_array_equal(tiled.cpu().numpy().view(np.uint32)[real],
                                  tile_words_128(ref_words, d_out, d_in)[real])
    assert abs(float(alpha.item()) - float(ref_alpha)) <= 1e-6 * float(ref_alpha)


def weff_bf16_ref(w_bits, words, alpha):
    """The oracle's exact W_eff rounded to float32, then to bf16 (nearest even): the value of one
    fp32 addition of the bf16 weight and +-alpha, rounded to bf16 (the fp64 sum of a bf16 and a
    float32 rounds to the same float32 as the fp32 addition does)."""
    weff = O.reconstruct_ref(O.bf16_bits_to_f64(w_bits), words, alpha)
    return WL.f32_to_bf16_bits(weff.astype(np.float32))


@pytest.mark.parametrize("d_out,d_in,layout,per_row", [(70, 96, "rowmajor", False),
                                                       (130, 1024, "tiled", False),
                                                       (257, 2048, "both", True),
                                                       (64, 640, "rowmajor", True)])
def test_reconstruct_bit_exact(d_out, d_in, layout, per_row):
    rng = np.random.default_rng(d_out + d_in)
    w_bits = WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32))
    delta = rng.laplace(0, 3e-4, size=(d_out, d_in)).astype(np.float32)
    words, alpha, tiled = compress_layout(delta, layout, per_row=per_row)
    w_eff = bd.reconstruct(bf16_dev(w_bits), (words, alpha, tiled))
    torch.cuda.synchronize()
    ref_words = O.pack_signs_ref(O.signs_ref(delta))
    a_gpu = alpha.cpu().numpy()  # the stored scale(s) the kernel applied
    want = weff_bf16_ref(w_bits, ref_words, a_gpu if per_row else a_gpu[0])
    np.testing.assert_array_equal(w_eff.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_unfused_equals_fused_prefill():
    """W_eff materialised, then the product with the base-model segment, against the fused
    prefill kernel (which rebuilds the same bf16 W_eff in registers): bit for bit, and both
    within the tolerance of the oracle."""
    d_out, d_in, m = 512, 1024, 700
    c = WL.linear_case(seed=614, d_out=d_out, d_in=d_in, m=m, num_variants=3, base_frac=0.0)
    perm, offs, segv = bd.plan_segments(c["token_variant"], 3)
    w, x = bf16_dev(c["w"]), bf16_dev(c["x"][perm])
    var = [compress_layout(d, "tiled") for d in c["deltas"]]
    fused = bd.matmul(x, w, var, offs, segv, out_dtype="f32", path="prefill")
    unfused = torch.empty_like(fused)
    for s, v in enumerate(segv):
        lo, hi = int(offs[s]), int(offs[s + 1])
        w_eff = bd.reconstruct(w, var[int(v)])
        bd.matmul(x[lo:hi].contiguous(), w_eff, [], [0, hi - lo], [-1], y=unfused[lo:hi],
                  out_dtype="f32", path="prefill")
    assert torch.equal(fused, unfused)
    var_ref = [O.compress_ref(d) for d in c["deltas"]]
    y_ref = O.matmul_ref(O.bf16_bits_to_f64(c["x"])[perm], O.bf16_bits_to_f64(c["w"]), var_ref,
                         offs, segv)
    assert row_rel_l2(unfused.cpu().numpy().astype(np.float64), y_ref).max() <= 5e-3


@pytest.mark.parametrize("d_out,d_in,dest", [(300, 2048, "tiled"), (128, 1024, "both"),
                                             (77, 96, "rowmajor")])
def test_upload_variant(d_out, d_in, dest):
    rng = np.random.default_rng(615 + d_out)
    delta = rng.laplace(0, 3e-4, size=(d_out, d_in)).astype(np.float32)
    ref_words, ref_alpha = O.compress_ref(delta)
    host_words = torch.from_numpy(ref_words.view(np.int32).copy()).pin_memory()
    host_alpha = torch.tensor([float(ref_alpha)], dtype=torch.float32).pin_memory()
    words = (torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
             if dest in ("rowmajor", "both") else None)
    tiled = (torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
             if dest in ("tiled", "both") else None)
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    bd.upload_variant(host_words, host_alpha, d_out, d_in, words=words, tiled=tiled, alpha=alpha)
    torch.cuda.synchronize()
    if words is not None:
        np.testing.assert_array_equal(words_host(words), ref_words)
    if tiled is not None:
        real = tile_words_128(np.ones_like(ref_words), d_out, d_in) == 1
        np.testing.assert_array_equal(tiled.cpu().numpy().view(np.uint32)[real],
                                      tile_words_128(ref_words, d_out, d_in)[real])
    assert float(alpha.item()) == float(ref_alpha)


def test_residency_serves_freshly_loaded_variant():
    """The cold-start path end to end: a manager with room for two of three variants of one
    matrix; each request that answers LOAD uploads the variant's stored (row-major) words into
    the memory of the slot it frees, records an event, and the variant becomes resident when
    poll finds the event done; the tokens of every freshly loaded variant then match the oracle.
    A held variant is never evicted while its request is in flight."""
    d_out, d_in, m = 256, 2048, 24
    rng = np.random.default_rng(616)
    w_bits = WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32))
    deltas = [rng.laplace(0, b, size=(d_out, d_in)).astype(np.float32) for b in (2e-4, 3e-4, 4e-4)]
    stored = [O.compress_ref(d) for d in deltas]   # the storage format, on the host
    host = [(torch.from_numpy(wd.view(np.int32).copy()).pin_memory(),
             torch.tensor([float(a)], dtype=torch.float32).pin_memory()) for wd, a in stored]
    nbytes = d_out * d_in // 8 + 4
    mgr = bd.Residency([nbytes] * 3, 2 * nbytes, num_pinned=0)
    slots = [(torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda"),
              torch.empty(1, dtype=torch.float32, device="cuda")) for _ in range(2)]
    free, where = [0, 1], {}
    w = bf16_dev(w_bits)
    upload_stream = torch.cuda.Stream()
    events = {}

    def serve(v):
        act, evicted = mgr.request(v, hold=True)
        assert act in (bd.Residency.HIT, bd.Residency.LOAD), act
        for e in evicted:
            free.append(where.pop(e))
        if act == bd.Residency.LOAD:
            slot = free.pop()
            where[v] = slot
            with torch.cuda.stream(upload_stream):
                bd.upload_variant(host[v][0], host[v][1], d_out, d_in, tiled=slots[slot][0],
                                  alpha=slots[slot][1], stream=upload_stream.cuda_stream)
                events[v] = torch.cuda.Event()
                events[v].record(upload_stream)
            mgr.load_enqueued(v, events[v])
            while mgr.state(v) != bd.Residency.RESIDENT:
                mgr.poll()
        tiled, alpha = slots[where[v]]
        x_bits = WL.f32_to_bf16_bits(rng.normal(size=(m, d_in)).astype(np.float32))
        y = bd.matmul(bf16_dev(x_bits), w, [(None, alpha, tiled)], [0, m], [0], out_dtype="f32")
        torch.cuda.synchronize()
        mgr.release(v)
        y_ref = O.matmul_ref(O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(w_bits), [stored[v]],
                             [0, m], [0])
        assert row_rel_l2(y.cpu().numpy().astype(np.float64), y_ref).max() <= 5e-3, v
        return act, evicted

    assert serve(0) == (bd.Residency.LOAD, [])
    assert serve(1) == (bd.Residency.LOAD, [])
    assert serve(0) == (bd.Residency.HIT, [])
    assert serve(2) == (bd.Residency.LOAD, [1])   # 1 is the least recently requested
    assert serve(1) == (bd.Residency.LOAD, [0])
    # held variants stay: with 2 and 1 both held a request for 0 finds no room; once 1 is
    # released it is the one evicted
    assert mgr.request(2, hold=True) == (bd.Residency.HIT, [])
    assert mgr.request(1, hold=True) == (bd.Residency.HIT, [])
    assert mgr.request(0) == (bd.Residency.NO_ROOM, [])
    mgr.release(1)
    assert mgr.request(0) == (bd.Residency.LOAD, [1])
    mgr.release(2)
