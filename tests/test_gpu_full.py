"""Parity at full size, in the launch configuration bench.py times: one 70B decoder block (q, k,
v, o, gate, up, down), 14 variants compressed on the GPU into the tiled sign layout only (as the
benchmark keeps them), one grouped decode launch (the split path for these batch sizes) with a
caller workspace.  The oracle cannot multiply the whole block quickly, so it checks alpha of every
variant of every linear over the whole Delta, and every token of every variant on 24 sampled
output rows of each linear, through its own fused linear on those rows."""
import numpy as np
import pytest

import oracle.bitdelta_oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bd = pytest.importorskip("tenant_serving_bitdelta_amd")


def _rows(d_out, rng):
    fixed = [0, 1, 127, 128, d_out - 2, d_out - 1]
    extra = rng.choice(d_out, size=18, replace=False)
    return np.unique(np.concatenate([fixed, extra]))


@pytest.mark.parametrize("config,m,dist", [(3, 64, "uniform"), (5, 256, "zipf")])
def test_full_size_block_sampled(config, m, dist):
    nvar = 14
    ids = WL.decode_token_ids(config, m, nvar, dist)
    perm, offs, segv = bd.plan_segments(ids, nvar)
    scales = WL.decode_variant_scales(config)
    rng = np.random.default_rng(1000 + config)

    layers = []
    for name, d_out, d_in in WL.BLOCK_LINEARS:
        print(f"  {name} {d_out}x{d_in}: compress and check alpha of {nvar} variants", flush=True)
        rows = _rows(d_out, rng)
        w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, 0, name, "w"))
        x = WL.gpu_normal_bf16(torch, (m, d_in), 1.0, WL.substream_seed(config, 0, name, "x"))
        variants, ref = [], []
        for v in range(nvar):
            d = WL.gpu_laplace_f32(torch, (d_out, d_in), scales[v],
                                   WL.substream_seed(config, 0, name, v, "delta"))
            alpha = torch.empty(1, dtype=torch.float32, device="cuda")
            tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
            bd.compress(d, None, alpha, tiled=tiled)
            variants.append((None, alpha, tiled))
            dh = d.cpu().numpy()
            del d
            a_ref = O.alpha_ref(dh)
            a_gpu = float(alpha.item())
            assert abs(a_gpu - float(a_ref)) <= 1e-6 * abs(float(a_ref)), (name, v, a_gpu, a_ref)
            # the oracle's compressed form of the sampled rows: their sign words and alpha
            ref.append((O.pack_signs_ref(O.signs_ref(dh[rows])), a_ref))
            del dh
        y = torch.empty((m, d_out), dtype=torch.bfloat16, device="cuda")
        layers.append((name, d_out, d_in, w, x, y, variants, rows, ref))
    # zeroed: its statistics word only ever grows (below: K-split handoffs across XCDs)
    ws = torch.zeros(sum(bd.matmul_workspace_bytes(m, d_in, "auto") for _, _, d_in, *_ in layers),
                     dtype=torch.uint8, device="cuda")
    probs = [(x, w, y, variants) for _, _, _, w, x, y, variants, _, _ in layers]
    assert bd.auto_path(m, offs, segv) == bd.PATHS["split"]
    bd.matmul_grouped(probs, offs, segv, workspace=ws)                      # bf16, as bench.py
    y32 = [torch.empty((m, d_out), dtype=torch.float32, device="cuda") for _, d_out, *_ in layers]
    bd.matmul_grouped([(x, w, yy, v) for (x, w, _, v), yy in zip(probs, y32)], offs, segv,
                      out_dtype="f32", workspace=ws)
    torch.cuda.synchronize()
    # each XCD serves its own run of the block's row blocks, and every split unit's pieces are on
    # one XCD's list: the first statistics block (past the activation parts, partial slots and
    # counters of all seven linears) counts handoffs whose pieces ran on several XCDs
    nstat = ws.numel() - len(layers) * 256
    stats = ws[nstat:nstat + 4].view(torch.int32).item()
    print(f"  split handoffs across XCDs: {stats}", flush=True)
    assert stats == 0

    worst = {}  # per output type: the largest row rel L2 and error / |delta term| over the block
    for (name, d_out, d_in, w, x, y, variants, rows, ref), yf in zip(layers, y32):
        wf = w[rows].float().cpu().numpy().astype(np.float64)
        xf = x.float().cpu().numpy().astype(np.float64)        # x is in segment order already
        got16 = y.float().cpu().numpy().astype(np.float64)[:, rows]
        got32 = yf.cpu().numpy().astype(np.float64)[:, rows]
        for s in range(len(segv)):
            v = int(segv[s])
            toks = np.arange(offs[s], offs[s + 1])
            words_r, a_ref = ref[v]
            y_ref = O.fused_linear_ref(xf[toks], wf, words_r, a_ref)
            delta_term = O.fused_linear_ref(xf[toks], np.zeros_like(wf), words_r, a_ref)
            for kind, got, row_tol, res_tol in (("bf16", got16[toks], 2e-2, 0.75),
                                                ("f32", got32[toks], 5e-3, 1e-2)):
                err = np.linalg.norm(got - y_ref, axis=1)
                rel = (err / np.linalg.norm(y_ref, axis=1)).max()
                res = (err / np.linalg.norm(delta_term, axis=1)).max()
                assert rel <= row_tol, (name, v)
                assert res <= res_tol, (name, v)
                w0 = worst.get(kind, (0.0, 0.0))
                worst[kind] = (max(w0[0], rel), max(w0[1], res))
    for kind, (rel, res) in worst.items():
        print(f"  {kind} output: max row rel L2 {rel:.3e}, max error / |delta term| {res:.3e}",
              flush=True)


def _check_rows(got, ref, delta_term, row_tol, res_tol, what):
    err = np.linalg.norm(got - ref, axis=1)
    rel = err / np.linalg.norm(ref, axis=1)
    res = err / np.linalg.norm(delta_term, axis=1)
    assert rel.max() <= row_tol, (what, "row rel L2", float(rel.max()))
    assert res.max() <= res_tol, (what, "delta residual", float(res.max()))


def test_full_size_gemv_one_token():
    """One token through the 8192 x 28672 down projection with one variant (the GEMV path, as
    bench.py --config 2 times it): 256 sampled output rows against the oracle, alpha over the
    whole Delta."""
    config, name, d_out, d_in = 2, "down", 8192, 28672
    rng = np.random.default_rng(1002)
    w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, 0, name, "w"))
    d = WL.gpu_laplace_f32(torch, (d_out, d_in), 2e-4, WL.substream_seed(config, 0, name, 0, "delta"))
    words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    bd.compress(d, words, alpha)
    ids = WL.decode_token_ids(config, 1, 1, "uniform")
    perm, offs, segv = bd.plan_segments(ids, 1)
    x = WL.gpu_normal_bf16(torch, (1, d_in), 1.0, WL.substream_seed(config, 0, name, "x"))
    assert bd.auto_path(1, offs, segv) == bd.PATHS["gemv"]
    y16 = bd.matmul(x, w, [(words, alpha)], offs, segv)
    y32 = bd.matmul(x, w, [(words, alpha)], offs, segv, out_dtype="f32")
    torch.cuda.synchronize()

    dh = d.cpu().numpy()
    del d
    a_ref = O.alpha_ref(dh)
    assert abs(float(alpha.item()) - float(a_ref)) <= 1e-6 * abs(float(a_ref))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, d_out - 2, d_out - 1],
                                     rng.choice(d_out, size=250, replace=False)]))
    s_rows = O.signs_ref(dh[rows]).astype(np.float64)
    np.testing.assert_array_equal(words[rows].cpu().numpy().view(np.uint32),
                                  O.pack_signs_ref(O.signs_ref(dh[rows])))
    wf = w[rows].float().cpu().numpy().astype(np.float64)
    xf = x.float().cpu().numpy().astype(np.float64)
    ref = xf @ (wf + np.float64(a_ref) * s_rows).T
    delta_term = np.float64(a_ref) * (xf @ s_rows.T)
    # the sampled outputs of the one token form its "row" here
    _check_rows(y16.float().cpu().numpy().astype(np.float64)[:, rows], ref, delta_term, 2e-2, 0.75,
                "bf16")
    _check_rows(y32.cpu().numpy().astype(np.float64)[:, rows], ref, delta_term, 1e-5, 1e-2, "f32")


def test_full_size_prefill_sampled():
    """The gate projection (28672 x 8192) over 4 requests x 2048 tokens on 4 of 14 resident
    variants, on the prefill path as bench.py --config 4 times it: 8 tokens of every segment on
    24 sampled output rows against the oracle."""
    config, name, d_out, d_in, nvar = 4, "gate", 28672, 8192, 14
    rng = np.random.default_rng(1004)
    scales = WL.decode_variant_scales(config)
    req_var = WL.prefill_request_variants(config, 4, nvar)
    ids = np.repeat(req_var, 2048).astype(np.int32)
    perm, offs, segv = bd.plan_segments(ids, nvar)
    m = ids.size
    w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, 0, name, "w"))
    x = WL.gpu_normal_bf16(torch, (m, d_in), 1.0, WL.substream_seed(config, 0, name, "x"))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, d_out - 2, d_out - 1],
                                     rng.choice(d_out, size=18, replace=False)]))
    variants, checked = [], {}
    for v in range(nvar):
        d = WL.gpu_laplace_f32(torch, (d_out, d_in), scales[v], WL.substream_seed(config, 0, name, v, "delta"))
        words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
        alpha = torch.empty(1, dtype=torch.float32, device="cuda")
        bd.compress(d, words, alpha)
        variants.append((words, alpha))
        if v in set(int(r) for r in req_var):
            dh = d.cpu().numpy()
            a_ref = O.alpha_ref(dh)
            assert abs(float(alpha.item()) - float(a_ref)) <= 1e-6 * abs(float(a_ref)), v
            checked[v] = (a_ref, O.signs_ref(dh[rows]).astype(np.float64))
            del dh
        del d
    y16 = torch.empty((m, d_out), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((m, d_out), dtype=torch.float32, device="cuda")
    bd.matmul_grouped([(x, w, y16, variants)], offs, segv, path="prefill")
    bd.matmul_grouped([(x, w, y32, variants)], offs, segv, path="prefill", out_dtype="f32")
    torch.cuda.synchronize()

    wf = w[rows].float().cpu().numpy().astype(np.float64)
    for sgi, v in enumerate(segv):
        lo, hi = int(offs[sgi]), int(offs[sgi + 1])
        toks = np.unique(np.concatenate([[lo, lo + 1, hi - 2, hi - 1], rng.integers(lo, hi, size=4)]))
        a_ref, s_rows = checked[int(v)]
        xf = x[toks].float().cpu().numpy().astype(np.float64)
        ref = xf @ (wf + np.float64(a_ref) * s_rows).T
        delta_term = np.float64(a_ref) * (xf @ s_rows.T)
        got16 = y16[toks][:, rows].float().cpu().numpy().astype(np.float64)
        got32 = y32[toks][:, rows].cpu().numpy().astype(np.float64)
        _check_rows(got16, ref, delta_term, 2e-2, 0.75, ("bf16", int(v)))
        _check_rows(got32, ref, delta_term, 5e-3, 0.75, ("f32", int(v)))


def test_full_size_compress_rows():
    """Per-row alphas at the down-projection shape (8192 x 28672, 28 column groups per row):
    every sign word against the oracle, and the alpha of 64 sampled rows (the first, the last
    and 62 seeded ones) against the oracle's exact row mean."""
    d_out, d_in = 8192, 28672
    delta = WL.gpu_laplace_f32(torch, (d_out, d_in), 3e-4, WL.substream_seed(6, 0, "down", 0, "delta"))
    words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
    alpha = torch.empty(d_out, dtype=torch.float32, device="cuda")
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    bd.compress_rows(delta, words, alpha, tiled=tiled)
    torch.cuda.synchronize()
    d_host = delta.cpu().numpy()
    ref_words = O.pack_signs_ref(O.signs_ref(d_host))
    np.testing.assert_array_equal(words.cpu().numpy().view(np.uint32), ref_words)
    rows = np.unique(np.concatenate([[0, d_out - 1],
                                     np.random.default_rng(80).integers(0, d_out, size=62)]))
    ref_a = O.alpha_rows_ref(d_host[rows]).astype(np.float64)
    got_a = alpha.cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.abs(got_a - ref_a) <= 1e-6 * ref_a)
    got_t = tiled.cpu().numpy().view(np.uint32).reshape(-1, 512)
    np.testing.assert_array_equal(got_t[0].reshape(128, 4), ref_words[:128, :4])


def test_full_size_compress_from_weights():
    """Compress from a (fine-tuned, base) bf16 pair at a 70B shape (8192 x 8192, the q / o
    projection): every sign word and alpha against the oracle's task vector."""
    d_out, d_in = 8192, 8192
    base = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(6, 0, "q", "w"))
    delta = WL.gpu_laplace_f32(torch, (d_out, d_in), 3e-4, WL.substream_seed(6, 0, "q", 0, "delta"))
    ft = (base.float() + delta).to(torch.bfloat16)
    del delta
    words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    bd.compress_from_weights(ft, base, words, alpha, tiled=tiled)
    torch.cuda.synchronize()
    ft_bits = ft.view(torch.int16).cpu().numpy().view(np.uint16)
    base_bits = base.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_words, ref_alpha = O.compress_from_weights_ref(ft_bits, base_bits)
    np.testing.assert_array_equal(words.cpu().numpy().view(np.uint32), ref_words)
    assert abs(float(alpha.item()) - float(ref_alpha)) <= 1e-6 * float(ref_alpha)
    got_t = tiled.cpu().numpy().view(np.uint32).reshape(-1, 512)
    # block (0, 0) of the tiled copy: rows 0..127, words 0..3 of each
    np.testing.assert_array_equal(got_t[0].reshape(128, 4), ref_words[:128, :4])
