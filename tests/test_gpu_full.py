"""Parity at full size, in the launch configuration bench.py times: one 70B decoder block (q, k,
v, o, gate, up, down), 14 variants compressed on the GPU, one grouped decode launch (the split
path for these batch sizes) with a caller workspace.  The oracle cannot multiply the whole block
quickly, so it checks every token of two variants on 24 sampled output rows of each linear,
with alpha computed by the oracle over the whole Delta."""
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
    counts = np.bincount(ids, minlength=nvar)
    present = [v for v in range(nvar) if counts[v] > 0]
    check_vars = sorted({max(present, key=lambda v: counts[v]), min(present, key=lambda v: counts[v])})
    rng = np.random.default_rng(1000 + config)

    layers = []
    for name, d_out, d_in in WL.BLOCK_LINEARS:
        w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, 0, name, "w"))
        x = WL.gpu_normal_bf16(torch, (m, d_in), 1.0, WL.substream_seed(config, 0, name, "x"))
        variants, deltas_checked = [], {}
        for v in range(nvar):
            d = WL.gpu_laplace_f32(torch, (d_out, d_in), scales[v],
                                   WL.substream_seed(config, 0, name, v, "delta"))
            words = torch.empty((d_out, d_in // 32), dtype=torch.int32, device="cuda")
            alpha = torch.empty(1, dtype=torch.float32, device="cuda")
            tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
            bd.compress(d, words, alpha, tiled=tiled)
            variants.append((words, alpha, tiled))
            if v in check_vars:
                deltas_checked[v] = d.cpu().numpy()
            del d
        y = torch.empty((m, d_out), dtype=torch.bfloat16, device="cuda")
        layers.append((name, d_out, d_in, w, x, y, variants, deltas_checked))
    ws = torch.empty(sum(bd.matmul_workspace_bytes(m, d_in, "auto") for _, _, d_in, *_ in layers),
                     dtype=torch.uint8, device="cuda")
    probs = [(x, w, y, variants) for _, _, _, w, x, y, variants, _ in layers]
    assert bd.auto_path(m, offs, segv) == bd.PATHS["split"]
    bd.matmul_grouped(probs, offs, segv, workspace=ws)                      # bf16, as bench.py
    y32 = [torch.empty((m, d_out), dtype=torch.float32, device="cuda") for _, d_out, *_ in layers]
    bd.matmul_grouped([(x, w, yy, v) for (x, w, _, v), yy in zip(probs, y32)], offs, segv,
                      out_dtype="f32", workspace=ws)
    torch.cuda.synchronize()

    for (name, d_out, d_in, w, x, y, variants, deltas), yf in zip(layers, y32):
        rows = _rows(d_out, rng)
        wf = w[rows].float().cpu().numpy().astype(np.float64)
        # x rows in segment order (x holds the batch in segment order already)
        xf = x.float().cpu().numpy().astype(np.float64)
        got16 = y.float().cpu().numpy().astype(np.float64)[:, rows]
        got32 = yf.cpu().numpy().astype(np.float64)[:, rows]
        for v in check_vars:
            d = deltas[v]
            a_ref = O.alpha_ref(d)
            a_gpu = float(variants[v][1].item())
            assert abs(a_gpu - float(a_ref)) <= 1e-6 * abs(float(a_ref)), (name, v)
            w_eff = wf + np.float64(a_ref) * O.signs_ref(d[rows]).astype(np.float64)
            toks = np.concatenate([np.arange(offs[s], offs[s + 1]) for s in range(len(segv))
                                   if segv[s] == v])
            ref = xf[toks] @ w_eff.T
            delta_term = np.float64(a_ref) * (xf[toks] @ O.signs_ref(d[rows]).astype(np.float64).T)
            for got, row_tol, res_tol in ((got16[toks], 2e-2, 0.75), (got32[toks], 5e-3, 1e-2)):
                err = np.linalg.norm(got - ref, axis=1)
                assert (err / np.linalg.norm(ref, axis=1)).max() <= row_tol, (name, v)
                assert (err / np.linalg.norm(delta_term, axis=1)).max() <= res_tol, (name, v)
