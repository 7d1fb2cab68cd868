"""The entry point that allocates nothing (bitdelta_matmul_grouped_noalloc, the SPLIT decode path
with the library's per-device scratch as its workspace) against bitdelta_matmul_grouped with a
caller workspace: two calls in a row, the second on a smaller batch, each bit for bit equal to
the workspace entry point (the same kernels and the same launch plan), plus the error cases it
rejects before enqueuing anything."""
import numpy as np
import pytest

import workloads as WL
from parity import bf16_dev, f32_dev

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


def _batch(seed, shapes, m, nv, dist, out_dtype):
    """Linears of the given shapes with nv tiled-only variants each, activations of m tokens in
    segment order, and two output tensors per linear (one per entry point)."""
    rng = np.random.default_rng(seed)
    ids = WL.variant_ids(rng, m, nv, dist)
    ids[rng.random(m) < 0.1] = -1
    perm, offs, segv = bd.plan_segments(ids, nv)
    ydt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    probs_a, probs_b = [], []
    for d_out, d_in in shapes:
        w = bf16_dev(WL.f32_to_bf16_bits(rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)))
        x = bf16_dev(WL.f32_to_bf16_bits(rng.normal(size=(m, d_in)).astype(np.float32)))
        variants = []
        for _ in range(nv):
            d = f32_dev(rng.laplace(0, rng.uniform(1e-4, 5e-4), size=(d_out, d_in)).astype(np.float32))
            tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
            alpha = torch.empty(1, dtype=torch.float32, device="cuda")
            bd.compress(d, None, alpha, tiled=tiled)
            variants.append((None, alpha, tiled))
        probs_a.append((x, w, torch.full((m, d_out), 7.0, dtype=ydt, device="cuda"), variants))
        probs_b.append((x, w, torch.full((m, d_out), -7.0, dtype=ydt, device="cuda"), variants))
    return probs_a, probs_b, offs, segv


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(out_dtype):
    calls = [
        # a 256-token batch over 14 variants and four linears (about 100 MB of scratch)
        (71, [(1024, 8192), (256, 8192), (2048, 4096), (512, 12288)], 256, 14, "zipf"),
        # then a smaller one: 40 tokens, 3 variants, two linears
        (72, [(640, 2048), (136, 1024)], 40, 3, "uniform"),
    ]
    for seed, shapes, m, nv, dist in calls:
        need = sum(bd.matmul_workspace_bytes(m, d_in, "split") for _, d_in in shapes)
        assert need <= bd.NOALLOC_SCRATCH_BYTES
        pa, pb, offs, segv = _batch(seed, shapes, m, nv, dist, out_dtype)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        bd.matmul_grouped(pa, offs, segv, out_dtype=out_dtype, path="split", workspace=ws)
        bd.matmul_grouped_noalloc(pb, offs, segv, out_dtype=out_dtype, path="auto")
        torch.cuda.synchronize()
        for (_, _, ya, _), (_, _, yb, _) in zip(pa, pb):
            assert torch.isfinite(ya.float()).all()
            assert torch.equal(ya, yb), (seed, out_dtype)


def test_noalloc_rejects_before_enqueuing():
    # eight linears of width 28672 at 256 tokens need about 350 MB: more than the scratch holds
    m, d_out, d_in = 256, 128, 28672
    assert 8 * bd.matmul_workspace_bytes(m, d_in, "split") > bd.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((m, d_in), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((d_out, d_in), dtype=torch.bfloat16, device="cuda")
    y = torch.full((m, d_out), 3.0, dtype=torch.bfloat16, device="cuda")
    tiled = torch.zeros(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    alpha = torch.zeros(1, dtype=torch.float32, device="cuda")
    var = [(None, alpha, tiled)]
    offs, segv = [0, 100, m], [-1, 0]
    with pytest.raises(bd.BitDeltaError) as err:
        bd.matmul_grouped_noalloc([(x, w, y, var)] * 8, offs, segv)
    assert err.value.status == 4
    # a batch AUTO sends to another path (3 tokens: GEMV), or a forced non-split path
    with pytest.raises(bd.BitDeltaError) as err:
        bd.matmul_grouped_noalloc([(x[:3], w, y[:3], var)], [0, 3], [0])
    assert err.value.status == 5
    with pytest.raises(bd.BitDeltaError) as err:
        bd.matmul_grouped_noalloc([(x, w, y, var)], offs, segv, path="stream")
    assert err.value.status == 5
    # a variant without the tiled words
    words = torch.zeros((d_out, d_in // 32), dtype=torch.int32, device="cuda")
    with pytest.raises(bd.BitDeltaError) as err:
        bd.matmul_grouped_noalloc([(x, w, y, [(words, alpha, None)])], offs, segv)
    assert err.value.status == 5
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)  # nothing ran
