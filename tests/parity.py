"""Shared helpers of the GPU parity tests: moving seeded inputs to the device, running the
library through its C ABI, and the error metrics the tolerances are stated in."""
import numpy as np

import oracle.bitdelta_oracle as O

# Per token row of y: ||y_gpu - y_ref||_2 / ||y_ref||_2 (fp64 oracle); the stated bound.
ROW_L2_TOL = 2e-2
# bf16 output: the error must stay well below the size of the delta term itself, so a kernel
# that dropped or flipped the delta (ratio ~1 or ~2) cannot pass.
DELTA_RESIDUAL_TOL_BF16 = 0.75


def torch_mod():
    import torch
    return torch


def bf16_dev(bits, dev="cuda"):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def f32_dev(a, dev="cuda"):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def words_host(words_t):
    return words_t.cpu().numpy().view(np.uint32)


def row_rel_l2(y, y_ref):
    num = np.linalg.norm(y - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    return num / np.maximum(den, 1e-300)


def delta_residual(y, y_ref, y_delta):
    """Per row ||y - y_ref|| / ||y_delta|| for rows whose delta term is nonzero."""
    dn = np.linalg.norm(y_delta, axis=1)
    keep = dn > 0
    return np.linalg.norm(y - y_ref, axis=1)[keep] / dn[keep]


def oracle_delta_term(x, variants, seg_offsets, seg_variant, d_out, d_in):
    """alpha_v * x S_v^T per segment (the part of y the sign bits contribute), fp64."""
    y = np.zeros((x.shape[0], d_out))
    for s, v in enumerate(seg_variant):
        lo, hi = seg_offsets[s], seg_offsets[s + 1]
        if v < 0 or hi <= lo:
            continue
        words, alpha = variants[v]
        sgn = O.unpack_signs_ref(words, d_in).astype(np.float64)
        a = np.asarray(alpha, dtype=np.float32).astype(np.float64)  # scalar or one per row
        y[lo:hi] = (x[lo:hi] @ sgn.T) * (a if a.ndim == 0 else a[None, :])
    return y


def gpu_compress(deltas_np, dev="cuda"):
    """Compress every delta on the device; returns [(words_t, alpha_t, tiled_t)] where tiled_t is
    the tiled copy of the sign words (None when d_in is not a multiple of 128)."""
    import tenant_serving_bitdelta_amd as bd
    torch = torch_mod()
    out = []
    for d in deltas_np:
        dt = f32_dev(d, dev)
        words = torch.empty((d.shape[0], d.shape[1] // 32), dtype=torch.int32, device=dev)
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
        nt = bd.sign_words_t128(d.shape[0], d.shape[1])
        tiled = torch.empty(nt, dtype=torch.int32, device=dev) if nt > 0 else None
        bd.compress(dt, words, alpha, tiled=tiled)
        out.append((words, alpha, tiled))
    return out


def tile_words_128(words, d_out, d_in):
    """Row-major sign words [d_out][d_in/32] -> the 128-row tiled order (padding rows zero): word
    (r, c) goes to ((r // 128) * (d_in // 128) + c // 4) * 512 + (r % 128) * 4 + c % 4."""
    wpr = d_in // 32
    nrb = (d_out + 127) // 128
    out = np.zeros(nrb * 128 * wpr, dtype=np.uint32)
    r = np.arange(d_out)[:, None]
    c = np.arange(wpr)[None, :]
    idx = ((r // 128) * (d_in // 128) + c // 4) * 512 + (r % 128) * 4 + c % 4
    out[idx.ravel()] = np.asarray(words, dtype=np.uint32).reshape(d_out, wpr).ravel()
    return out
