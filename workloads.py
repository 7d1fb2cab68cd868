"""Seeded synthetic inputs for the BitDelta hot path.

This module is shared by the tests, the smoke check and the benchmark.  It only draws random
numbers and lays them out (weights, deltas, activations, per-token variant ids); it holds none
of the method's arithmetic (no alpha, no sign packing, no products).

Distributions follow the workloads the BitDelta post's serving setup implies (70B-shaped
linears, 14 fine-tuned variants, deltas modelled as Laplace(0, b) in "The mathematical
foundation"):

* base weights: N(0, 0.02) drawn in float32, rounded to bf16 (round-to-nearest-even);
* deltas: Laplace(0, b) in float32 (optionally with a fraction of exact +0.0);
* activations: N(0, 1) rounded to bf16;
* variant ids: uniform, truncated Zipf, or one distinct variant per request.

Small cases use numpy's default_rng on the CPU; full-size cases (too large to draw on the host)
are drawn on the GPU with torch's seeded generator, one independent stream per tensor.
"""
from __future__ import annotations

import hashlib

import numpy as np

# 70B-class decoder block: (name, d_out, d_in)
BLOCK_LINEARS = (
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def substream_seed(*key) -> int:
    """Independent 63-bit seed for a (config, block, linear, variant, tensor) key."""
    h = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def zipf_probs(num: int, s: float) -> np.ndarray:
    """Truncated Zipf over ranks 1..num: P(k) proportional to k^-s."""
    p = np.arange(1, num + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def variant_ids(rng: np.random.Generator, m: int, num_variants: int, dist: str, zipf_s: float = 1.1):
    if dist == "uniform":
        return rng.integers(0, num_variants, size=m).astype(np.int32)
    if dist == "zipf":
        return rng.choice(num_variants, size=m, p=zipf_probs(num_variants, zipf_s)).astype(np.int32)
    raise ValueError(dist)


# ---------------------------------------------------------------------------------------------
# CPU (numpy) cases
# ---------------------------------------------------------------------------------------------

def config1():
    """One 256x512 matrix, seed 0, draw order W_base, Delta, zero mask, x.  W ~ N(0, 0.02),
    Delta ~ Laplace(0, 1e-3) with 1% exact +0.0, x 4x512 ~ N(0, 1), one variant."""
    rng = np.random.default_rng(0)
    w = f32_to_bf16_bits(rng.normal(0.0, 0.02, size=(256, 512)).astype(np.float32))
    delta = rng.laplace(0.0, 1e-3, size=(256, 512)).astype(np.float32)
    zero = rng.random(size=(256, 512)) < 0.01
    delta[zero] = np.float32(0.0)
    x = f32_to_bf16_bits(rng.normal(0.0, 1.0, size=(4, 512)).astype(np.float32))
    return {"w": w, "deltas": [delta], "x": x, "token_variant": np.zeros(4, dtype=np.int32)}


def linear_case(seed: int, d_out: int, d_in: int, m: int, num_variants: int,
                b_range=(1e-4, 5e-4), dist: str = "uniform", zero_frac: float = 0.0,
                base_frac: float = 0.0, w_std: float = 0.02):
    """A generic segmented-batch case on the CPU.  Returns bf16 bit arrays for W and x, float32
    deltas, per-variant Laplace scales and per-token variant ids (``base_frac`` of the tokens
    are routed to the base model, id -1)."""
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits(rng.normal(0.0, w_std, size=(d_out, d_in)).astype(np.float32))
    scales = rng.uniform(b_range[0], b_range[1], size=num_variants)
    deltas = []
    for v in range(num_variants):
        d = rng.laplace(0.0, scales[v], size=(d_out, d_in)).astype(np.float32)
        if zero_frac > 0:
            d[rng.random(size=d.shape) < zero_frac] = np.float32(0.0)
        deltas.append(d)
    x = f32_to_bf16_bits(rng.normal(0.0, 1.0, size=(m, d_in)).astype(np.float32))
    ids = variant_ids(rng, m, num_variants, dist) if num_variants > 0 else np.full(m, -1, np.int32)
    if base_frac > 0:
        ids = np.where(rng.random(size=m) < base_frac, -1, ids).astype(np.int32)
    return {"w": w, "deltas": deltas, "x": x, "token_variant": ids, "scales": scales}


# ---------------------------------------------------------------------------------------------
# GPU (torch) draws for full-size cases; torch is only used as a seeded random source here.
# ---------------------------------------------------------------------------------------------

def _gen(torch, device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def gpu_normal_bf16(torch, shape, std, seed, device="cuda"):
    """N(0, std) drawn in float32 on the device and rounded to bf16 (torch rounds to nearest
    even)."""
    g = _gen(torch, device, seed)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t.to(torch.bfloat16)


def gpu_laplace_f32(torch, shape, b, seed, device="cuda", out=None):
    """Laplace(0, b) in float32 as b * (E1 - E2) with E1, E2 iid Exp(1) (the difference of two
    independent unit exponentials is a unit Laplace variable).  ``out`` may be a preallocated
    float32 buffer of the same number of elements."""
    g = _gen(torch, device, seed)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    else:
        out = out.view(shape)
    out.exponential_(1.0, generator=g)
    e2 = torch.empty_like(out).exponential_(1.0, generator=g)
    out.sub_(e2).mul_(float(b))
    del e2
    return out


def decode_variant_scales(config: int, num_variants: int = 14):
    rng = np.random.default_rng(substream_seed(config, "scales"))
    return rng.uniform(1e-4, 5e-4, size=num_variants)


def decode_token_ids(config: int, m: int, num_variants: int, dist: str):
    rng = np.random.default_rng(substream_seed(config, "ids"))
    return variant_ids(rng, m, num_variants, dist)


def prefill_request_variants(config: int, requests: int, num_variants: int):
    rng = np.random.default_rng(substream_seed(config, "requests"))
    return rng.choice(num_variants, size=requests, replace=False).astype(np.int32)
