"""CPU oracle for the BitDelta hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
anything from this package.  The product library (``tenant_serving_bitdelta_amd``) never imports,
links or executes it, and shares no code, table or helper with it.

Source of truth: the hanzo blog post "BitDelta: serving 14 Zen models from one GPU cluster"
(2026-02-28, published in five translations with identical content; called "the BitDelta post"
below).  Every function cites the section of that post it follows.
"""
from .bitdelta_oracle import (  # noqa: F401
    alpha_ref,
    signs_ref,
    pack_signs_ref,
    unpack_signs_ref,
    compress_ref,
    packed_nbytes_ref,
    reconstruct_ref,
    fused_linear_ref,
    plan_segments_ref,
    matmul_ref,
    matmul_bruteforce,
    bf16_bits_to_f64,
)
