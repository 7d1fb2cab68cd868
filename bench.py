"""Benchmark of the BitDelta hot path on one MI355X.

Default workload (headline): a stack of 20 decoder blocks of a 70B-class model (q, o 8192x8192;
k, v 1024x8192; gate, up 28672x8192; down 8192x28672), 14 fine-tuned variants resident as
1-bit deltas.  Set-up compresses all 14 x 140 deltas on the GPU (alpha + sign packing,
Laplace(0, b) deltas drawn per matrix and discarded), then a step is one decode pass of a
256-token batch whose variant ids follow a truncated Zipf(1.1) over the 14 variants: the
segment plan plus one grouped fused reconstruct-and-multiply launch per block over its seven
linears (independent synthetic activations per linear).

Prints ONE JSON line on stdout; progress goes to stderr.  The default run also measures, after
the headline and reported under "sub_results", the other workloads with their own rooflines:
one down_proj GEMV (1 token, 1 variant; weights rotated over copies that together exceed the
memory-side cache), one block with a 64-token uniform batch, the prefill of gate and up with
4 requests x 2048 tokens on 4 of 14 variants, the unfused comparison (W_eff written to HBM,
then a plain product) for the last two, and a device-to-device copy as the measured bandwidth
ceiling.  --config N runs one workload alone (2, 3, 4 or 5).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as WL  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
NUM_VARIANTS = 14


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=None, choices=(2, 3, 4, 5),
                   help="run one workload alone (default: the headline plus every sub-result)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the HIP-graph replay timing of the decode block / step workloads")
    p.add_argument("--no-sub", action="store_true", help="default run: the headline only")
    p.add_argument("--unfused", action="store_true",
                   help="--config 3 or 4: also time the unfused comparison")
    p.add_argument("--path", default="auto", choices=("auto", "gemv", "stream", "split", "prefill"),
                   help="decode kernel family (auto: what the library picks)")
    p.add_argument("--alpha-rows", action="store_true",
                   help="decode configs: compress every variant with one alpha per output row")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy a 1 GiB device buffer three times (a plain copy kernel of known "
                        "size, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


# ---------------------------------------------------------------------------------------------
# measured HBM traffic of the split kernel (rocprofv3 counters, summarised under profiles/)
# ---------------------------------------------------------------------------------------------

TRAFFIC_PROFILE = os.path.join(ROOT, "profiles",
                               "split_kernel__decode_20x70b_m256_14var__hbm_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "tenant_serving_bitdelta_amd", "csrc", f)
                   for f in ("split.hip", "split_sched.cpp", "bd_internal.h", "api.cpp")]


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when the split-path
    sources changed since the counters were taken (or there is no summary)."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    sha = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val or sha.group(1) != sources_sha256():
        return None
    return int(val.group(1))


def copy_calibration(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_calibration": {"bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 3}}


# ---------------------------------------------------------------------------------------------
# workload construction (device memory via torch; all compute in libbitdelta)
# ---------------------------------------------------------------------------------------------

class Linear:
    def __init__(self, name, d_out, d_in):
        self.name, self.d_out, self.d_in = name, d_out, d_in
        self.w = None
        self.variants = []
        self.x = None
        self.y = None


def build_layers(torch, bd, config, blocks, linears, scales, compress_timer, nvar=NUM_VARIANTS,
                 alpha_rows=False):
    dev = "cuda"
    maxn = max(d_out * d_in for _, d_out, d_in in linears)
    dbuf = torch.empty(maxn, dtype=torch.float32, device=dev)
    ws_bytes = max(max(bd.compress_workspace_bytes(d_out, d_in),
                       bd.compress_rows_workspace_bytes(d_out, d_in)) for _, d_out, d_in in linears)
    ws = torch.empty(max(ws_bytes, 8) // 8, dtype=torch.float64, device=dev)
    layers = []
    for b in range(blocks):
        blk = []
        for name, d_out, d_in in linears:
            L = Linear(name, d_out, d_in)
            L.w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, b, name, "w"))
            for v in range(nvar):
                delta = WL.gpu_laplace_f32(torch, (d_out, d_in), scales[v],
                                           WL.substream_seed(config, b, name, v, "delta"),
                                           out=dbuf[:d_out * d_in])
                # one resident layout per variant: the tiled words the kernels stream (the
                # row-major words only where d_in % 128 != 0)
                nt = bd.sign_words_t128(d_out, d_in)
                tiled = torch.empty(nt, dtype=torch.int32, device=dev) if nt > 0 else None
                words = (None if tiled is not None else
                         torch.empty((d_out, d_in // 32), dtype=torch.int32, device=dev))
                alpha = torch.empty(d_out if alpha_rows else 1, dtype=torch.float32, device=dev)
                compress_timer.start()
                if alpha_rows:
                    bd.compress_rows(delta, words, alpha, workspace=ws, tiled=tiled)
                else:
                    bd.compress(delta, words, alpha, workspace=ws, tiled=tiled)
                # reads Delta once, writes the sign words (one layout) and alpha
                compress_timer.stop(4 * d_out * d_in + d_out * d_in // 8 + 4 * alpha.numel())
                L.variants.append((words, alpha, tiled))
            blk.append(L)
        layers.append(blk)
        log(f"[setup] block {b + 1}/{blocks} built and compressed")
    del dbuf
    return layers


class EventTimer:
    """Sums kernel durations between pairs of HIP events on torch's current stream.  Events are
    created ahead (``reserve``) so that creating them costs nothing inside a timed loop."""

    def __init__(self, torch, reserve=0):
        self.torch = torch
        self.pairs = []
        self.bytes = 0
        self._spare = [self._new() for _ in range(2 * reserve)]

    def _new(self):
        return self.torch.cuda.Event(enable_timing=True)

    def _event(self):
        return self._spare.pop() if self._spare else self._new()

    def start(self):
        e = self._event()
        e.record()
        self._open = e

    def stop(self, nbytes=0):
        e = self._event()
        e.record()
        self.pairs.append((self._open, e))
        self.bytes += nbytes

    def durations_ms(self):
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.pairs]

    def total_ms(self):
        return sum(self.durations_ms())


def spread(values, scale=1.0):
    """Median, p10 and p90 of ``values`` (times ``scale``)."""
    v = np.asarray(values, dtype=np.float64) * scale
    if v.size == 0:
        return None
    return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
            "p90": float(np.percentile(v, 90)), "n": int(v.size)}


def measure_graph_step(args, torch, run_step, outputs, tokens, checks=3):
    """One whole step (every grouped call of it) captured once into a HIP graph and replayed.
    Each of ``checks`` replays is compared bit for bit with an eager step, with the outputs
    cleared and the eager step run between replays; then ``args.steps`` replays are timed, each
    between HIP events, and their wall time over the lot gives tokens/s."""
    run_step()
    torch.cuda.synchronize()
    ref = [y.clone() for y in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_step()
    torch.cuda.synchronize()
    equal = True
    for _ in range(checks):
        for y in outputs:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        equal = equal and all(torch.equal(y, r) for y, r in zip(outputs, ref))
        run_step()
        torch.cuda.synchronize()
        equal = equal and all(torch.equal(y, r) for y, r in zip(outputs, ref))
    for _ in range(args.warmup):
        g.replay()
    rt = EventTimer(torch, reserve=args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rt.start()
        g.replay()
        rt.stop()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    del g
    return {"tokens_per_s": tokens * 1e3 / ms, "ms_per_step": ms,
            "replay_ms": spread(rt.durations_ms()),
            "replays_checked": checks, "equal_to_eager": bool(equal)}


def measure_compress_pair(torch, bd, reps=5):
    """Compress from a (fine-tuned, base) bf16 pair at the gate / up shape (28672 x 8192): the
    task vector is never formed.  Algorithmic bytes: both matrices read (2 x 2 B per element),
    the sign words written in the kernels' (tiled) layout (n / 8) and alpha."""
    d_out, d_in = 28672, 8192
    base = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(6, 0, "gate", "w"))
    delta = WL.gpu_laplace_f32(torch, (d_out, d_in), 3e-4, WL.substream_seed(6, 0, "gate", 0, "delta"))
    ft = (base.float() + delta).to(torch.bfloat16)
    del delta
    words = None
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(bd.compress_workspace_bytes(d_out, d_in), 8) // 8, dtype=torch.float64,
                     device="cuda")
    for _ in range(2):
        bd.compress_from_weights(ft, base, words, alpha, workspace=ws, tiled=tiled)
    t = EventTimer(torch, reserve=reps)
    n = d_out * d_in
    for _ in range(reps):
        t.start()
        bd.compress_from_weights(ft, base, words, alpha, workspace=ws, tiled=tiled)
        t.stop(4 * n + n // 8 + 4)
    ms = t.total_ms() / reps
    gbs = t.bytes / reps / (ms / 1e3) / 1e9
    del base, ft, words, tiled, ws
    return {"shape": [d_out, d_in], "ms": ms, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS}


def measure_compress_rows(torch, bd, reps=5):
    """Compress with one alpha per output row at the gate / up shape (28672 x 8192).
    Algorithmic bytes: Delta read (4 B per element), the sign words written in the kernels'
    (tiled) layout (n / 8) and the d_out alphas."""
    d_out, d_in = 28672, 8192
    delta = WL.gpu_laplace_f32(torch, (d_out, d_in), 3e-4, WL.substream_seed(6, 0, "gate", 0, "delta"))
    words = None
    alpha = torch.empty(d_out, dtype=torch.float32, device="cuda")
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(bd.compress_rows_workspace_bytes(d_out, d_in), 8) // 8,
                     dtype=torch.float64, device="cuda")
    for _ in range(2):
        bd.compress_rows(delta, words, alpha, workspace=ws, tiled=tiled)
    t = EventTimer(torch, reserve=reps)
    n = d_out * d_in
    for _ in range(reps):
        t.start()
        bd.compress_rows(delta, words, alpha, workspace=ws, tiled=tiled)
        t.stop(4 * n + n // 8 + 4 * d_out)
    ms = t.total_ms() / reps
    gbs = t.bytes / reps / (ms / 1e3) / 1e9
    del delta, words, tiled, ws
    return {"shape": [d_out, d_in], "ms": ms, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS}


def measure_delta_upload(torch, bd, reps=8):
    """Cold start of a variant: its stored (row-major) sign words and scale moved from pinned host
    memory into the layout the kernels read, through bitdelta_upload_variant (a host-to-device
    copy, then the re-layout into the tiled words), timed with HIP events on torch's stream for
    the 28672 x 8192 gate projection, and the time this gives for a whole 70B variant (80 decoder
    blocks of q, k, v, o, gate, up, down).  The plain copy engine rate of 1 GiB pinned copies is
    reported beside it."""
    d_out, d_in = 28672, 8192
    nw = d_out * d_in // 32
    host_words = torch.randint(-2**31, 2**31 - 1, (nw,), dtype=torch.int32).pin_memory()
    host_alpha = torch.tensor([3e-4], dtype=torch.float32).pin_memory()
    tiled = torch.empty(bd.sign_words_t128(d_out, d_in), dtype=torch.int32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    staging = torch.empty(nw * 4, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        bd.upload_variant(host_words, host_alpha, d_out, d_in, tiled=tiled, alpha=alpha,
                          staging=staging)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        bd.upload_variant(host_words, host_alpha, d_out, d_in, tiled=tiled, alpha=alpha,
                          staging=staging)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = (nw * 4 + 4) / (ms / 1e3) / 1e9
    shapes = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192),
              (28672, 8192), (8192, 28672)]
    variant = 80 * sum(d_o * d_i // 8 + 4 for d_o, d_i in shapes)
    del host_words, tiled, staging
    # the copy engine alone: 1 GiB from pinned host memory
    nbytes = 1 << 30
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dev.copy_(host, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        dev.copy_(host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = nbytes / (e0.elapsed_time(e1) / 3 / 1e3) / 1e9
    del host, dev
    return {"source": "pinned host memory over PCIe, through bitdelta_upload_variant",
            "matrix": [d_out, d_in], "ms_per_matrix": ms, "gbs": gbs,
            "variant_bytes_70b": variant, "variant_ms": variant / (gbs * 1e9) * 1e3,
            "copy_engine_gbs_1gib": copy_gbs}


def measure_unfused(torch, bd, blk, offs, segv, path, steps, warmup):
    """The unfused comparison the post argues against ("Serving architecture": W_eff materialised
    in HBM against the fused kernel's bandwidth): for every linear and every variant segment of
    the batch, W_eff = bf16(W_base + alpha * sign) is written to HBM (bitdelta_reconstruct) and
    the segment's tokens are multiplied with it as a plain product (the base-model segment of
    bitdelta_matmul, W_eff given as the weights); base-model tokens use W_base directly.
    Algorithmic bytes per variant segment and linear: W_base and the sign words read and W_eff
    written (2n + n/8 + 2n), W_eff read again (2n), the segment's activations and outputs."""
    weff = {L.name: torch.empty((L.d_out, L.d_in), dtype=torch.bfloat16, device="cuda") for L in blk}
    m = int(offs[-1])
    ws = torch.empty(max(max(bd.matmul_workspace_bytes(m, L.d_in, path) for L in blk), 256),
                     dtype=torch.uint8, device="cuda")
    nbytes = 0
    for L in blk:
        n = L.d_out * L.d_in
        for s_i, v in enumerate(segv):
            ln = int(offs[s_i + 1] - offs[s_i])
            nbytes += (2 * n + n // 8 + 4 + 2 * n if v >= 0 else 0) + 2 * n + 2 * ln * (L.d_in + L.d_out)

    def step():
        for L in blk:
            for s_i, v in enumerate(segv):
                lo, hi = int(offs[s_i]), int(offs[s_i + 1])
                w = L.w
                if v >= 0:
                    w = bd.reconstruct(L.w, L.variants[int(v)], w_eff=weff[L.name])
                bd.matmul(L.x[lo:hi], w, [], [0, hi - lo], [-1], y=L.y[lo:hi], path=path,
                          workspace=ws)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    base_bytes = sum(2 * L.d_out * L.d_in for L in blk)
    del weff, ws
    return {"ms_per_step": ms, "tokens_per_s": m * 1e3 / ms, "bytes_per_step": nbytes,
            "gbs": nbytes / (ms / 1e3) / 1e9, "bytes_over_base_weights": nbytes / base_bytes,
            "launches_per_step": sum(len(segv) + int(np.sum(segv >= 0)) for _ in blk)}


def measure_unfused_decode(args, torch, bd, blk, ids, nvar, m, fused_launch_ms):
    _, offs, segv = bd.plan_segments(ids, nvar)
    r = measure_unfused(torch, bd, blk, offs, segv, args.path, max(3, args.steps // 4), 1)
    n_active = int(np.sum(segv >= 0))
    fused_bytes = decode_bytes(blk, m, n_active)
    r.update({"fused_ms_per_step": fused_launch_ms, "unfused_over_fused_time": r["ms_per_step"] / fused_launch_ms,
              "fused_bytes_per_step": fused_bytes,
              "fused_bytes_over_base_weights": fused_bytes / sum(2 * L.d_out * L.d_in for L in blk)})
    return r


def decode_bytes(blk, m, n_active, alpha_rows=False):
    tot = 0
    for L in blk:
        n = L.d_out * L.d_in
        tot += (2 * n + n_active * (n // 8 + 4 * (L.d_out if alpha_rows else 1)) + 2 * m * L.d_in +
                2 * m * L.d_out)
    return tot


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the same workload
# ---------------------------------------------------------------------------------------------

def cpu_baseline_decode(torch, config, linears_sample, scales, perm, offs, segv, m, total_elems, nvar):
    from oracle import bitdelta_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    elapsed, elems = 0.0, 0
    for name, d_out, d_in in linears_sample:
        # regenerate the sampled linear's inputs from the same seeds (device draw, host copy)
        w = WL.gpu_normal_bf16(torch, (d_out, d_in), 0.02, WL.substream_seed(config, 0, name, "w"))
        wf = w.float().cpu().numpy().astype(np.float64)
        variants = []
        for v in range(nvar):
            d = WL.gpu_laplace_f32(torch, (d_out, d_in), scales[v],
                                   WL.substream_seed(config, 0, name, v, "delta")).cpu().numpy()
            variants.append(O.compress_ref(d))
        x = WL.gpu_normal_bf16(torch, (m, d_in), 1.0, WL.substream_seed(config, 0, name, "x"))
        xf = x.float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        O.matmul_ref(xf, wf, variants, offs, segv)
        elapsed += time.perf_counter() - t0
        elems += d_out * d_in
        log(f"[cpu baseline] oracle on {name} ({d_out}x{d_in}): {elapsed:.1f}s so far")
    est_step = elapsed * total_elems / elems
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": m / est_step, "unit": "tokens/s", "cores": int(cores),
            "blas_threads": int(blas_threads), "extrapolated": True, "kind": "oracle",
            "sample": (f"oracle matmul of block 0's {'+'.join(n for n, _, _ in linears_sample)} "
                       f"({elems} weights, all {m} tokens, {nvar} variant(s)) in {elapsed:.1f}s on the host, "
                       f"scaled by weight count to the full step ({total_elems} weights); "
                       f"numpy elementwise on 1 thread, BLAS on {blas_threads}")}


# ---------------------------------------------------------------------------------------------

def run_decode(args, torch, bd, config, cpu_baseline=True, rotate=1, unfused=False):
    if config == 5:
        blocks, m, dist = 20, 256, "zipf"
        linears = list(WL.BLOCK_LINEARS)
    elif config == 3:
        blocks, m, dist = 1, 64, "uniform"
        linears = list(WL.BLOCK_LINEARS)
    else:  # config 2
        blocks, m, dist = 1, 1, "uniform"
        linears = [("down", 8192, 28672)]
    scales = WL.decode_variant_scales(config) if config != 2 else np.array([2e-4])
    nvar = NUM_VARIANTS if config != 2 else 1
    ids = WL.decode_token_ids(config, m, nvar, dist)
    perm, offs, segv = bd.plan_segments(ids, nvar)
    n_active = int(np.sum(segv >= 0))
    log(f"[setup] config {config}: {blocks} block(s), M={m}, segments={list(np.diff(offs))}")

    comp = EventTimer(torch)
    layers = build_layers(torch, bd, config, blocks, linears, scales, comp, nvar,
                          alpha_rows=args.alpha_rows)
    comp_ms = comp.total_ms()
    if rotate > 1:
        # copies of the block (weights and sign words) in distinct memory, so consecutive steps
        # never find their weights in the memory-side cache
        base = layers[0]
        for _ in range(rotate - 1):
            blk = []
            for L in base:
                C = Linear(L.name, L.d_out, L.d_in)
                C.w = L.w.clone()
                C.variants = [tuple(None if t is None else t.clone() for t in v) for v in L.variants]
                blk.append(C)
            layers.append(blk)
    for b, blk in enumerate(layers):
        for L in blk:
            L.x = WL.gpu_normal_bf16(torch, (m, L.d_in), 1.0, WL.substream_seed(config, b, L.name, "x"))
            L.y = torch.empty((m, L.d_out), dtype=torch.bfloat16, device="cuda")
    # one workspace for the whole step (blocks run one after another on one stream)
    ws_bytes = max(sum(bd.matmul_workspace_bytes(m, L.d_in, args.path) for L in blk) for blk in layers)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    step_blocks = [layers] if rotate == 1 else [[blk] for blk in layers]
    step_no = [0]

    def run_blocks(blocks_of_step, timer=None):
        # plan (host) + one grouped call per block (split path: activation prologue + main kernel)
        _, o, s = bd.plan_segments(ids, nvar)
        for blk in blocks_of_step:
            probs = [(L.x, L.w, L.y, L.variants) for L in blk]
            if timer:
                timer.start()
            bd.matmul_grouped(probs, o, s, path=args.path, workspace=ws)
            if timer:
                timer.stop()

    def step(timer=None, step_timer=None):
        if step_timer:
            step_timer.start()
        run_blocks(step_blocks[step_no[0] % len(step_blocks)], timer)
        if step_timer:
            step_timer.stop()
        step_no[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kt = EventTimer(torch, reserve=args.steps * len(layers))
    st = EventTimer(torch, reserve=args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(kt, st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = kt.durations_ms()
    kern_ms = sum(launch_ms)
    step_ms = st.durations_ms()
    graph = None
    if config in (3, 5) and not args.no_graph:
        try:
            graph = measure_graph_step(args, torch, lambda: run_blocks(step_blocks[0]),
                                       [L.y for blk in step_blocks[0] for L in blk], m)
        except Exception as e:  # capture not available: the eager timing stands
            graph = {"error": f"{type(e).__name__}: {e}"[:300]}
    # the decode block and the 20-block step are timed as one replayed HIP graph of the whole
    # step when its replays equal the eager outputs bit for bit; the eager timing is kept beside
    ms_eager = ms_step
    timing = "eager launches"
    if graph and graph.get("equal_to_eager"):
        ms_step = graph["ms_per_step"]
        timing = "HIP graph replay of the whole step (replays checked equal to eager, bit for bit)"
    launches = len(kt.pairs)
    bytes_launch = decode_bytes(layers[0], m, n_active, args.alpha_rows)  # every block has the same shapes
    avg_launch_s = kern_ms / launches / 1e3
    achieved = bytes_launch / avg_launch_s / 1e9
    total_elems = sum(L.d_out * L.d_in for blk in step_blocks[0] for L in blk)
    path = bd.auto_path(m, offs, segv) if args.path == "auto" else bd.PATHS[args.path]
    # compress from a weight pair, after the timed region (default workload only)
    pair = measure_compress_pair(torch, bd) if config == 5 else None
    rows = measure_compress_rows(torch, bd) if config == 5 else None
    upload = measure_delta_upload(torch, bd) if config == 5 else None
    unf = (measure_unfused_decode(args, torch, bd, layers[0], ids, nvar, m, kern_ms / launches)
           if unfused else None)
    resident_sign_bytes = sum(int(t.numel()) * 4 for blk in step_blocks[0] for L in blk
                              for v in L.variants for t in (v[0], v[2]) if t is not None)

    cpu = None
    if cpu_baseline and not args.no_cpu_baseline:
        sample = [l for l in linears if l[0] in ("q", "k", "v", "o", "gate")] or linears
        cpu = cpu_baseline_decode(torch, config, sample, scales, perm, offs, segv, m, total_elems,
                                  nvar)

    comp_bytes = comp.bytes
    names = {2: "down_proj GEMV 8192x28672, 1 token, 1 variant",
             3: "one 70B decoder block (7 linears), 64-token uniform batch, 14 variants",
             5: "20 x 70B decoder blocks (140 linears), 256-token Zipf(1.1) batch, 14 variants"}
    return {
        "metric": "fused BitDelta matmul tokens/s + achieved HBM GB/s (% peak), 14 variants",
        "value": m * 1e3 / ms_step,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "timing": timing,
        "eager": {"value": m * 1e3 / ms_eager, "ms_per_step": ms_eager},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {1: "bf16 in, fp32 arithmetic", 2: "bf16 MFMA (fp32 accumulate)",
                  4: "bf16 MFMA + fp4 x fp6 MFMA (fp32 accumulate)"}.get(path, "bf16"),
        "data": "synthetic (seeded; random weights/deltas)",
        "config": {"workload": names[config] + (", one alpha per output row" if args.alpha_rows else ""),
                   "config_index": config, "tokens_per_step": m,
                   "segments": [int(v) for v in np.diff(offs)], "active_variants": n_active,
                   "launches_per_step": launches // args.steps,
                   "kernel_path": {1: "gemv", 2: "stream", 3: "prefill", 4: "split"}[path],
                   "weight_copies_rotated": rotate,
                   "resident_sign_bytes": resident_sign_bytes,
                   "parallelism": "single GPU"},
        "hbm_gbs_step": bytes_launch * len(step_blocks[0]) / (ms_step / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if (config == 5 and path == 4) else None,
                     "kernel": {1: "gemv_kernel", 2: "stream_kernel",
                                4: "split_act_kernel + split_kernel"}.get(path, "?"),
                     "bytes_per_launch": bytes_launch, "avg_launch_us": avg_launch_s * 1e6,
                     "launch_us": spread(launch_ms, 1e3)},
        "step_ms": spread(step_ms),
        "graph": graph,
        "compress": {"matrices": len(comp.pairs), "bytes": comp_bytes, "ms": comp_ms,
                     "gbs": comp_bytes / (comp_ms / 1e3) / 1e9,
                     "frac": comp_bytes / (comp_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "compress_from_weights": pair,
        "compress_rows": rows,
        "delta_upload": upload,
        "unfused": unf,
        "cpu_baseline": cpu,
    }


def run_prefill(args, torch, bd, unfused=False):
    config = 4
    linears = [("gate", 28672, 8192), ("up", 28672, 8192)]
    scales = WL.decode_variant_scales(config)
    req_var = WL.prefill_request_variants(config, 4, NUM_VARIANTS)
    ids = np.repeat(req_var, 2048).astype(np.int32)
    perm, offs, segv = bd.plan_segments(ids, NUM_VARIANTS)
    m = ids.size
    comp = EventTimer(torch)
    layers = build_layers(torch, bd, config, 1, linears, scales, comp)[0]
    for L in layers:
        L.x = WL.gpu_normal_bf16(torch, (m, L.d_in), 1.0, WL.substream_seed(config, 0, L.name, "x"))
        L.y = torch.empty((m, L.d_out), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def step(timer=None):
        _, o, s = bd.plan_segments(ids, NUM_VARIANTS)
        probs = [(L.x, L.w, L.y, L.variants) for L in layers]
        if timer:
            timer.start()
        bd.matmul_grouped(probs, o, s, path="prefill")
        if timer:
            timer.stop()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kt = EventTimer(torch, reserve=args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(kt)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = kt.durations_ms()
    kern_ms = sum(launch_ms) / len(launch_ms)
    flops = sum(2.0 * m * L.d_out * L.d_in for L in layers)
    achieved = flops / (kern_ms / 1e3) / 1e12
    unf = None
    if unfused:
        unf = measure_unfused(torch, bd, layers, offs, segv, "prefill", max(2, args.steps // 4), 1)
        unf.update({"fused_ms_per_step": kern_ms, "unfused_over_fused_time": unf["ms_per_step"] / kern_ms,
                    "tflops_unfused": flops / (unf["ms_per_step"] / 1e3) / 1e12})
    return {
        "metric": "fused BitDelta matmul tokens/s (prefill, bf16 MFMA), 14 variants resident",
        "value": m * 1e3 / ms_step, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 MFMA (fp32 accumulate)",
        "data": "synthetic (seeded; random weights/deltas)",
        "config": {"workload": "prefill gate+up 28672x8192, 4 requests x 2048 tokens on 4 of 14 variants",
                   "config_index": 4, "tokens_per_step": m, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "prefill_kernel", "flops_per_launch": flops,
                     "avg_launch_us": kern_ms * 1e3, "launch_us": spread(launch_ms, 1e3)},
        "unfused": unf,
        "cpu_baseline": None,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); the BitDelta hot "
              "path here is single-GPU and multi-GPU runs are not part of this benchmark.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import tenant_serving_bitdelta_amd as bd
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)), flush=True)
        return
    if args.config == 4:
        res = run_prefill(args, torch, bd, unfused=args.unfused)
    elif args.config is not None:
        res = run_decode(args, torch, bd, args.config, rotate=4 if args.config == 2 else 1,
                         unfused=args.unfused and args.config == 3)
    else:
        res = run_decode(args, torch, bd, 5)
        if not args.no_sub:
            res["sub_results"] = sub_results(args, torch, bd, res)
    print(json.dumps(res), flush=True)


def _sub(r):
    """The fields of a workload's result that the headline line carries for it."""
    keep = ("value", "unit", "ms_per_step", "timing", "eager", "dtype", "unfused", "step_ms", "graph")
    d = {k: r[k] for k in keep if k in r}
    d["workload"] = r["config"]["workload"]
    d["config_index"] = r["config"]["config_index"]
    d["roofline"] = {k: r["roofline"][k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                                   "kernel", "avg_launch_us", "launch_us")
                      if k in r["roofline"]}
    return d


def measure_copy_ceiling(torch, reps=5):
    """Device-to-device copy of a 2 GiB buffer (hipMemcpyAsync): bytes read + written per second,
    the bandwidth a plain copy reaches on this GPU; and a read-only stream (row sums over 4 GiB).
    The larger of the two is the measured ceiling."""
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    copy_gbs = 2 * n / (ms / 1e3) / 1e9
    # read-only: row sums over 4 GiB of float32 (rows of 1024, torch's reduction kernel; a
    # single sum of the whole tensor streams at about 4 TB/s only), the kind of stream the
    # read-dominated kernels here are (a copy also writes as many bytes as it reads)
    x = src.view(torch.float32)
    del dst
    big = torch.cat([x, x]).view(-1, 1024)
    del src, x
    big.sum(dim=1)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        big.sum(dim=1)
    e1.record()
    torch.cuda.synchronize()
    rms = e0.elapsed_time(e1) / reps
    read_gbs = big.numel() * 4 / (rms / 1e3) / 1e9
    del big
    return {"what": "device-to-device copy of 2 GiB (hipMemcpyAsync), read + write bytes; and "
                    "float32 row sums over 4 GiB (read only)",
            "copy_gbs": copy_gbs, "read_gbs": read_gbs, "gbs": max(copy_gbs, read_gbs), "ms": ms}


def sub_results(args, torch, bd, head):
    """The other workloads, each with its own roofline, measured after the headline (its memory
    freed first)."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    out = {}
    steps = max(4, args.steps // 2)
    sub_args = argparse.Namespace(**vars(args))
    sub_args.steps, sub_args.warmup = steps, max(1, args.warmup)
    log("[sub] copy ceiling")
    ceil = measure_copy_ceiling(torch)
    out["copy_ceiling"] = ceil
    head["roofline"]["frac_of_copy_ceiling"] = head["roofline"]["achieved"] / ceil["gbs"]
    log("[sub] config 2: GEMV, 1 token, weights rotated over 4 copies")
    out["gemv_1tok"] = _sub(run_decode(sub_args, torch, bd, 2, cpu_baseline=False, rotate=4))
    gc.collect()
    torch.cuda.empty_cache()
    log("[sub] config 3: one block, 64 tokens, with the unfused comparison")
    out["block_64tok"] = _sub(run_decode(sub_args, torch, bd, 3, cpu_baseline=False, unfused=True))
    gc.collect()
    torch.cuda.empty_cache()
    log("[sub] config 4: prefill, with the unfused comparison")
    out["prefill_4x2048"] = _sub(run_prefill(sub_args, torch, bd, unfused=True))
    gc.collect()
    torch.cuda.empty_cache()
    log("[sub] the headline workload with one alpha per output row")
    rows_args = argparse.Namespace(**vars(sub_args))
    rows_args.alpha_rows = True
    out["alpha_rows_20x70b"] = _sub(run_decode(rows_args, torch, bd, 5, cpu_baseline=False))
    for k in ("gemv_1tok", "block_64tok", "alpha_rows_20x70b"):
        out[k]["roofline"]["frac_of_copy_ceiling"] = out[k]["roofline"]["achieved"] / ceil["gbs"]
    return out


if __name__ == "__main__":
    main()
