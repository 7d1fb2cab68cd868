"""Python binding of libbitdelta (the MI355X BitDelta hot path).

Thin ctypes marshalling only: every step of compression and of the fused reconstruct-and-
multiply runs in the library's HIP kernels.  torch is used to hold device memory and to name
the current HIP stream.  If the library is not built this module raises on first use; there
is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "BitDeltaError", "lib", "abi_version", "sign_words", "compress_workspace_bytes",
    "compress_rows", "compress_rows_workspace_bytes", "compress_from_weights",
    "compress", "plan_segments", "matmul", "matmul_grouped", "auto_path", "PATHS",
    "matmul_workspace_bytes", "sign_words_t128", "reconstruct", "upload_variant", "Residency",
    "matmul_grouped_noalloc", "NOALLOC_SCRATCH_BYTES",
]

ABI_VERSION = 7
NOALLOC_SCRATCH_BYTES = 128 << 20  # BITDELTA_NOALLOC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitdelta.so")

PATHS = {"auto": 0, "gemv": 1, "stream": 2, "prefill": 3, "split": 4}
_OUT = {"bf16": 0, "f32": 1}
MAX_VARIANTS = 64
MAX_PROBLEMS = 8


class BitDeltaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        name = _lib().bitdelta_status_string(int(status)).decode() if _LIB is not None else str(status)
        if self.status == 6 and _LIB is not None:  # BITDELTA_ERR_HIP: name the runtime's error
            name += f" [{_LIB.bitdelta_last_hip_error_string().decode()}]"
        super().__init__(f"{what}: {name} (status {status})" if what else f"{name} (status {status})")


class _Variant(ctypes.Structure):
    _fields_ = [("sign_words", ctypes.c_void_p), ("sign_words_t128", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p), ("alpha_per_row", ctypes.c_int32)]


class _Problem(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p), ("w_base", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64),
        ("variants", ctypes.POINTER(_Variant)), ("num_variants", ctypes.c_int32),
    ]


_LIB = None
_i32p = ctypes.POINTER(ctypes.c_int32)


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
        # torch first: its HIP runtime is then the one the library binds to.  Loaded the other
        # way round, a process can end up with two HIP runtimes (torch's bundled copy and the
        # system one) whose kernels and device memory do not mix.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.bitdelta_abi_version.restype = ctypes.c_int
        L.bitdelta_status_string.restype = ctypes.c_char_p
        L.bitdelta_status_string.argtypes = [ctypes.c_int]
        L.bitdelta_last_hip_error.restype = ctypes.c_int32
        L.bitdelta_last_hip_error_string.restype = ctypes.c_char_p
        L.bitdelta_sign_words.restype = ctypes.c_int64
        L.bitdelta_sign_words.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.bitdelta_compress_workspace_bytes.restype = ctypes.c_size_t
        L.bitdelta_compress_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.bitdelta_compress.restype = ctypes.c_int
        L.bitdelta_compress.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_compress_from_weights.restype = ctypes.c_int
        L.bitdelta_compress_from_weights.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_void_p, ctypes.c_void_p,
                                                     ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_compress_rows.restype = ctypes.c_int
        L.bitdelta_compress_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_compress_rows_workspace_bytes.restype = ctypes.c_size_t
        L.bitdelta_compress_rows_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.bitdelta_residency_create.restype = ctypes.c_int
        L.bitdelta_residency_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                                ctypes.c_int64, ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_void_p)]
        L.bitdelta_residency_destroy.restype = None
        L.bitdelta_residency_destroy.argtypes = [ctypes.c_void_p]
        L.bitdelta_residency_request.restype = ctypes.c_int
        L.bitdelta_residency_request.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                 _i32p, _i32p, _i32p]
        L.bitdelta_residency_release.restype = ctypes.c_int
        L.bitdelta_residency_release.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.bitdelta_residency_holds.restype = ctypes.c_int64
        L.bitdelta_residency_holds.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.bitdelta_residency_load_enqueued.restype = ctypes.c_int
        L.bitdelta_residency_load_enqueued.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                                       ctypes.c_void_p]
        L.bitdelta_residency_poll.restype = ctypes.c_int
        L.bitdelta_residency_poll.argtypes = [ctypes.c_void_p, _i32p, _i32p]
        L.bitdelta_reconstruct.restype = ctypes.c_int
        L.bitdelta_reconstruct.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.POINTER(_Variant), ctypes.c_void_p,
                                           ctypes.c_void_p]
        L.bitdelta_upload_variant.restype = ctypes.c_int
        L.bitdelta_upload_variant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_residency_load_done.restype = ctypes.c_int
        L.bitdelta_residency_load_done.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.bitdelta_residency_state.restype = ctypes.c_int32
        L.bitdelta_residency_state.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.bitdelta_residency_used_bytes.restype = ctypes.c_int64
        L.bitdelta_residency_used_bytes.argtypes = [ctypes.c_void_p]
        L.bitdelta_sign_words_t128.restype = ctypes.c_int64
        L.bitdelta_sign_words_t128.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.bitdelta_plan_segments.restype = ctypes.c_int
        L.bitdelta_plan_segments.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32, _i32p, _i32p,
                                             _i32p, _i32p]
        L.bitdelta_matmul.restype = ctypes.c_int
        L.bitdelta_matmul.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_Variant),
                                      ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_matmul_grouped.restype = ctypes.c_int
        L.bitdelta_matmul_grouped.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32,
                                              ctypes.c_int64, _i32p, _i32p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]
        L.bitdelta_matmul_grouped_noalloc.restype = ctypes.c_int
        L.bitdelta_matmul_grouped_noalloc.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32,
                                                      ctypes.c_int64, _i32p, _i32p, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_void_p]
        L.bitdelta_matmul_workspace_bytes.restype = ctypes.c_size_t
        L.bitdelta_matmul_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64,
                                                      ctypes.c_int32]
        L.bitdelta_auto_path.restype = ctypes.c_int32
        L.bitdelta_auto_path.argtypes = [ctypes.c_int64, _i32p, _i32p, ctypes.c_int32]
        _LIB = L
    return _LIB


lib = _lib


def _check(status: int, what: str):
    if status != 0:
        raise BitDeltaError(status, what)


def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_i32p)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _temp(nbytes, device, stream, dtype_name="uint8"):
    """A scratch device tensor for one call whose kernels run on ``stream`` (None: torch's
    current stream).  torch's caching allocator must not hand the block to another tensor while
    those kernels still use it, so on another stream the block is recorded as in use there."""
    import torch
    dtype = getattr(torch, dtype_name)
    n = max(int(nbytes), 1) // torch.empty((), dtype=dtype).element_size()
    t = torch.empty(max(n, 1), dtype=dtype, device=device)
    if stream is not None and int(stream) != torch.cuda.current_stream(device).cuda_stream:
        t.record_stream(torch.cuda.ExternalStream(int(stream), device=device))
    return t


def _numel_at_least(t, n, what):
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements, needs at least {n}")


def _numel_exact(t, n, what):
    if t.numel() != n:
        raise ValueError(f"{what} holds {t.numel()} elements, needs exactly {n}")


def _check_shape(t, shape, what):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, needs {tuple(shape)}")


_DTYPES = {}


def _dev(t, dtype_name, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA/HIP torch tensor")
    want = _DTYPES.get(dtype_name)
    if want is None:
        want = _DTYPES[dtype_name] = getattr(torch, dtype_name.split(".")[1])
    if t.dtype is not want:
        raise TypeError(f"{what} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def abi_version() -> int:
    return int(_lib().bitdelta_abi_version())


def sign_words(d_out: int, d_in: int) -> int:
    return int(_lib().bitdelta_sign_words(d_out, d_in))


def sign_words_t128(d_out: int, d_in: int) -> int:
    """Words of the tiled sign copy (128-row blocks x 128-column steps), -1 if d_in % 128."""
    return int(_lib().bitdelta_sign_words_t128(d_out, d_in))


def compress_workspace_bytes(d_out: int, d_in: int) -> int:
    return int(_lib().bitdelta_compress_workspace_bytes(d_out, d_in))


def _compress_outputs(d_out, d_in, words, tiled, alpha, alpha_n):
    """Pointers of compress outputs after checking their sizes: ``words`` (int32, d_out * d_in / 32
    elements) and ``tiled`` (int32, at least sign_words_t128 elements) may each be None, not both."""
    if words is None and tiled is None:
        raise ValueError("give the row-major words, the tiled words, or both")
    if d_in % 32:
        raise ValueError("d_in must be a multiple of 32")
    wptr = tptr = None
    if words is not None:
        _numel_exact(words, d_out * d_in // 32, "words")
        wptr = _dev(words, "torch.int32", "words")
    if tiled is not None:
        nt = sign_words_t128(d_out, d_in)
        if nt < 0:
            raise ValueError("the tiled layout needs d_in % 128 == 0")
        _numel_at_least(tiled, nt, "tiled sign words")
        tptr = _dev(tiled, "torch.int32", "tiled sign words")
    _numel_exact(alpha, alpha_n, "alpha")
    return wptr, tptr, _dev(alpha, "torch.float32", "alpha")


def _workspace_arg(workspace, need, device, stream):
    """(tensor, pointer, bytes) of a caller's workspace (the library checks its size), or of a
    scratch tensor sized ``need`` when None."""
    if workspace is None:
        workspace = _temp(max(need, 8), device, stream, "float64")
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def compress(delta, words, alpha, workspace=None, stream=None, tiled=None):
    """alpha = mean|delta| and packed sign bits of one float32 [d_out, d_in] matrix.
    ``words``: int32 tensor [d_out, d_in // 32] (uint32 bit patterns) or None, ``alpha``: float32
    [1], ``tiled``: int32 tensor of sign_words_t128(d_out, d_in) words for the tiled layout, or
    None (at least one of words / tiled)."""
    d_out, d_in = delta.shape
    wptr, tptr, aptr = _compress_outputs(d_out, d_in, words, tiled, alpha, 1)
    ws, ws_ptr, ws_bytes = _workspace_arg(workspace, compress_workspace_bytes(d_out, d_in),
                                          delta.device, stream)
    _check(_lib().bitdelta_compress(
        _dev(delta, "torch.float32", "delta"), d_out, d_in, wptr, tptr, aptr, ws_ptr, ws_bytes,
        _stream(stream)), "bitdelta_compress")
    return words, alpha


def compress_from_weights(w_ft, w_base, words, alpha, workspace=None, stream=None, tiled=None):
    """compress() of Delta = w_ft - w_base for two bf16 [d_out, d_in] matrices, Delta never
    formed.  Outputs as for compress()."""
    d_out, d_in = w_base.shape
    if tuple(w_ft.shape) != (d_out, d_in):
        raise ValueError("w_ft and w_base must have the same shape")
    wptr, tptr, aptr = _compress_outputs(d_out, d_in, words, tiled, alpha, 1)
    ws, ws_ptr, ws_bytes = _workspace_arg(workspace, compress_workspace_bytes(d_out, d_in),
                                          w_base.device, stream)
    _check(_lib().bitdelta_compress_from_weights(
        _dev(w_ft, "torch.bfloat16", "w_ft"), _dev(w_base, "torch.bfloat16", "w_base"), d_out, d_in,
        wptr, tptr, aptr, ws_ptr, ws_bytes, _stream(stream)), "bitdelta_compress_from_weights")
    return words, alpha


def compress_rows_workspace_bytes(d_out: int, d_in: int) -> int:
    return int(_lib().bitdelta_compress_rows_workspace_bytes(d_out, d_in))


def compress_rows(delta, words, alpha, workspace=None, stream=None, tiled=None):
    """compress() with one scale per output row: ``alpha`` is float32 [d_out]; pass the result to
    matmul as (words, alpha[, tiled]) and it is applied row by row."""
    d_out, d_in = delta.shape
    wptr, tptr, aptr = _compress_outputs(d_out, d_in, words, tiled, alpha, d_out)
    ws, ws_ptr, ws_bytes = _workspace_arg(workspace, compress_rows_workspace_bytes(d_out, d_in),
                                          delta.device, stream)
    _check(_lib().bitdelta_compress_rows(
        _dev(delta, "torch.float32", "delta"), d_out, d_in, wptr, tptr, aptr, ws_ptr, ws_bytes,
        _stream(stream)), "bitdelta_compress_rows")
    return words, alpha


def plan_segments(token_variant, num_variants: int):
    """Stable grouping of tokens by variant (base -1 first).  Returns numpy int32
    (perm, seg_offsets, seg_variant)."""
    ids, ids_p = _i32(token_variant)
    m = ids.size
    perm = np.zeros(max(m, 1), dtype=np.int32)
    offs = np.zeros(num_variants + 2, dtype=np.int32)
    segv = np.zeros(num_variants + 1, dtype=np.int32)
    ns = ctypes.c_int32(0)
    _check(_lib().bitdelta_plan_segments(
        ids_p, m, num_variants, perm.ctypes.data_as(_i32p), offs.ctypes.data_as(_i32p),
        segv.ctypes.data_as(_i32p), ctypes.byref(ns)), "bitdelta_plan_segments")
    n = ns.value
    return perm[:m].copy(), offs[:n + 1].copy(), segv[:n].copy()


def matmul_workspace_bytes(m: int, d_in: int, path="auto") -> int:
    """Device workspace one linear of a matmul call on ``path`` needs (bytes, 0 if none)."""
    return int(_lib().bitdelta_matmul_workspace_bytes(m, d_in, PATHS[path]))


def _workspace(workspace, need, device, stream):
    """(pointer, bytes, tensor) of the caller's workspace tensor, or of a scratch one sized
    ``need`` when None (none at all when ``need`` is 0)."""
    if workspace is None:
        if need == 0:
            return None, 0, None
        workspace = _temp(need, device, stream)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def auto_path(m: int, seg_offsets, seg_variant) -> int:
    o, op = _i32(seg_offsets)
    v, vp = _i32(seg_variant)
    return int(_lib().bitdelta_auto_path(m, op, vp, v.size))


def _variant_struct(v, item, d_out, d_in, i=0):
    """Fill one _Variant from (words, alpha) or (words, alpha, tiled_words): words (row-major,
    d_out * d_in / 32 int32) or tiled_words (at least sign_words_t128 int32) may be None, not both;
    alpha holds one float32 (per matrix) or d_out of them (per output row)."""
    words, alpha = item[0], item[1]
    tiled = item[2] if len(item) > 2 else None
    if words is None and tiled is None:
        raise ValueError(f"variant {i}: needs row-major or tiled sign words")
    if words is not None:
        _numel_exact(words, d_out * d_in // 32, f"variant {i} sign words")
        v.sign_words = _dev(words, "torch.int32", "sign words")
    if tiled is not None:
        nt = sign_words_t128(d_out, d_in)
        if nt < 0:
            raise ValueError(f"variant {i}: tiled sign words need d_in % 128 == 0")
        _numel_at_least(tiled, nt, f"variant {i} tiled sign words")
        v.sign_words_t128 = _dev(tiled, "torch.int32", "tiled sign words")
    n = alpha.numel()
    if n != 1 and n != d_out:
        raise ValueError(f"variant {i}: alpha must hold 1 or d_out = {d_out} values, not {n}")
    v.alpha = _dev(alpha, "torch.float32", "alpha")
    v.alpha_per_row = 1 if n > 1 else 0


def _variants_array(variants, d_out, d_in):
    """variants: list of (words, alpha[, tiled_words]) tuples (None for ids the call never uses)."""
    arr = (_Variant * max(len(variants), 1))()
    for i, item in enumerate(variants):
        if item is not None:
            _variant_struct(arr[i], item, d_out, d_in, i)
    return arr


def _problems_array(problems, m, out_dtype):
    """ctypes array of bitdelta_problem for (x, w_base, y, variants) tuples, sizes checked; the
    second value keeps the variant arrays alive."""
    if not 1 <= len(problems) <= MAX_PROBLEMS:
        raise ValueError("1..8 problems per call")
    parr = (_Problem * len(problems))()
    keep = []
    for i, (x, w, y, variants) in enumerate(problems):
        if w.dim() != 2:
            raise ValueError("w_base must be [d_out, d_in]")
        d_out, d_in = int(w.shape[0]), int(w.shape[1])
        _check_shape(x, (m, d_in), f"problem {i} x")
        _check_shape(y, (m, d_out), f"problem {i} y")
        varr = _variants_array(variants, d_out, d_in)
        keep.append(varr)
        parr[i].x = _dev(x, "torch.bfloat16", "x")
        parr[i].w_base = _dev(w, "torch.bfloat16", "w_base")
        parr[i].y = _dev(y, "torch.bfloat16" if out_dtype == "bf16" else "torch.float32", "y")
        parr[i].d_out, parr[i].d_in = d_out, d_in
        parr[i].variants = ctypes.cast(varr, ctypes.POINTER(_Variant))
        parr[i].num_variants = len(variants)
    return parr, keep


def matmul_grouped(problems, seg_offsets, seg_variant, out_dtype="bf16", path="auto", stream=None,
                   workspace=None):
    """Fused y = x (W_base + alpha_v sign_v)^T for several linears sharing one segmentation.
    ``problems``: list of (x, w_base, y, variants) with variants a list of (words, alpha).
    ``workspace``: device tensor of at least the summed matmul_workspace_bytes (allocated here
    when None)."""
    offs, offs_p = _i32(seg_offsets)
    segv, segv_p = _i32(seg_variant)
    m = int(offs[-1]) if offs.size else 0
    parr, keep = _problems_array(problems, m, out_dtype)
    # the library checks the size of a caller's workspace itself; only a missing one is sized here
    need = 0 if workspace is not None else sum(
        matmul_workspace_bytes(m, int(w.shape[1]), path) for _, w, _, _ in problems)
    ws_ptr, ws_bytes, ws = _workspace(workspace, need, problems[0][1].device, stream)
    _check(_lib().bitdelta_matmul_grouped(parr, len(problems), m, offs_p, segv_p, segv.size,
                                          _OUT[out_dtype], PATHS[path], ws_ptr, ws_bytes,
                                          _stream(stream)),
           "bitdelta_matmul_grouped")
    return [p[2] for p in problems]


def matmul_grouped_noalloc(problems, seg_offsets, seg_variant, out_dtype="bf16", path="auto",
                           stream=None):
    """matmul_grouped on the SPLIT path with the library's own per-device scratch as workspace:
    the call allocates no device memory (for callers that cannot).  Batches the SPLIT path does
    not serve raise BitDeltaError (status 5); calls that overlap on one device must not be made."""
    offs, offs_p = _i32(seg_offsets)
    segv, segv_p = _i32(seg_variant)
    m = int(offs[-1]) if offs.size else 0
    parr, keep = _problems_array(problems, m, out_dtype)
    _check(_lib().bitdelta_matmul_grouped_noalloc(parr, len(problems), m, offs_p, segv_p, segv.size,
                                                  _OUT[out_dtype], PATHS[path], _stream(stream)),
           "bitdelta_matmul_grouped_noalloc")
    return [p[2] for p in problems]


def matmul(x, w_base, variants, seg_offsets, seg_variant, y=None, out_dtype="bf16", path="auto",
           stream=None, workspace=None):
    """Fused y = x (W_base + alpha_v sign_v)^T over a token batch grouped by variant."""
    import torch
    if y is None:
        y = torch.empty((x.shape[0], w_base.shape[0]), device=x.device,
                        dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    if path != "auto":
        matmul_grouped([(x, w_base, y, variants)], seg_offsets, seg_variant, out_dtype, path,
                       stream, workspace)
        return y
    offs, offs_p = _i32(seg_offsets)
    segv, segv_p = _i32(seg_variant)
    if w_base.dim() != 2:
        raise ValueError("w_base must be [d_out, d_in]")
    d_out, d_in = int(w_base.shape[0]), int(w_base.shape[1])
    m = int(offs[-1]) if offs.size else 0
    _check_shape(x, (m, d_in), "x")
    _check_shape(y, (m, d_out), "y")
    varr = _variants_array(variants, d_out, d_in)
    ws_ptr, ws_bytes, ws = _workspace(
        workspace, 0 if workspace is not None else matmul_workspace_bytes(m, d_in), x.device, stream)
    _check(_lib().bitdelta_matmul(
        _dev(x, "torch.bfloat16", "x"), _dev(w_base, "torch.bfloat16", "w_base"),
        m, d_out, d_in, varr, len(variants),
        offs_p, segv_p, segv.size,
        _dev(y, "torch.bfloat16" if out_dtype == "bf16" else "torch.float32", "y"),
        _OUT[out_dtype], ws_ptr, ws_bytes, _stream(stream)), "bitdelta_matmul")
    return y


class Residency:
    """The library's delta residency manager (host only): request(v) -> (action, evicted ids),
    with action one of HIT, LOAD, QUEUED, NO_ROOM; load_done(v) when a load has finished."""
    HIT, LOAD, QUEUED, NO_ROOM = 0, 1, 2, 3
    ABSENT, LOADING, RESIDENT = 0, 1, 2

    def __init__(self, variant_bytes, capacity_bytes: int, num_pinned: int = 6):
        L = _lib()
        self._n = len(variant_bytes)
        sizes = (ctypes.c_int64 * max(self._n, 1))(*[int(b) for b in variant_bytes])
        h = ctypes.c_void_p()
        _check(L.bitdelta_residency_create(self._n, sizes, int(capacity_bytes), int(num_pinned),
                                           ctypes.byref(h)), "bitdelta_residency_create")
        self._h = h

    def request(self, v: int, hold: bool = False):
        """(action, evicted ids).  hold=True: an answer other than NO_ROOM makes this request a
        holder of v, which is not evicted until release(v)."""
        # output buffers per call, so that threads sharing a manager never read each other's
        ev = (ctypes.c_int32 * self._n)()
        act, ne = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib().bitdelta_residency_request(self._h, int(v), 1 if hold else 0,
                                                 ctypes.byref(act), ev, ctypes.byref(ne)),
               "bitdelta_residency_request")
        return act.value, [ev[i] for i in range(ne.value)]

    def release(self, v: int):
        _check(_lib().bitdelta_residency_release(self._h, int(v)), "bitdelta_residency_release")

    def holds(self, v: int) -> int:
        return int(_lib().bitdelta_residency_holds(self._h, int(v)))

    def load_enqueued(self, v: int, event):
        """Attach the event recorded after v's upload (a torch.cuda.Event that has been
        recorded); poll() then makes v resident once the event has completed.  Keep the event
        alive until then."""
        _check(_lib().bitdelta_residency_load_enqueued(self._h, int(v),
                                                       ctypes.c_void_p(int(event.cuda_event))),
               "bitdelta_residency_load_enqueued")

    def poll(self):
        """Variants whose attached upload event has completed since the last poll (now resident)."""
        out = (ctypes.c_int32 * self._n)()
        nc = ctypes.c_int32()
        _check(_lib().bitdelta_residency_poll(self._h, out, ctypes.byref(nc)),
               "bitdelta_residency_poll")
        return [out[i] for i in range(nc.value)]

    def load_done(self, v: int):
        _check(_lib().bitdelta_residency_load_done(self._h, int(v)), "bitdelta_residency_load_done")

    def state(self, v: int) -> int:
        return int(_lib().bitdelta_residency_state(self._h, int(v)))

    def used_bytes(self) -> int:
        return int(_lib().bitdelta_residency_used_bytes(self._h))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.bitdelta_residency_destroy(h)
            self._h = None


def reconstruct(w_base, variant, w_eff=None, stream=None):
    """W_eff = bf16(W_base + alpha * sign) written to a bf16 [d_out, d_in] tensor (the unfused
    reconstruction; the fused matmul never forms it).  ``variant``: (words, alpha[, tiled])."""
    import torch
    if w_base.dim() != 2:
        raise ValueError("w_base must be [d_out, d_in]")
    d_out, d_in = int(w_base.shape[0]), int(w_base.shape[1])
    if w_eff is None:
        w_eff = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=w_base.device)
    _check_shape(w_eff, (d_out, d_in), "w_eff")
    v = _Variant()
    _variant_struct(v, variant, d_out, d_in)
    _check(_lib().bitdelta_reconstruct(_dev(w_base, "torch.bfloat16", "w_base"), d_out, d_in,
                                       ctypes.byref(v), _dev(w_eff, "torch.bfloat16", "w_eff"),
                                       _stream(stream)), "bitdelta_reconstruct")
    return w_eff


def upload_variant(host_words, host_alpha, d_out: int, d_in: int, words=None, tiled=None,
                   alpha=None, staging=None, stream=None):
    """Host -> device upload of one compressed matrix of a variant, into the layout the kernels
    read.  ``host_words``: CPU int32 tensor of d_out * d_in / 32 row-major words (pinned memory
    makes the copy asynchronous); ``host_alpha``: CPU float32 tensor of 1 or d_out scales;
    ``words`` / ``tiled``: device destinations (at least one); ``alpha``: device float32
    destination; ``staging``: device scratch of d_out * d_in / 8 bytes when only ``tiled`` is
    given (allocated here when None).  Returns (words, tiled, alpha)."""
    import torch
    if host_words.is_cuda or host_alpha.is_cuda:
        raise TypeError("host_words and host_alpha must be CPU tensors")
    if host_words.dtype is not torch.int32 or host_alpha.dtype is not torch.float32:
        raise TypeError("host_words must be int32 and host_alpha float32")
    if not host_words.is_contiguous() or not host_alpha.is_contiguous():
        raise ValueError("host tensors must be contiguous")
    if d_in % 32:
        raise ValueError("d_in must be a multiple of 32")
    _numel_exact(host_words, d_out * d_in // 32, "host_words")
    na = host_alpha.numel()
    if na != 1 and na != d_out:
        raise ValueError("host_alpha must hold 1 or d_out scales")
    if alpha is None:
        raise ValueError("a device alpha tensor is required")
    wptr, tptr, aptr = _compress_outputs(d_out, d_in, words, tiled, alpha, na)
    sptr, sbytes = None, 0
    if words is None:
        nb = d_out * d_in // 8
        if staging is None:
            staging = _temp(nb, alpha.device, stream)
        if not staging.is_cuda or not staging.is_contiguous():
            raise ValueError("staging must be a contiguous device tensor")
        sptr, sbytes = staging.data_ptr(), staging.numel() * staging.element_size()
    _check(_lib().bitdelta_upload_variant(host_words.data_ptr(), host_alpha.data_ptr(), na, d_out,
                                          d_in, wptr, tptr, aptr, sptr, sbytes, _stream(stream)),
           "bitdelta_upload_variant")
    return words, tiled, alpha
