"""Host-side checks of libbitdelta that need no GPU: the library loads, exports every entry
point include/bitdelta.h declares, plans segments like the oracle, and rejects every invalid
argument on the host before anything is enqueued (fake device addresses are never touched on
these paths)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.bitdelta_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitdelta.h")

bd = pytest.importorskip("tenant_serving_bitdelta_amd")
if not os.path.exists(bd.LIB_PATH):
    pytest.skip("libbitdelta.so not built", allow_module_level=True)

L = bd.lib()
OK, INVALID, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5
FAKE = 0x7F0000000000  # 256-byte aligned fake device address, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bitdelta_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), f"{n} declared in bitdelta.h but not exported"


def test_abi_version_and_status_strings():
    assert bd.abi_version() == bd.ABI_VERSION == 7
    for s in range(7):
        assert L.bitdelta_status_string(s)
    assert L.bitdelta_status_string(99) == b"unknown status"


def test_sign_words_and_workspace():
    # tiled copy: rows padded to blocks of 128, same words per row
    assert bd.sign_words_t128(4096, 4096) == 4096 * 128
    assert bd.sign_words_t128(1000, 128) == 1024 * 4
    assert bd.sign_words_t128(8, 96) == -1
    assert bd.sign_words(4096, 4096) == 4096 * 128
    assert bd.sign_words(256, 512) == 4096
    assert bd.sign_words(8, 33) == -1 and bd.sign_words(-1, 32) == -1
    # the packed matrix is 1/32 of fp32 storage: words * 4 bytes = d_out * d_in / 8
    assert bd.sign_words(4096, 4096) * 4 == 4096 * 512
    assert bd.compress_workspace_bytes(256, 512) >= 8
    assert bd.compress_workspace_bytes(8192, 28672) % 8 == 0
    assert bd.compress_workspace_bytes(8192, 28672) <= 16384 * 8
    assert bd.compress_workspace_bytes(10, 31) == 0


@pytest.mark.parametrize("m,nv,seed", [(0, 3, 0), (1, 1, 1), (7, 2, 2), (64, 14, 3), (256, 14, 4), (1000, 64, 5)])
def test_plan_matches_oracle(m, nv, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, nv, size=m).astype(np.int32)
    perm, offs, segv = bd.plan_segments(ids, nv)
    rp, ro, rv = O.plan_segments_ref(ids, nv)
    np.testing.assert_array_equal(perm, rp)
    np.testing.assert_array_equal(offs, ro if m else np.array([0], np.int32))
    np.testing.assert_array_equal(segv, rv)


def test_plan_rejects_bad_ids():
    with pytest.raises(bd.BitDeltaError) as e:
        bd.plan_segments([0, 3], 3)
    assert e.value.status == INVALID
    with pytest.raises(bd.BitDeltaError):
        bd.plan_segments([-2], 3)
    with pytest.raises(bd.BitDeltaError):
        bd.plan_segments([0], 65)


def _compress(delta, d_out, d_in, words, alpha, ws, ws_bytes, tiled=None):
    return L.bitdelta_compress(delta, d_out, d_in, words, tiled, alpha, ws, ws_bytes, None)


def test_compress_validation():
    ws = bd.compress_workspace_bytes(64, 64)
    assert _compress(None, 64, 64, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress(FAKE, 64, 64, None, FAKE, FAKE, ws) == INVALID
    assert _compress(FAKE, 0, 64, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress(FAKE, 64, 48, FAKE, FAKE, FAKE, ws) == SHAPE
    assert _compress(FAKE + 4, 64, 64, FAKE, FAKE, FAKE, ws) == ALIGN
    assert _compress(FAKE, 64, 64, FAKE + 2, FAKE, FAKE, ws) == ALIGN
    assert _compress(FAKE, 64, 64, FAKE, FAKE, FAKE + 4, ws) == ALIGN
    assert _compress(FAKE, 64, 64, FAKE, FAKE, FAKE, ws - 8) == WORKSPACE
    # the tiled copy needs d_in % 128 == 0 and 16-byte alignment
    assert _compress(FAKE, 64, 64, FAKE, FAKE, FAKE, ws, tiled=FAKE) == SHAPE
    ws2 = bd.compress_workspace_bytes(64, 128)
    assert _compress(FAKE, 64, 128, FAKE, FAKE, FAKE, ws2, tiled=FAKE + 4) == ALIGN


def _compress_pair(ft, base, d_out, d_in, words, alpha, ws, ws_bytes, tiled=None):
    return L.bitdelta_compress_from_weights(ft, base, d_out, d_in, words, tiled, alpha, ws, ws_bytes,
                                            None)


def test_compress_from_weights_validation():
    ws = bd.compress_workspace_bytes(64, 96)
    assert _compress_pair(None, FAKE, 64, 96, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress_pair(FAKE, None, 64, 96, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress_pair(FAKE, FAKE, 64, 96, None, FAKE, FAKE, ws) == INVALID
    assert _compress_pair(FAKE, FAKE, 0, 96, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress_pair(FAKE, FAKE, 64, 48, FAKE, FAKE, FAKE, ws) == SHAPE
    assert _compress_pair(FAKE + 8, FAKE, 64, 96, FAKE, FAKE, FAKE, ws) == ALIGN
    assert _compress_pair(FAKE, FAKE + 8, 64, 96, FAKE, FAKE, FAKE, ws) == ALIGN
    assert _compress_pair(FAKE, FAKE, 64, 96, FAKE + 2, FAKE, FAKE, ws) == ALIGN
    assert _compress_pair(FAKE, FAKE, 64, 96, FAKE, FAKE, FAKE, ws - 8) == WORKSPACE
    assert _compress_pair(FAKE, FAKE, 64, 96, FAKE, FAKE, FAKE, ws, tiled=FAKE) == SHAPE
    # the row-tile form serves every d_in: its partials fit the compress workspace
    assert bd.compress_workspace_bytes(64, 96) >= 8 * ((64 + 7) // 8)


def _compress_rows(delta, d_out, d_in, words, alpha, ws, ws_bytes, tiled=None):
    return L.bitdelta_compress_rows(delta, d_out, d_in, words, tiled, alpha, ws, ws_bytes, None)


def test_compress_rows_validation():
    ws = bd.compress_rows_workspace_bytes(64, 96)
    assert ws == 64 * 1 * 8  # one fp64 partial per row and 1024-column group
    assert bd.compress_rows_workspace_bytes(10, 2080) == 10 * 3 * 8
    assert bd.compress_rows_workspace_bytes(0, 96) == 0 and bd.compress_rows_workspace_bytes(4, 48) == 0
    assert _compress_rows(None, 64, 96, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress_rows(FAKE, 64, 96, None, FAKE, FAKE, ws) == INVALID
    assert _compress_rows(FAKE, 64, 96, FAKE, None, FAKE, ws) == INVALID
    assert _compress_rows(FAKE, 0, 96, FAKE, FAKE, FAKE, ws) == INVALID
    assert _compress_rows(FAKE, 64, 48, FAKE, FAKE, FAKE, ws) == SHAPE
    assert _compress_rows(FAKE + 8, 64, 96, FAKE, FAKE, FAKE, ws) == ALIGN
    assert _compress_rows(FAKE, 64, 96, FAKE + 2, FAKE, FAKE, ws) == ALIGN
    assert _compress_rows(FAKE, 64, 96, FAKE, FAKE + 2, FAKE, ws) == ALIGN
    assert _compress_rows(FAKE, 64, 96, FAKE, FAKE, FAKE + 4, ws) == ALIGN
    assert _compress_rows(FAKE, 64, 96, FAKE, FAKE, FAKE, ws - 8) == WORKSPACE
    assert _compress_rows(FAKE, 64, 96, FAKE, FAKE, FAKE, ws, tiled=FAKE) == SHAPE
    assert _compress_rows(FAKE, 64, 128, FAKE, FAKE, FAKE, ws, tiled=FAKE + 8) == ALIGN


def test_alpha_per_row_flag_validation():
    """alpha_per_row must be 0 or 1, checked before anything is enqueued."""
    o = np.array([0, 8], dtype=np.int32)
    v = np.array([0], dtype=np.int32)
    op = o.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    vp = v.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    varr = (bd._Variant * 1)()
    varr[0].sign_words, varr[0].sign_words_t128, varr[0].alpha = FAKE, FAKE, FAKE
    prob = (bd._Problem * 1)()
    prob[0].x, prob[0].w_base, prob[0].y = FAKE, FAKE, FAKE
    prob[0].d_out, prob[0].d_in = 256, 256
    prob[0].variants = ctypes.cast(varr, ctypes.POINTER(bd._Variant))
    prob[0].num_variants = 1
    for flag, path, want in [(2, 0, INVALID), (-1, 0, INVALID)]:
        varr[0].alpha_per_row = flag
        assert L.bitdelta_matmul_grouped(prob, 1, 8, op, vp, 1, 0, path, FAKE, 1 << 40, None) == want


def _matmul(x, w, m, d_out, d_in, variants, offs, segv, y, y_dtype=0, path=None, ws=FAKE,
            ws_bytes=1 << 40):
    o = np.ascontiguousarray(offs, dtype=np.int32)
    v = np.ascontiguousarray(segv, dtype=np.int32)
    op = o.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    vp = v.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    varr = (bd._Variant * max(len(variants), 1))()
    for i, var in enumerate(variants):
        varr[i].sign_words, varr[i].alpha = var[0], var[1]
        if len(var) > 2:
            varr[i].sign_words_t128 = var[2]
    if path is None:
        return L.bitdelta_matmul(x, w, m, d_out, d_in, varr, len(variants), op, vp, v.size, y,
                                 y_dtype, ws, ws_bytes, None)
    prob = (bd._Problem * 1)()
    prob[0].x, prob[0].w_base, prob[0].y = x, w, y
    prob[0].d_out, prob[0].d_in = d_out, d_in
    prob[0].variants = ctypes.cast(varr, ctypes.POINTER(bd._Variant))
    prob[0].num_variants = len(variants)
    return L.bitdelta_matmul_grouped(prob, 1, m, op, vp, v.size, y_dtype, path, ws, ws_bytes,
                                     None)


def test_matmul_validation():
    V = [(FAKE, FAKE), (FAKE + 256, FAKE + 512)]
    good = dict(x=FAKE, w=FAKE, m=8, d_out=64, d_in=64, variants=V, offs=[0, 3, 8], segv=[0, 1], y=FAKE)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return _matmul(**a)

    assert call(x=None) == INVALID
    assert call(w=None) == INVALID
    assert call(y=None) == INVALID
    assert call(d_in=48) == SHAPE
    assert call(d_out=0) == INVALID
    assert call(offs=[0, 3, 7]) == SHAPE          # last offset != M
    assert call(offs=[1, 3, 8]) == SHAPE          # first offset != 0
    assert call(offs=[0, 5, 3, 8], segv=[0, 1, 0]) == SHAPE  # not monotone
    assert call(segv=[0, 2]) == INVALID           # variant id out of range
    assert call(segv=[-2, 1]) == INVALID
    assert call(x=FAKE + 8) == ALIGN
    assert call(w=FAKE + 2) == ALIGN
    assert call(y=FAKE + 4) == ALIGN
    assert call(variants=[(FAKE + 2, FAKE), (FAKE, FAKE)]) == ALIGN
    assert call(variants=[(None, FAKE), (FAKE, FAKE)]) == INVALID
    # tiled words alone are a complete variant, but need d_in % 128 == 0 and 16-byte alignment
    assert call(variants=[(None, FAKE, FAKE), (FAKE, FAKE)]) == SHAPE
    assert call(d_in=128, variants=[(None, FAKE, FAKE + 4), (FAKE, FAKE)], path=3) == ALIGN
    assert call(variants=[(None, None, FAKE), (FAKE, FAKE)]) == INVALID
    assert call(y_dtype=7) == INVALID
    assert call(path=9) == INVALID
    assert call(path=1) == UNSUPPORTED            # the GEMV path takes at most 4 tokens
    # d_in = 64 is not a multiple of 128: the decode paths refuse it when forced
    assert call(path=2) == UNSUPPORTED
    assert call(path=4) == UNSUPPORTED
    # SPLIT also needs the tiled sign words of every variant the batch uses
    assert call(d_in=128, path=4) == UNSUPPORTED
    # an unused variant may be absent
    assert call(m=0, offs=[0, 0, 0]) == OK         # empty batch: nothing enqueued
    assert call(m=0, offs=[0], segv=[]) == OK
    assert call(m=0, offs=[0], segv=[], x=None, y=None) == OK  # empty tensors have no storage
    assert call(m=0, offs=[0], segv=[], w=None) == INVALID


def test_split_workspace_validation():
    V = [(FAKE, FAKE, FAKE + 4096), (FAKE + 256, FAKE + 512, FAKE + 8192)]
    need = bd.matmul_workspace_bytes(8, 128)
    good = dict(x=FAKE, w=FAKE, m=8, d_out=64, d_in=128, variants=V, offs=[0, 3, 8], segv=[0, 1],
                y=FAKE, path=4)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return _matmul(**a)

    assert call(ws=None, ws_bytes=0) == WORKSPACE
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=FAKE + 16, ws_bytes=need) == ALIGN
    assert call(path=0, ws=None, ws_bytes=0) == WORKSPACE   # AUTO picks SPLIT for 8 tokens
    assert call(m=0, offs=[0, 0, 0], ws=None, ws_bytes=0) == OK


def test_matmul_workspace_bytes():
    # per token (M rounded up to 16): a bf16 copy (2 bytes per element), the two fp6 terms
    # (1.5 bytes per element) and one 4-byte scale word per 32 elements, each region rounded
    # up to 256 bytes; then the linear's share of the call's partial slots (128 slots of
    # 128 rows x 4 bytes per token), of its split counters (128 x 8 bytes) and a 256-byte
    # statistics block
    # and one fp32 correction sum per token and 128 columns
    part = lambda mp: 128 * 128 * 4 * mp + 128 * 8 + 256
    assert bd.matmul_workspace_bytes(256, 8192) == (256 * 8192 * 2 + 256 * 8192 * 3 // 2
                                                    + 256 * 8192 // 8 + 256 * 8192 // 32 + part(256))
    assert bd.matmul_workspace_bytes(5, 128, "split") == (16 * 128 * 2 + 16 * 128 * 3 // 2 + 256
                                                          + 256 + part(16))
    assert bd.matmul_workspace_bytes(4, 8192) == 0            # AUTO -> GEMV, no workspace
    assert bd.matmul_workspace_bytes(300, 8192) == 0          # AUTO -> PREFILL
    assert bd.matmul_workspace_bytes(64, 8192, "stream") == 0
    assert bd.matmul_workspace_bytes(0, 8192, "split") == 0
    assert bd.matmul_workspace_bytes(64, 8192, "split") % 256 == 0


def test_auto_path_choice():
    assert bd.auto_path(1, [0, 1], [0]) == 1
    assert bd.auto_path(4, [0, 2, 4], [0, 3]) == 1
    assert bd.auto_path(64, [0, 64], [0]) == 4
    assert bd.auto_path(256, [0, 100, 256], [-1, 5]) == 4
    assert bd.auto_path(8192, [0, 2048, 4096, 6144, 8192], [0, 1, 2, 3]) == 3
    assert bd.auto_path(8, [0, 9], [0]) == -1


def _variant(words=FAKE, alpha=FAKE, tiled=None, per_row=0):
    v = bd._Variant()
    v.sign_words, v.alpha, v.sign_words_t128, v.alpha_per_row = words, alpha, tiled, per_row
    return v


def test_reconstruct_validation():
    R = L.bitdelta_reconstruct

    def call(w=FAKE, d_out=64, d_in=64, var=None, out=FAKE + 1024 * 1024):
        v = _variant() if var is None else var
        return R(w, d_out, d_in, ctypes.byref(v), out, None)

    assert call(w=None) == INVALID
    assert call(out=None) == INVALID
    assert R(FAKE, 64, 64, None, FAKE, None) == INVALID
    assert call(var=_variant(words=None)) == INVALID
    assert call(var=_variant(alpha=None)) == INVALID
    assert call(var=_variant(per_row=3)) == INVALID
    assert call(d_out=0) == INVALID
    assert call(d_in=48) == SHAPE
    assert call(var=_variant(words=None, tiled=FAKE)) == SHAPE      # tiled needs d_in % 128
    assert call(w=FAKE + 8) == ALIGN
    assert call(out=FAKE + 8) == ALIGN
    assert call(var=_variant(words=FAKE + 2)) == ALIGN
    assert call(d_in=128, var=_variant(words=None, tiled=FAKE + 4)) == ALIGN


def test_upload_validation():
    U = L.bitdelta_upload_variant
    host = np.zeros(64 * 128 // 32, dtype=np.uint32)
    ha = np.zeros(64, dtype=np.float32)
    hp, ap = host.ctypes.data, ha.ctypes.data

    def call(hw=hp, hal=ap, na=1, d_out=64, d_in=128, words=FAKE, tiled=None, alpha=FAKE,
             staging=None, sb=0):
        return U(hw, hal, na, d_out, d_in, words, tiled, alpha, staging, sb, None)

    assert call(hw=None) == INVALID
    assert call(hal=None) == INVALID
    assert call(alpha=None) == INVALID
    assert call(words=None) == INVALID                 # no destination
    assert call(na=2) == INVALID                       # 1 or d_out scales
    assert call(d_out=0) == INVALID
    assert call(d_in=48) == SHAPE
    assert call(d_in=96, tiled=FAKE) == SHAPE
    assert call(words=None, tiled=FAKE) == WORKSPACE   # tiled alone needs staging
    assert call(words=None, tiled=FAKE, staging=FAKE, sb=64 * 128 // 8 - 1) == WORKSPACE
    assert call(words=None, tiled=FAKE, staging=FAKE + 4, sb=64 * 128 // 8) == ALIGN
    assert call(tiled=FAKE + 8) == ALIGN
    assert call(words=FAKE + 4, tiled=FAKE) == ALIGN   # read back 16 bytes at a time
    assert call(words=FAKE + 2) == ALIGN
    assert call(alpha=FAKE + 2) == ALIGN
