"""CPU checks of the C-ABI library: it loads, exports every symbol that
include/lynx.h declares, rejects bad arguments before touching a GPU, and
its host-side constant tables agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lynx.h")
LIB = os.path.join(ROOT, "long_context_serving_amd", "_lib", "liblynx.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from long_context_serving_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lynx_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("lynx_quantize_pages", "lynx_quantize_kv_pages", "lynx_dequantize_anchor",
                     "lynx_dequantize_full",
                     "lynx_decode_attention_anchor", "lynx_decode_attention_full",
                     "lynx_decode_attention_workspace_size", "lynx_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


class CPlanes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("anchor", "residual", "page_min", "page_range", "chunk_mean", "chunk_maxabs")]


def _fake_planes(base=0x10000):
    return CPlanes(*(base + 0x1000 * i for i in range(6)))


def test_argument_errors_are_reported_before_any_launch(lib):
    P = ctypes.c_void_p
    lib.lynx_quantize_pages.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.POINTER(CPlanes), P]
    pl = _fake_planes()
    kv = P(0x20000)
    assert lib.lynx_quantize_pages(None, 4, 8, 128, 0, ctypes.byref(pl), None) == -1
    assert lib.lynx_quantize_pages(kv, 4, 8, 64, 0, ctypes.byref(pl), None) == -2
    assert lib.lynx_quantize_pages(kv, -1, 8, 128, 0, ctypes.byref(pl), None) == -2
    assert lib.lynx_quantize_pages(kv, 4, 0, 128, 0, ctypes.byref(pl), None) == -2
    assert lib.lynx_quantize_pages(kv, 4, 8, 128, 3, ctypes.byref(pl), None) == -7
    assert lib.lynx_quantize_pages(P(0x20001), 4, 8, 128, 0, ctypes.byref(pl), None) == -3
    bad = _fake_planes()
    bad.residual = None
    assert lib.lynx_quantize_pages(kv, 4, 8, 128, 0, ctypes.byref(bad), None) == -1
    bad = _fake_planes()
    bad.chunk_mean = 0x30004
    assert lib.lynx_quantize_pages(kv, 4, 8, 128, 1, ctypes.byref(bad), None) == -3
    # zero pages is a no-op that needs no device
    assert lib.lynx_quantize_pages(kv, 0, 8, 128, 0, ctypes.byref(pl), None) == 0

    lib.lynx_quantize_kv_pages.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(CPlanes), ctypes.POINTER(CPlanes), P]
    kv2 = P(0x50000)
    pv = _fake_planes(0x60000)
    q2 = lib.lynx_quantize_kv_pages
    assert q2(kv, None, 4, 8, 128, ctypes.byref(pl), ctypes.byref(pv), None) == -1
    assert q2(kv, kv2, 4, 8, 128, ctypes.byref(pl), None, None) == -1
    assert q2(kv, kv2, 4, 8, 64, ctypes.byref(pl), ctypes.byref(pv), None) == -2
    assert q2(kv, kv2, -1, 8, 128, ctypes.byref(pl), ctypes.byref(pv), None) == -2
    assert q2(kv, kv2, 1 << 28, 8, 128, ctypes.byref(pl), ctypes.byref(pv), None) == -2  # 2 P H > 2^31 - 1
    assert q2(kv, P(0x50008), 4, 8, 128, ctypes.byref(pl), ctypes.byref(pv), None) == -3
    bad = _fake_planes()
    bad.residual = None
    assert q2(kv, kv2, 4, 8, 128, ctypes.byref(pl), ctypes.byref(bad), None) == -1
    assert q2(kv, kv2, 0, 8, 128, ctypes.byref(pl), ctypes.byref(pv), None) == 0

    for name in ("lynx_dequantize_anchor", "lynx_dequantize_full"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.POINTER(CPlanes), ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, P, P]
        assert fn(ctypes.byref(pl), 4, 8, 128, 0, None, None) == -1
        assert fn(ctypes.byref(pl), 4, 8, 100, 0, P(0x40000), None) == -2
        assert fn(ctypes.byref(pl), 0, 8, 128, 1, P(0x40000), None) == 0
    # the anchor dequantizer never needs the residual plane
    nores = _fake_planes()
    nores.residual = None
    assert lib.lynx_dequantize_full(ctypes.byref(nores), 4, 8, 128, 0, P(0x40000), None) == -1
    assert lib.lynx_dequantize_anchor(ctypes.byref(nores), 0, 8, 128, 0, P(0x40000), None) == 0

    lib.lynx_decode_attention_workspace_size.restype = ctypes.c_size_t
    lib.lynx_decode_attention_workspace_size.argtypes = [ctypes.c_int32] * 5
    need = lib.lynx_decode_attention_workspace_size(2, 8, 64, 128, 16)
    assert need > 0
    assert lib.lynx_decode_attention_workspace_size(2, 8, 60, 128, 16) == 0   # Hq % H != 0
    assert lib.lynx_decode_attention_workspace_size(2, 2, 64, 128, 16) == 0   # group 32 > 16
    for name in ("lynx_decode_attention_anchor", "lynx_decode_attention_full"):
        fn = getattr(lib, name)
        fn.argtypes = [P, ctypes.POINTER(CPlanes), ctypes.POINTER(CPlanes), P, P,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_int64, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        q, out, ws = P(0x50000), P(0x60000), P(0x70000)
        args = lambda **kw: dict(dict(q=q, bt=None, sl=None, B=2, H=8, Hq=64, D=128, mp=16, pool=32,
                                      ws=ws, wsb=need), **kw)

        def call(a):
            return fn(a["q"], ctypes.byref(pl), ctypes.byref(pl), a["bt"], a["sl"], a["B"], a["H"],
                      a["Hq"], a["D"], a["mp"], a["pool"], 0.088, out, None, a["ws"], a["wsb"], None)
        assert call(args(q=None)) == -1
        assert call(args(D=96)) == -2
        assert call(args(Hq=60)) == -2
        assert call(args(pool=31)) == -2            # contiguous pools too small for B*max_pages
        assert call(args(wsb=need - 1)) == -4
        assert call(args(ws=None)) == -4
        assert call(args(q=P(0x50002))) == -3
        assert call(args(B=0)) == 0                 # empty batch: no-op

    lib.lynx_verify_attention_workspace_size.restype = ctypes.c_size_t
    lib.lynx_verify_attention_workspace_size.argtypes = [ctypes.c_int32] * 6
    vneed = lib.lynx_verify_attention_workspace_size(2, 4, 8, 64, 128, 16)
    assert vneed > lib.lynx_decode_attention_workspace_size(2, 8, 64, 128, 16)
    assert lib.lynx_verify_attention_workspace_size(2, 0, 8, 64, 128, 16) == 0    # tq < 1
    assert lib.lynx_verify_attention_workspace_size(2, 65, 8, 64, 128, 16) == 0   # tq > 64
    for name in ("lynx_verify_attention", "lynx_draft_attention"):
        fn = getattr(lib, name)
        fn.argtypes = [P, ctypes.c_int32, ctypes.POINTER(CPlanes), ctypes.POINTER(CPlanes), P, P, P,
                       P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_int64, ctypes.c_float, P, P, ctypes.c_size_t, P]
        q, out, ws, tk, tv, tl = (P(0x50000), P(0x60000), P(0x70000), P(0x80000), P(0x90000),
                                  P(0xA0000))
        args = lambda **kw: dict(dict(q=q, tq=4, bt=None, pt=None, tk=tk, tv=tv, tl=tl, B=2, H=8,
                                      Hq=64, D=128, mp=16, pool=32, ws=ws, wsb=vneed), **kw)

        def vcall(a):
            return fn(a["q"], a["tq"], ctypes.byref(pl), ctypes.byref(pl), a["bt"], a["pt"], a["tk"],
                      a["tv"], a["tl"], a["B"], a["H"], a["Hq"], a["D"], a["mp"], a["pool"], 0.088,
                      out, a["ws"], a["wsb"], None)
        assert vcall(args(q=None)) == -1
        assert vcall(args(tk=None)) == -1
        assert vcall(args(tl=None)) == -1
        assert vcall(args(tq=0)) == -2
        assert vcall(args(tq=65)) == -2
        assert vcall(args(D=96)) == -2
        assert vcall(args(pool=31)) == -2
        assert vcall(args(wsb=vneed - 1)) == -4
        assert vcall(args(tv=P(0x90008))) == -3
        assert vcall(args(B=0)) == 0


def test_verify_workspace_follows_the_split_rule(lib):
    """The verify workspace holds one (m, l, o) partial per (query row, KV
    head, part, query head): parts = the page runs plus the bf16 tail's.
    Runs are sized so that at most 256 blocks cover the call (2048 for the
    VALU kernel of groups above 8) when the work items fit in that many,
    one run per item beyond: with GQA group 8 and 3 or more query tokens an
    item (a block's rows) is 16 rows (tq <= 16) or 32 of a request and a KV
    head, otherwise one row.  m is fp64, l fp32, o 128 fp32."""
    lib.lynx_verify_attention_workspace_size.restype = ctypes.c_size_t
    lib.lynx_verify_attention_workspace_size.argtypes = [ctypes.c_int32] * 6

    def expected(requests, tq, H, Hq, max_pages):
        g = Hq // H
        if g == 8 and tq >= 3:
            rows_per_block = 16 if tq <= 16 else 32
            units = requests * H * -(-tq // rows_per_block)
        else:
            units = requests * tq * H
        target = 256 if g <= 8 else 2048
        runs = 1 if units >= target else target // units
        pps = min(max(-(-max_pages // runs), 1), max_pages)
        parts = -(-max_pages // pps) + 1
        n = requests * tq * H * parts * g
        return ((n + 1) & ~1) * 8 + ((n + 3) & ~3) * 4 + n * 128 * 4

    for requests, tq, H, Hq, max_pages in ((1, 64, 8, 64, 128), (1, 33, 8, 64, 128),
                                           (1, 17, 8, 64, 128), (1, 16, 8, 64, 128),
                                           (1, 5, 8, 64, 128), (1, 4, 8, 64, 128),
                                           (1, 2, 8, 64, 128), (3, 1, 8, 64, 128),
                                           (3, 37, 2, 16, 4), (2, 7, 2, 32, 3),
                                           (1, 64, 2, 16, 32), (4, 1, 8, 64, 2),
                                           (2, 3, 4, 64, 64)):
        got = lib.lynx_verify_attention_workspace_size(requests, tq, H, Hq, 128, max_pages)
        assert got == expected(requests, tq, H, Hq, max_pages), (requests, tq, H, Hq, max_pages)


def test_cut_entry_points_reject_bad_arguments(lib):
    P = ctypes.c_void_p
    lib.lynx_split_stream_bytes.restype = ctypes.c_size_t
    lib.lynx_split_stream_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    assert lib.lynx_split_stream_bytes(3, 2, 5) == 3 * 2 * 5 * 4096
    assert lib.lynx_split_stream_bytes(3, 2, 0) == 0
    lib.lynx_split_planes.argtypes = [ctypes.POINTER(CPlanes), ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, P, P, P]
    pl = _fake_planes()
    a, r = P(0x80000), P(0x90000)
    assert lib.lynx_split_planes(ctypes.byref(pl), 4, 8, 128, 0, a, r, None) == -7   # bits 0
    assert lib.lynx_split_planes(ctypes.byref(pl), 4, 8, 128, 8, a, r, None) == -7   # bits 8
    assert lib.lynx_split_planes(ctypes.byref(pl), 4, 8, 64, 3, a, r, None) == -2
    assert lib.lynx_split_planes(ctypes.byref(pl), 4, 8, 128, 3, None, r, None) == -1
    assert lib.lynx_split_planes(ctypes.byref(pl), 4, 8, 128, 3, P(0x80004), r, None) == -3
    assert lib.lynx_split_planes(ctypes.byref(pl), 0, 8, 128, 3, None, None, None) == 0
    lib.lynx_dequantize_split.argtypes = [P, P, ctypes.c_int32, ctypes.POINTER(CPlanes),
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, P, P]
    out = P(0xA0000)
    assert lib.lynx_dequantize_split(a, None, 9, ctypes.byref(pl), 4, 8, 128, 0, out, None) == -7
    assert lib.lynx_dequantize_split(a, None, 3, ctypes.byref(pl), 4, 8, 128, 2, out, None) == -7
    assert lib.lynx_dequantize_split(None, None, 3, ctypes.byref(pl), 4, 8, 128, 0, out, None) == -1
    assert lib.lynx_dequantize_split(a, P(0x90008), 3, ctypes.byref(pl), 4, 8, 128, 1, out, None) == -3
    assert lib.lynx_dequantize_split(a, None, 3, ctypes.byref(pl), 0, 8, 128, 1, None, None) == 0

    # the encoder writing a cut directly
    lib.lynx_quantize_pages_split.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(CPlanes), P]
    kvp = P(0x20000)
    assert lib.lynx_quantize_pages_split(kvp, 4, 8, 128, 0, 0, ctypes.byref(pl), None) == -7
    assert lib.lynx_quantize_pages_split(kvp, 4, 8, 128, 0, 8, ctypes.byref(pl), None) == -7
    assert lib.lynx_quantize_pages_split(kvp, 4, 8, 128, 2, 3, ctypes.byref(pl), None) == -7
    assert lib.lynx_quantize_pages_split(kvp, 4, 8, 96, 0, 3, ctypes.byref(pl), None) == -2
    assert lib.lynx_quantize_pages_split(None, 4, 8, 128, 0, 3, ctypes.byref(pl), None) == -1
    assert lib.lynx_quantize_pages_split(P(0x20008), 4, 8, 128, 0, 3, ctypes.byref(pl), None) == -3
    assert lib.lynx_quantize_pages_split(None, 0, 8, 128, 0, 3, ctypes.byref(pl), None) == 0

    # fused attention over cut streams
    lib.lynx_decode_attention_split.argtypes = [P, ctypes.POINTER(CPlanes), ctypes.POINTER(CPlanes),
                                                ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int64, ctypes.c_float, P, P,
                                                P, ctypes.c_size_t, P]
    kp, vp = _fake_planes(0x10000), _fake_planes(0x40000)
    q, o, ws = P(0x20000), P(0x30000), P(0x50000)

    def acall(bits=3, full=1, B=2, H=8, Hq=64, D=128, mp=4, pool=8, qq=q, k=kp, v=vp, wsb=1 << 20):
        return lib.lynx_decode_attention_split(qq, ctypes.byref(k), ctypes.byref(v), bits, full, None,
                                               None, B, H, Hq, D, mp, pool, 0.088, o, None, ws, wsb,
                                               None)
    assert acall(bits=0) == -7
    assert acall(bits=8) == -7
    assert acall(D=64) == -2
    assert acall(Hq=96) == -2            # group 12: cut streams need the matrix-core kernel
    assert acall(pool=7) == -2           # batch * max_pages pages must exist without a block table
    assert acall(qq=None) == -1
    nores = CPlanes(kp.anchor, None, kp.page_min, kp.page_range, kp.chunk_mean, kp.chunk_maxabs)
    assert acall(k=nores) == -1          # the full code reads the residual stream
    assert acall(wsb=0) == -4
    assert acall(B=0) == 0


def test_status_strings(lib):
    lib.lynx_status_string.restype = ctypes.c_char_p
    for code in range(-8, 1):
        assert lib.lynx_status_string(code)
    assert lib.lynx_status_string(-99) == b"unknown status"


def test_code_thresholds_agree_with_the_oracle(lib):
    """T[k] is the first fp32 u the oracle puts on level >= k (away from the
    oracle's 2^-20 boundary window)."""
    buf = (ctypes.c_float * 128)()
    lib.lynx_code_thresholds(buf)
    T = np.array(buf[:], np.float32)
    assert T[0] == 0.0 and np.all(np.diff(T) > 0) and T[-1] < 1.0
    below = np.nextafter(T[1:], np.float32(0.0)).astype(np.float32)
    q_at, f_at = oracle.codes(T[1:])
    q_below, f_below = oracle.codes(below)
    k = np.arange(1, 128)
    ok_at = (q_at == k) | (f_at != 0)
    ok_below = (q_below == k - 1) | (f_below != 0)
    assert ok_at.all() and ok_below.all()


def test_decode_table_agrees_with_the_oracle(lib):
    buf = (ctypes.c_float * 256)()
    lib.lynx_decode_table(buf)
    y = np.array(buf[:], np.float32)
    ref = oracle.yhat(np.arange(-128, 128))
    assert np.array_equal(y, ref.astype(np.float32))     # correctly rounded fp32 of the fp64 value


def test_static_scratch_call_rejects_shapes_beyond_its_scratch(lib):
    """lynx_decode_attention_full_static: shape errors and shapes whose
    partials exceed the library's static scratch are refused on the host,
    before any device is touched."""
    P = ctypes.c_void_p
    lib.lynx_decode_attention_full_static.argtypes = [
        P, ctypes.POINTER(CPlanes), ctypes.POINTER(CPlanes), P, P, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, P, P, P]
    lib.lynx_decode_attention_workspace_size.argtypes = [ctypes.c_int32] * 5
    lib.lynx_decode_attention_workspace_size.restype = ctypes.c_size_t
    kp, vp = _fake_planes(0x10000), _fake_planes(0x40000)

    def call(B, H=1, Hq=8, D=128, mp=4):
        return lib.lynx_decode_attention_full_static(P(0x20000), ctypes.byref(kp), ctypes.byref(vp),
                                                     P(0x50000), None, B, H, Hq, D, mp, 1 << 20,
                                                     0.088, P(0x30000), None, None)
    cap = 32 << 20
    big = 16384
    assert lib.lynx_decode_attention_workspace_size(big, 1, 8, 128, 4) > cap
    assert call(big) == -8
    assert call(4, D=64) == -2
    assert call(4, H=3, Hq=8) == -2
    assert call(0) == 0
