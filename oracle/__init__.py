"""CPU oracle for Lynx progressive KV-cache quantization (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``long_context_serving_amd``) never imports it, and it
never imports the product path.

This module is argument marshalling only: every step of the method runs in
``lynx_oracle.c`` (see its header for the passages it follows and the
readings it takes).  Arrays are numpy; bf16 tensors travel as their uint16
bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

PAGE = 256
CHUNK = 32
NCHUNK = PAGE // CHUNK
FLAG_NEAR_HALF = 1
FLAG_SUM_INEXACT = 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_encode.argtypes = [P, i64, i32, i32, P, P, P, P, P, P, i32]
    lib.oracle_encode.restype = i32
    lib.oracle_tau.argtypes = [P, i64, P]
    lib.oracle_tau.restype = None
    lib.oracle_codes.argtypes = [P, P, i64, P, P, i32]
    lib.oracle_codes.restype = None
    lib.oracle_yhat.argtypes = [P, i64, P]
    lib.oracle_yhat.restype = None
    lib.oracle_split.argtypes = [P, i64, P, P]
    lib.oracle_split.restype = None
    lib.oracle_join.argtypes = [P, P, i64, P]
    lib.oracle_join.restype = None
    lib.oracle_dequant.argtypes = [P, P, P, P, P, P, i64, i32, i32, P, i32]
    lib.oracle_dequant.restype = i32
    lib.oracle_attention.argtypes = [P, P, P, i32, i64, i32, i32, i32,
                                     ctypes.c_double, P, P, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_split_bits.argtypes = [P, i64, i32, P, P]
    lib.oracle_split_bits.restype = i32
    lib.oracle_join_bits.argtypes = [P, P, i64, i32, P]
    lib.oracle_join_bits.restype = i32
    lib.oracle_dequant_bits.argtypes = [P, P, i32, P, P, P, P, i64, i32, i32, P, i32]
    lib.oracle_dequant_bits.restype = i32
    lib.oracle_prefix_attention.argtypes = [P, P, P, P, i32, i32, i64, i32, i32, i32,
                                            ctypes.c_double, P, i32]
    lib.oracle_prefix_attention.restype = i32
    lib.oracle_uniform_codes.argtypes = [P, i64, i64, i32, P]
    lib.oracle_uniform_codes.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def encode(x_bf16, nthreads: int = 0):
    """Quantize bf16 pages.  x_bf16: uint16 [P][256][H][D].

    Returns a dict with codes (int8 [P][256][H][D]), page_min/page_range
    (fp32 [P][H][D]), chunk_mean/chunk_maxabs (fp32 [P][H][8][D]) and flags
    (uint8 [P][256][H][D], FLAG_* bits).
    """
    x = _c(x_bf16, np.uint16)
    if x.ndim != 4 or x.shape[1] != PAGE:
        raise ValueError("x must be [P][256][H][D]")
    P, _, H, D = x.shape
    out = dict(
        codes=np.empty(x.shape, np.int8),
        page_min=np.empty((P, H, D), np.float32),
        page_range=np.empty((P, H, D), np.float32),
        chunk_mean=np.empty((P, H, NCHUNK, D), np.float32),
        chunk_maxabs=np.empty((P, H, NCHUNK, D), np.float32),
        flags=np.empty(x.shape, np.uint8),
    )
    rc = _load().oracle_encode(_ptr(x), P, H, D, _ptr(out["codes"]), _ptr(out["page_min"]),
                               _ptr(out["page_range"]), _ptr(out["chunk_mean"]),
                               _ptr(out["chunk_maxabs"]), _ptr(out["flags"]), nthreads)
    if rc != 0:
        raise ValueError("oracle_encode rejected its arguments")
    return out


def tau(u):
    u = _c(u, np.float32)
    out = np.empty(u.shape, np.float64)
    _load().oracle_tau(_ptr(u), u.size, _ptr(out))
    return out


def codes(u, negative=None, nthreads: int = 0):
    """8-bit codes for magnitudes u in [0,1] with an optional sign mask."""
    u = _c(u, np.float32)
    neg = None if negative is None else _c(negative, np.uint8)
    q = np.empty(u.shape, np.int8)
    flag = np.empty(u.shape, np.uint8)
    _load().oracle_codes(_ptr(u), _ptr(neg), u.size, _ptr(q), _ptr(flag), nthreads)
    return q, flag


def yhat(q):
    q = _c(q, np.int32)
    out = np.empty(q.shape, np.float64)
    _load().oracle_yhat(_ptr(q), q.size, _ptr(out))
    return out


def split(q):
    q = _c(q, np.int8)
    a = np.empty(q.shape, np.int8)
    r = np.empty(q.shape, np.uint8)
    _load().oracle_split(_ptr(q), q.size, _ptr(a), _ptr(r))
    return a, r


def join(anchor, residual=None):
    """Full code 16a + r, or the draft code 16a + 7 when residual is None."""
    a = _c(anchor, np.int8)
    r = None if residual is None else _c(residual, np.uint8)
    q = np.empty(a.shape, np.int32)
    _load().oracle_join(_ptr(a), _ptr(r), a.size, _ptr(q))
    return q


def dequant(anchor, residual, scales, nthreads: int = 0):
    """xhat (float64 [P][256][H][D]); residual None = anchor-only draft."""
    a = _c(anchor, np.int8)
    r = None if residual is None else _c(residual, np.uint8)
    P, _, H, D = a.shape
    pm = _c(scales["page_min"], np.float32)
    pr = _c(scales["page_range"], np.float32)
    cm = _c(scales["chunk_mean"], np.float32)
    cs = _c(scales["chunk_maxabs"], np.float32)
    out = np.empty(a.shape, np.float64)
    rc = _load().oracle_dequant(_ptr(a), _ptr(r), _ptr(pm), _ptr(pr), _ptr(cm), _ptr(cs),
                                P, H, D, _ptr(out), nthreads)
    if rc != 0:
        raise ValueError("oracle_dequant rejected its arguments")
    return out


def attention(q, k, v, sm_scale: float, want_logits: bool = False, nthreads: int = 0):
    """Brute-force single-query GQA attention in float64.

    q: [B][Hq][D]; k, v: [B][T][H][D].  Returns out [B][Hq][D] (and the
    scaled logits [B][Hq][T] when want_logits).
    """
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    B, Hq, D = q.shape
    _, T, H, _ = k.shape
    out = np.empty((B, Hq, D), np.float64)
    logits = np.empty((B, Hq, T), np.float64) if want_logits else None
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), B, T, H, Hq, D, float(sm_scale),
                                  _ptr(out), _ptr(logits), nthreads)
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return (out, logits) if want_logits else out


def split_bits(q, anchor_bits: int):
    """A b + (8 - b) cut of the 8-bit codes: (anchor int8, residual uint8)."""
    q = _c(q, np.int8)
    a = np.empty(q.shape, np.int8)
    r = np.empty(q.shape, np.uint8)
    if _load().oracle_split_bits(_ptr(q), q.size, anchor_bits, _ptr(a), _ptr(r)) != 0:
        raise ValueError("anchor_bits must be 1 .. 8")
    return a, r


def join_bits(anchor, residual, anchor_bits: int):
    """Full code (residual given) or draft code (residual None) of a cut."""
    a = _c(anchor, np.int8)
    r = None if residual is None else _c(residual, np.uint8)
    q = np.empty(a.shape, np.int32)
    if _load().oracle_join_bits(_ptr(a), _ptr(r), a.size, anchor_bits, _ptr(q)) != 0:
        raise ValueError("anchor_bits must be 1 .. 8")
    return q


def dequant_bits(anchor, residual, anchor_bits: int, scales, nthreads: int = 0):
    """xhat (float64 [P][256][H][D]) of a b + (8 - b) cut; residual None = draft."""
    a = _c(anchor, np.int8)
    r = None if residual is None else _c(residual, np.uint8)
    P, _, H, D = a.shape
    pm = _c(scales["page_min"], np.float32)
    pr = _c(scales["page_range"], np.float32)
    cm = _c(scales["chunk_mean"], np.float32)
    cs = _c(scales["chunk_maxabs"], np.float32)
    out = np.empty(a.shape, np.float64)
    rc = _load().oracle_dequant_bits(_ptr(a), _ptr(r), anchor_bits, _ptr(pm), _ptr(pr), _ptr(cm),
                                     _ptr(cs), P, H, D, _ptr(out), nthreads)
    if rc != 0:
        raise ValueError("oracle_dequant_bits rejected its arguments")
    return out


def prefix_attention(q, k, v, visible, sm_scale: float, nthreads: int = 0):
    """Several query tokens per request, token i over the first visible[b][i]
    cached tokens, in float64.

    q: [B][Tq][Hq][D]; k, v: [B][T][H][D]; visible: [B][Tq].  Returns
    out [B][Tq][Hq][D].
    """
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    vis = _c(visible, np.int64)
    B, Tq, Hq, D = q.shape
    _, T, H, _ = k.shape
    if vis.shape != (B, Tq):
        raise ValueError("visible must be [B][Tq]")
    out = np.empty((B, Tq, Hq, D), np.float64)
    rc = _load().oracle_prefix_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(vis), B, Tq, T, H, Hq, D,
                                         float(sm_scale), _ptr(out), nthreads)
    if rc != 0:
        raise ValueError("oracle_prefix_attention rejected its arguments")
    return out


def verify_attention(q_bits, pages_k, pages_v, tail_k_bits, tail_v_bits, tail_len, sm_scale: float,
                     nthreads: int = 0):
    """Attention of the Tq newest tokens of each request over its cache.

    q_bits [B][Tq][Hq][D] bf16 bits.  pages_k / pages_v: per request, the
    dequantized pages as float64 [n_b * 256][H][D] (n_b may be 0).
    tail_k_bits / tail_v_bits: per request, bf16 bits [>= tail_len[b]][H][D];
    the last Tq tail tokens are the query tokens themselves, so token i sees
    every page token and tail tokens 0 .. tail_len - Tq + i.
    Returns out [B][Tq][Hq][D] (float64).
    """
    qf = bf16_bits_to_float(q_bits).astype(np.float64)
    B, Tq = qf.shape[0], qf.shape[1]
    outs = []
    for b in range(B):
        n_tail = int(tail_len[b])
        if n_tail < Tq:
            raise ValueError("the tail must hold the query tokens")
        tk = bf16_bits_to_float(np.asarray(tail_k_bits[b])[:n_tail]).astype(np.float64)
        tv = bf16_bits_to_float(np.asarray(tail_v_bits[b])[:n_tail]).astype(np.float64)
        k = np.concatenate([np.asarray(pages_k[b], np.float64), tk])[None]
        v = np.concatenate([np.asarray(pages_v[b], np.float64), tv])[None]
        n_pages_tok = len(pages_k[b])
        vis = (n_pages_tok + n_tail - Tq + 1 + np.arange(Tq, dtype=np.int64))[None]
        outs.append(prefix_attention(qf[b:b + 1], k, v, vis, sm_scale, nthreads)[0])
    return np.stack(outs)


def uniform_codes(x, bits: int):
    """Uniform `bits`-bit grid shared by all columns of each row of x [rows][cols]."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    out = np.empty(x.shape, np.int32)
    _load().oracle_uniform_codes(_ptr(x), rows, cols, bits, _ptr(out))
    return out


def bf16_bits_to_float(x_bf16):
    """Exact widening of bf16 bit patterns to float32 (no arithmetic)."""
    return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)
