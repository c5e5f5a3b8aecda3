"""Thin Python binding of liblynx (include/lynx.h).

Argument marshalling only: every step of the method runs in the HIP
library.  PyTorch supplies device memory and streams.  If the library has
not been built this module raises on import -- there is no fallback path.
"""
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblynx.so")

PAGE = 256
CHUNK = 32
CHUNKS = 8
HEAD_DIM = 128
MAX_GROUP = 16
MAX_QUERY_TOKENS = 64
TAIL_TOKENS = 320
ROLE_KEY = 0
ROLE_VALUE = 1

LYNX_OK = 0

if not os.path.exists(LIB_PATH):
    raise ImportError("liblynx.so is not built (%s); run `python -m long_context_serving_amd.build` "
                      "or __graft_entry__.build()" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)


class _CPlanes(ctypes.Structure):
    _fields_ = [("anchor", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("page_min", ctypes.c_void_p), ("page_range", ctypes.c_void_p),
                ("chunk_mean", ctypes.c_void_p), ("chunk_maxabs", ctypes.c_void_p)]


_P = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_lib.lynx_plane_bytes.argtypes = [_i64, _i32]
_lib.lynx_plane_bytes.restype = _sz
_lib.lynx_page_scale_bytes.argtypes = [_i64, _i32]
_lib.lynx_page_scale_bytes.restype = _sz
_lib.lynx_chunk_scale_bytes.argtypes = [_i64, _i32]
_lib.lynx_chunk_scale_bytes.restype = _sz
_lib.lynx_quantize_pages.argtypes = [_P, _i64, _i32, _i32, _i32, ctypes.POINTER(_CPlanes), _P]
_lib.lynx_quantize_pages.restype = ctypes.c_int
_lib.lynx_quantize_kv_pages.argtypes = [_P, _P, _i64, _i32, _i32, ctypes.POINTER(_CPlanes),
                                        ctypes.POINTER(_CPlanes), _P]
_lib.lynx_quantize_kv_pages.restype = ctypes.c_int
for _name in ("lynx_dequantize_anchor", "lynx_dequantize_full"):
    getattr(_lib, _name).argtypes = [ctypes.POINTER(_CPlanes), _i64, _i32, _i32, _i32, _P, _P]
    getattr(_lib, _name).restype = ctypes.c_int
_lib.lynx_decode_attention_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
_lib.lynx_decode_attention_workspace_size.restype = _sz
for _name in ("lynx_decode_attention_anchor", "lynx_decode_attention_full"):
    getattr(_lib, _name).argtypes = [_P, ctypes.POINTER(_CPlanes), ctypes.POINTER(_CPlanes), _P, _P,
                                     _i32, _i32, _i32, _i32, _i32, _i64, ctypes.c_float, _P, _P, _P,
                                     _sz, _P]
    getattr(_lib, _name).restype = ctypes.c_int
_lib.lynx_decode_attention_full_static.argtypes = [_P, ctypes.POINTER(_CPlanes),
                                                   ctypes.POINTER(_CPlanes), _P, _P, _i32, _i32,
                                                   _i32, _i32, _i32, _i64, ctypes.c_float, _P, _P,
                                                   _P]
_lib.lynx_decode_attention_full_static.restype = ctypes.c_int
_lib.lynx_verify_attention_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.lynx_verify_attention_workspace_size.restype = _sz
for _name in ("lynx_verify_attention", "lynx_draft_attention"):
    getattr(_lib, _name).argtypes = [_P, _i32, ctypes.POINTER(_CPlanes), ctypes.POINTER(_CPlanes),
                                     _P, _P, _P, _P, _P, _i32, _i32, _i32, _i32, _i32, _i64,
                                     ctypes.c_float, _P, _P, _sz, _P]
    getattr(_lib, _name).restype = ctypes.c_int
_lib.lynx_split_stream_bytes.argtypes = [_i64, _i32, _i32]
_lib.lynx_split_stream_bytes.restype = _sz
_lib.lynx_split_planes.argtypes = [ctypes.POINTER(_CPlanes), _i64, _i32, _i32, _i32, _P, _P, _P]
_lib.lynx_split_planes.restype = ctypes.c_int
_lib.lynx_dequantize_split.argtypes = [_P, _P, _i32, ctypes.POINTER(_CPlanes), _i64, _i32, _i32,
                                       _i32, _P, _P]
_lib.lynx_dequantize_split.restype = ctypes.c_int
_lib.lynx_quantize_pages_split.argtypes = [_P, _i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_CPlanes), _P]
_lib.lynx_quantize_pages_split.restype = ctypes.c_int
_lib.lynx_decode_attention_split.argtypes = [_P, ctypes.POINTER(_CPlanes), ctypes.POINTER(_CPlanes),
                                             _i32, _i32, _P, _P, _i32, _i32, _i32, _i32, _i32, _i64,
                                             ctypes.c_float, _P, _P, _P, _sz, _P]
_lib.lynx_decode_attention_split.restype = ctypes.c_int
_lib.lynx_status_string.argtypes = [ctypes.c_int]
_lib.lynx_status_string.restype = ctypes.c_char_p
_lib.lynx_code_thresholds.argtypes = [_P]
_lib.lynx_code_thresholds.restype = None
_lib.lynx_decode_table.argtypes = [_P]
_lib.lynx_decode_table.restype = None
_lib.lynx_selftest_code_map.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _P, _P]
_lib.lynx_selftest_code_map.restype = ctypes.c_int
_lib.lynx_version.argtypes = []
_lib.lynx_version.restype = ctypes.c_char_p


class LynxError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, _lib.lynx_status_string(status).decode(), status))
        self.status = status


def _check(status: int, what: str):
    if status != LYNX_OK:
        raise LynxError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def version() -> str:
    return _lib.lynx_version().decode()


def code_thresholds() -> "list[float]":
    buf = (ctypes.c_float * 128)()
    _lib.lynx_code_thresholds(ctypes.cast(buf, _P))
    return list(buf)


def decode_table() -> "list[float]":
    buf = (ctypes.c_float * 256)()
    _lib.lynx_decode_table(ctypes.cast(buf, _P))
    return list(buf)


def selftest_code_map(begin_bits: int = 0, end_bits: int = 0x3F800001, stream=None) -> int:
    """Number of fp32 u in [begin, end) bit patterns where the encoder's fast
    level path disagrees with the exact threshold count (runs on the GPU)."""
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    _check(_lib.lynx_selftest_code_map(begin_bits, end_bits, _ptr(cnt), _stream(stream)),
           "lynx_selftest_code_map")
    return int(cnt.item())


@dataclass
class Planes:
    """One encoded K (role 0) or V (role 1) tensor of one layer.

    anchor / residual: uint8, 16 KiB per (page, head) each, layout by role
    (see include/lynx.h); scales: fp32 [P][H][128] and [P][H][8][128].
    """
    anchor: torch.Tensor
    residual: Optional[torch.Tensor]
    page_min: torch.Tensor
    page_range: torch.Tensor
    chunk_mean: torch.Tensor
    chunk_maxabs: torch.Tensor
    num_pages: int
    heads: int
    role: int

    def c(self) -> _CPlanes:
        return _CPlanes(*(None if t is None else t.data_ptr() for t in
                          (self.anchor, self.residual, self.page_min, self.page_range,
                           self.chunk_mean, self.chunk_maxabs)))

    def without_residual(self) -> "Planes":
        return Planes(self.anchor, None, self.page_min, self.page_range, self.chunk_mean,
                      self.chunk_maxabs, self.num_pages, self.heads, self.role)

    def nbytes(self, with_residual: bool = True) -> int:
        n = self.anchor.numel() + self.page_min.numel() * 4 * 2 + self.chunk_mean.numel() * 4 * 2
        if with_residual and self.residual is not None:
            n += self.residual.numel()
        return n


def alloc_planes(num_pages: int, heads: int, role: int, device="cuda") -> Planes:
    pb = _lib.lynx_plane_bytes(num_pages, heads)
    return Planes(
        anchor=torch.empty(pb, dtype=torch.uint8, device=device),
        residual=torch.empty(pb, dtype=torch.uint8, device=device),
        page_min=torch.empty((num_pages, heads, HEAD_DIM), dtype=torch.float32, device=device),
        page_range=torch.empty((num_pages, heads, HEAD_DIM), dtype=torch.float32, device=device),
        chunk_mean=torch.empty((num_pages, heads, CHUNKS, HEAD_DIM), dtype=torch.float32, device=device),
        chunk_maxabs=torch.empty((num_pages, heads, CHUNKS, HEAD_DIM), dtype=torch.float32, device=device),
        num_pages=num_pages, heads=heads, role=role)


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("expected bf16 (or its 16-bit patterns), got %s" % x.dtype)


def quantize_pages(kv: torch.Tensor, role: int, out: Optional[Planes] = None, stream=None) -> Planes:
    """Encode bf16 pages [P][256][H][128] into anchor/residual planes + scales."""
    kv = _bf16_bits(kv)
    if kv.dim() != 4 or kv.shape[1] != PAGE or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [P][256][H][128] bf16 tensor")
    P, _, H, D = kv.shape
    if out is None:
        out = alloc_planes(P, H, role, kv.device)
    cp = out.c()
    _check(_lib.lynx_quantize_pages(_ptr(kv), P, H, D, role, ctypes.byref(cp), _stream(stream)),
           "lynx_quantize_pages")
    return out


def quantize_kv_pages(k: torch.Tensor, v: torch.Tensor, out_k: Optional[Planes] = None,
                      out_v: Optional[Planes] = None, stream=None):
    """Encode a layer's K and V pages (bf16 [P][256][H][128] each) in one
    launch; the same planes as quantize_pages on each.  Returns (K, V) planes."""
    k, v = _bf16_bits(k), _bf16_bits(v)
    for name, x in (("k", k), ("v", v)):
        if x.dim() != 4 or x.shape[1] != PAGE or not x.is_contiguous():
            raise ValueError("%s must be a contiguous [P][256][H][128] bf16 tensor" % name)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    P, _, H, D = k.shape
    if out_k is None:
        out_k = alloc_planes(P, H, ROLE_KEY, k.device)
    if out_v is None:
        out_v = alloc_planes(P, H, ROLE_VALUE, v.device)
    if out_k.role != ROLE_KEY or out_v.role != ROLE_VALUE:
        raise ValueError("out_k must be key planes and out_v value planes")
    ck, cv = out_k.c(), out_v.c()
    _check(_lib.lynx_quantize_kv_pages(_ptr(k), _ptr(v), P, H, D, ctypes.byref(ck), ctypes.byref(cv),
                                       _stream(stream)), "lynx_quantize_kv_pages")
    return out_k, out_v


def dequantize(planes: Planes, full: bool = True, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """fp32 reconstruction [P][256][H][128]; full=False is the anchor-only draft."""
    P, H = planes.num_pages, planes.heads
    if out is None:
        out = torch.empty((P, PAGE, H, HEAD_DIM), dtype=torch.float32, device=planes.anchor.device)
    cp = planes.c()
    fn = _lib.lynx_dequantize_full if full else _lib.lynx_dequantize_anchor
    _check(fn(ctypes.byref(cp), P, H, HEAD_DIM, planes.role, _ptr(out), _stream(stream)),
           "lynx_dequantize_%s" % ("full" if full else "anchor"))
    return out


def workspace_size(batch: int, heads: int, q_heads: int, max_pages: int) -> int:
    return int(_lib.lynx_decode_attention_workspace_size(batch, heads, q_heads, HEAD_DIM, max_pages))


def alloc_workspace(batch: int, heads: int, q_heads: int, max_pages: int,
                    device="cuda") -> torch.Tensor:
    """Decode-attention workspace of the size the library asks for."""
    need = workspace_size(batch, heads, q_heads, max_pages)
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=device)


def decode_attention(q: torch.Tensor, k: Planes, v: Planes, max_pages: int, full: bool = True,
                     block_table: Optional[torch.Tensor] = None,
                     seq_lens: Optional[torch.Tensor] = None,
                     sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     scores: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Single-query GQA decode attention over the compact planes.

    q: bf16 [B][Hq][128].  k (role 0) and v (role 1) are page pools; request b
    reads pool pages block_table[b] (or b*max_pages + i when block_table is
    None).  Returns fp32 [B][Hq][128].
    """
    q = _bf16_bits(q)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][Hq][128] bf16 tensor")
    B, Hq, D = q.shape
    H = k.heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, Hq, max_pages, q.device)
    fn = _lib.lynx_decode_attention_full if full else _lib.lynx_decode_attention_anchor
    kc, vc = k.c(), v.c()
    _check(fn(_ptr(q), ctypes.byref(kc), ctypes.byref(vc), _ptr(block_table), _ptr(seq_lens),
              B, H, Hq, D, max_pages, min(k.num_pages, v.num_pages), float(sm_scale), _ptr(out),
              _ptr(scores), _ptr(workspace), workspace.numel(), _stream(stream)),
           "lynx_decode_attention_%s" % ("full" if full else "anchor"))
    return out


def decode_attention_full_static(q: torch.Tensor, k: Planes, v: Planes, max_pages: int,
                                 block_table: Optional[torch.Tensor] = None,
                                 seq_lens: Optional[torch.Tensor] = None,
                                 sm_scale: Optional[float] = None,
                                 out: torch.Tensor = None, scores: Optional[torch.Tensor] = None,
                                 stream=None) -> torch.Tensor:
    """decode_attention(full=True) with the library's static scratch in
    place of a workspace (lynx_decode_attention_full_static): the library
    allocates nothing; `out` must be given.  Calls on one GPU must not
    overlap."""
    q = _bf16_bits(q)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][Hq][128] bf16 tensor")
    if out is None:
        raise ValueError("out must be given: this call allocates nothing")
    B, Hq, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    kc, vc = k.c(), v.c()
    _check(_lib.lynx_decode_attention_full_static(
        _ptr(q), ctypes.byref(kc), ctypes.byref(vc), _ptr(block_table), _ptr(seq_lens), B, k.heads,
        Hq, D, max_pages, min(k.num_pages, v.num_pages), float(sm_scale), _ptr(out), _ptr(scores),
        _stream(stream)), "lynx_decode_attention_full_static")
    return out


def alloc_verify_workspace(batch: int, tq: int, heads: int, q_heads: int, max_pages: int,
                           device="cuda") -> torch.Tensor:
    """Workspace for verify_attention (its contents need no initialisation)."""
    n = _lib.lynx_verify_attention_workspace_size(batch, tq, heads, q_heads, HEAD_DIM, max_pages)
    if n == 0:
        raise ValueError("unsupported verify attention shape")
    return torch.zeros((n + 15) // 16 * 16, dtype=torch.uint8, device=device)


def alloc_tail(batch: int, heads: int, device="cuda") -> torch.Tensor:
    """bf16 tail buffer [B][TAIL_TOKENS][H][128] (as int16 bit patterns)."""
    return torch.zeros((batch, TAIL_TOKENS, heads, HEAD_DIM), dtype=torch.int16, device=device)


def verify_attention(q: torch.Tensor, k: Planes, v: Planes, max_pages: int,
                     tail_k: torch.Tensor, tail_v: torch.Tensor, tail_len: torch.Tensor,
                     full: bool = True, block_table: Optional[torch.Tensor] = None,
                     page_tokens: Optional[torch.Tensor] = None,
                     sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of each request's tq newest tokens over its pages and bf16 tail.

    q: bf16 [B][tq][Hq][128]; tail_k / tail_v: bf16 [B][TAIL_TOKENS][H][128];
    tail_len: int32 [B] on the device.  full=True is the verify pass over
    Q_full, full=False the draft (anchor plane only).  Returns fp32
    [B][tq][Hq][128].
    """
    q = _bf16_bits(q)
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][tq][Hq][128] bf16 tensor")
    B, tq, Hq, D = q.shape
    H = k.heads
    tk, tv = _bf16_bits(tail_k), _bf16_bits(tail_v)
    for t in (tk, tv):
        if tuple(t.shape) != (B, TAIL_TOKENS, H, HEAD_DIM) or not t.is_contiguous():
            raise ValueError("tail tensors must be contiguous [B][%d][H][128] bf16" % TAIL_TOKENS)
    if tail_len.dtype != torch.int32 or tail_len.numel() != B:
        raise ValueError("tail_len must be int32 [B]")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, tq, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_verify_workspace(B, tq, H, Hq, max_pages, q.device)
    fn = _lib.lynx_verify_attention if full else _lib.lynx_draft_attention
    kc, vc = k.c(), v.c()
    _check(fn(_ptr(q), tq, ctypes.byref(kc), ctypes.byref(vc), _ptr(block_table), _ptr(page_tokens),
              _ptr(tk), _ptr(tv), _ptr(tail_len), B, H, Hq, D, max_pages,
              min(k.num_pages, v.num_pages), float(sm_scale), _ptr(out), _ptr(workspace),
              workspace.numel(), _stream(stream)),
           "lynx_%s_attention" % ("verify" if full else "draft"))
    return out


def planes_view(p: Planes, first_page: int, num_pages: int) -> Planes:
    """Planes of pages first_page .. first_page + num_pages - 1 of a pool
    (views into the same memory; the layouts are page-major)."""
    if first_page < 0 or num_pages < 0 or first_page + num_pages > p.num_pages:
        raise ValueError("page range outside the pool")
    tile = _lib.lynx_plane_bytes(1, p.heads)
    a0, a1 = first_page * tile, (first_page + num_pages) * tile
    return Planes(p.anchor[a0:a1], None if p.residual is None else p.residual[a0:a1],
                  p.page_min[first_page:first_page + num_pages],
                  p.page_range[first_page:first_page + num_pages],
                  p.chunk_mean[first_page:first_page + num_pages],
                  p.chunk_maxabs[first_page:first_page + num_pages],
                  num_pages=num_pages, heads=p.heads, role=p.role)


def split_planes(p: Planes, anchor_bits: int, stream=None):
    """b + (8 - b) cut of encoded planes: (anchor stream, residual stream),
    uint8 tensors of b * 4096 and (8 - b) * 4096 bytes per (page, head)."""
    P, H = p.num_pages, p.heads
    na = _lib.lynx_split_stream_bytes(P, H, anchor_bits)
    nr = _lib.lynx_split_stream_bytes(P, H, 8 - anchor_bits)
    a = torch.empty(max(na, 16), dtype=torch.uint8, device=p.anchor.device)
    r = torch.empty(max(nr, 16), dtype=torch.uint8, device=p.anchor.device)
    cp = p.c()
    _check(_lib.lynx_split_planes(ctypes.byref(cp), P, H, HEAD_DIM, anchor_bits, _ptr(a), _ptr(r),
                                  _stream(stream)), "lynx_split_planes")
    return a[:na], r[:nr]


def dequantize_split(anchor: torch.Tensor, residual: Optional[torch.Tensor], anchor_bits: int,
                     scales: Planes, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """fp32 reconstruction [P][256][H][128] from b + (8 - b) streams; residual
    None is the draft.  `scales` supplies the page and chunk scales."""
    P, H = scales.num_pages, scales.heads
    if out is None:
        out = torch.empty((P, PAGE, H, HEAD_DIM), dtype=torch.float32, device=anchor.device)
    cp = scales.c()
    _check(_lib.lynx_dequantize_split(_ptr(anchor), _ptr(residual), anchor_bits, ctypes.byref(cp), P,
                                      H, HEAD_DIM, scales.role, _ptr(out), _stream(stream)),
           "lynx_dequantize_split")
    return out


def cut_planes(p: Planes, anchor_bits: int, stream=None) -> Planes:
    """The planes of p re-cut b + (8 - b): anchor and residual are the two
    streams, the scales are p's own tensors (shared, not copied)."""
    a, r = split_planes(p, anchor_bits, stream)
    return Planes(a, r, p.page_min, p.page_range, p.chunk_mean, p.chunk_maxabs,
                  num_pages=p.num_pages, heads=p.heads, role=p.role)


def decode_attention_split(q: torch.Tensor, k: Planes, v: Planes, anchor_bits: int, max_pages: int,
                           full: bool = True, block_table: Optional[torch.Tensor] = None,
                           seq_lens: Optional[torch.Tensor] = None,
                           sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           scores: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_attention over b + (8 - b) streams (k, v from cut_planes with
    the same anchor_bits); full=False is the draft of the b-bit anchor."""
    q = _bf16_bits(q)
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][Hq][128] bf16 tensor")
    B, Hq, D = q.shape
    H = k.heads
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, Hq, max_pages, q.device)
    kc, vc = k.c(), v.c()
    _check(_lib.lynx_decode_attention_split(
        _ptr(q), ctypes.byref(kc), ctypes.byref(vc), anchor_bits, int(bool(full)), _ptr(block_table),
        _ptr(seq_lens), B, H, Hq, D, max_pages, min(k.num_pages, v.num_pages), float(sm_scale),
        _ptr(out), _ptr(scores), _ptr(workspace), workspace.numel(), _stream(stream)),
        "lynx_decode_attention_split")
    return out


def alloc_cut_planes(num_pages: int, heads: int, role: int, anchor_bits: int,
                     device="cuda") -> Planes:
    """Planes whose anchor / residual hold b + (8 - b) streams."""
    na = _lib.lynx_split_stream_bytes(num_pages, heads, anchor_bits)
    nr = _lib.lynx_split_stream_bytes(num_pages, heads, 8 - anchor_bits)
    return Planes(torch.empty(max(na, 16), dtype=torch.uint8, device=device)[:na],
                  torch.empty(max(nr, 16), dtype=torch.uint8, device=device)[:nr],
                  torch.empty((num_pages, heads, HEAD_DIM), dtype=torch.float32, device=device),
                  torch.empty((num_pages, heads, HEAD_DIM), dtype=torch.float32, device=device),
                  torch.empty((num_pages, heads, CHUNKS, HEAD_DIM), dtype=torch.float32, device=device),
                  torch.empty((num_pages, heads, CHUNKS, HEAD_DIM), dtype=torch.float32, device=device),
                  num_pages=num_pages, heads=heads, role=role)


def quantize_pages_split(kv: torch.Tensor, role: int, anchor_bits: int, out: Optional[Planes] = None,
                         stream=None) -> Planes:
    """Encode bf16 pages [P][256][H][128] straight into a b + (8 - b) cut
    (the streams cut_planes(quantize_pages(kv, role), b) would give)."""
    kv = _bf16_bits(kv)
    if kv.dim() != 4 or kv.shape[1] != PAGE or not kv.is_contiguous():
        raise ValueError("kv must be a contiguous [P][256][H][128] bf16 tensor")
    P, _, H, D = kv.shape
    if out is None:
        out = alloc_cut_planes(P, H, role, anchor_bits, kv.device)
    cp = out.c()
    _check(_lib.lynx_quantize_pages_split(_ptr(kv), P, H, D, role, anchor_bits, ctypes.byref(cp),
                                          _stream(stream)), "lynx_quantize_pages_split")
    return out
