"""Progressive plane streaming: the anchor stream first, the residual after.

Page "Lynx: the KV cache does not have to arrive whole", section 4: the
anchor planes land first and drafting starts on them while the residual
planes keep arriving under strict priority (anchors always drained first);
once a layer's residual is in, attention runs on the full reconstruction.
Section 1 describes the layer-wise pipelining this is compared with.

One GPU, one request, L layers.  The encoded planes of every layer sit in
pinned host memory (as received from a prefill node).  A single copy stream
at default priority carries, in FIFO order, every layer's anchor plane and
scales (K and V) and then every layer's residual planes, so the anchors are
drained first.  The compute stream runs layer l's draft (anchor-only)
attention as soon as its anchors land and its full attention as soon as its
residuals land.  Events on both streams time the whole schedule.

The comparison schedules run on the same link: Lynx-INT8 layer-wise (each
layer's complete planes, then its full attention) and a bf16 copy of the raw
cache (its attention is not part of this library; only the copy is timed).

Everything here is orchestration of copies, events and calls into liblynx:
the arithmetic runs in the HIP kernels.
"""
import time
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import torch

from . import lynx

SCALE_FIELDS = ("page_min", "page_range", "chunk_mean", "chunk_maxabs")


def _planes_tensors(p: lynx.Planes, anchor: bool, residual: bool) -> List[torch.Tensor]:
    out = []
    if anchor:
        out += [p.anchor] + [getattr(p, f) for f in SCALE_FIELDS]
    if residual:
        out.append(p.residual)
    return out


def pinned_like(p: lynx.Planes) -> lynx.Planes:
    """Empty pinned host planes shaped like p."""
    mk = lambda t: torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    return lynx.Planes(mk(p.anchor), mk(p.residual), *(mk(getattr(p, f)) for f in SCALE_FIELDS),
                       num_pages=p.num_pages, heads=p.heads, role=p.role)


def device_like(p: lynx.Planes, device) -> lynx.Planes:
    mk = lambda t: torch.empty(t.shape, dtype=t.dtype, device=device)
    return lynx.Planes(mk(p.anchor), mk(p.residual), *(mk(getattr(p, f)) for f in SCALE_FIELDS),
                       num_pages=p.num_pages, heads=p.heads, role=p.role)


def copy_planes(dst: lynx.Planes, src: lynx.Planes, anchor: bool, residual: bool):
    for d, s in zip(_planes_tensors(dst, anchor, residual), _planes_tensors(src, anchor, residual)):
        d.copy_(s, non_blocking=True)


def planes_bytes(p: lynx.Planes, anchor: bool, residual: bool) -> int:
    return sum(t.numel() * t.element_size() for t in _planes_tensors(p, anchor, residual))


class PacedLink:
    """An emulated link of `gbps` gigabits per second from pinned host memory
    to the GPU (page "Lynx: the KV cache does not have to arrive whole",
    section 5: the benefit is measured at 10-50 Gbps between servers).

    Copies are cut into pieces; a piece is released to the copy stream only
    when the emulated link would have delivered its last byte (start time +
    cumulative bytes / rate), the host waiting for that moment.  The PCIe
    copy that follows is 5-40x faster than the emulated rates, so a piece
    lands shortly after its release time.
    """

    def __init__(self, gbps: float, copy_stream: torch.cuda.Stream, piece_bytes: int = 4 << 20):
        self.rate = gbps * 1e9 / 8.0
        self.piece = piece_bytes
        self.stream = copy_stream
        self.sent = 0
        self.t0 = 0.0

    def start(self, event: torch.cuda.Event):
        """Begin the link's clock; `event` is recorded on the copy stream at
        the same moment (the reference of every reported time)."""
        torch.cuda.synchronize()
        self.sent = 0
        event.record(self.stream)
        self.t0 = time.perf_counter()

    def send(self, dst: torch.Tensor, src: torch.Tensor):
        d, s = dst.view(-1), src.view(-1)
        es = s.element_size()
        step = max(1, self.piece // es)
        with torch.cuda.stream(self.stream):
            for a in range(0, s.numel(), step):
                b = min(s.numel(), a + step)
                self.sent += (b - a) * es
                release = self.t0 + self.sent / self.rate
                while time.perf_counter() < release:
                    pass
                d[a:b].copy_(s[a:b], non_blocking=True)


@dataclass
class Layer:
    """One layer of the arriving cache: pinned host planes of K and V and the
    layer's decode query (device, bf16 bits [1][Hq][128])."""
    host_k: lynx.Planes
    host_v: lynx.Planes
    q: torch.Tensor


class ProgressiveStream:
    """Device buffers, streams and events for streaming a list of layers."""

    def __init__(self, layers: Sequence[Layer], device="cuda", sm_scale: Optional[float] = None):
        self.layers = list(layers)
        self.device = torch.device(device)
        self.dev_k = [device_like(l.host_k, self.device) for l in self.layers]
        self.dev_v = [device_like(l.host_v, self.device) for l in self.layers]
        k0 = self.layers[0].host_k
        self.pages, self.heads = k0.num_pages, k0.heads
        self.q_heads = self.layers[0].q.shape[1]
        self.sm_scale = sm_scale
        self.ws = lynx.alloc_workspace(1, self.heads, self.q_heads, self.pages, self.device)
        shape = (1, self.q_heads, lynx.HEAD_DIM)
        self.out_draft = [torch.empty(shape, dtype=torch.float32, device=self.device) for _ in self.layers]
        self.out_full = [torch.empty(shape, dtype=torch.float32, device=self.device) for _ in self.layers]
        self.copy_stream = torch.cuda.Stream(self.device)      # default priority
        self.compute_stream = torch.cuda.Stream(self.device)   # default priority

    def anchor_bytes(self) -> int:
        return sum(planes_bytes(l.host_k, True, False) + planes_bytes(l.host_v, True, False)
                   for l in self.layers)

    def residual_bytes(self) -> int:
        return sum(planes_bytes(l.host_k, False, True) + planes_bytes(l.host_v, False, True)
                   for l in self.layers)

    def _attend(self, i: int, full: bool, scores: Optional[torch.Tensor] = None):
        k, v = self.dev_k[i], self.dev_v[i]
        if not full:
            k, v = k.without_residual(), v.without_residual()
        lynx.decode_attention(self.layers[i].q, k, v, self.pages, full=full,
                              sm_scale=self.sm_scale, out=self.out_full[i] if full else self.out_draft[i],
                              scores=scores, workspace=self.ws, stream=self.compute_stream)

    def run_progressive(self) -> Dict[str, float]:
        """Anchor-first streaming with drafts on arrival; returns times in ms
        from the start event (first copy issued)."""
        n = len(self.layers)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        start = ev()
        a_in, r_in = [ev() for _ in range(n)], [ev() for _ in range(n)]
        d_beg, d_end = [ev() for _ in range(n)], [ev() for _ in range(n)]
        f_beg, f_end = [ev() for _ in range(n)], [ev() for _ in range(n)]
        cur = torch.cuda.current_stream(self.device)
        torch.cuda.synchronize(self.device)
        start.record(cur)
        self.copy_stream.wait_event(start)
        self.compute_stream.wait_event(start)
        with torch.cuda.stream(self.copy_stream):
            for i, l in enumerate(self.layers):
                copy_planes(self.dev_k[i], l.host_k, True, False)
                copy_planes(self.dev_v[i], l.host_v, True, False)
                a_in[i].record(self.copy_stream)
            for i, l in enumerate(self.layers):
                copy_planes(self.dev_k[i], l.host_k, False, True)
                copy_planes(self.dev_v[i], l.host_v, False, True)
                r_in[i].record(self.copy_stream)
        with torch.cuda.stream(self.compute_stream):
            for i in range(n):
                self.compute_stream.wait_event(a_in[i])
                d_beg[i].record(self.compute_stream)
                self._attend(i, full=False)
                d_end[i].record(self.compute_stream)
            for i in range(n):
                self.compute_stream.wait_event(r_in[i])
                f_beg[i].record(self.compute_stream)
                self._attend(i, full=True)
                f_end[i].record(self.compute_stream)
        torch.cuda.synchronize(self.device)
        t = lambda e: start.elapsed_time(e)
        dur = lambda b, e: sum(b[i].elapsed_time(e[i]) for i in range(n))
        return {
            "anchors_landed_ms": t(a_in[-1]),
            "residuals_landed_ms": t(r_in[-1]),
            "first_draft_layer_ms": t(d_end[0]),
            "all_drafts_ms": t(d_end[-1]),
            "all_full_ms": t(f_end[-1]),
            "draft_attention_ms": dur(d_beg, d_end),
            "full_attention_ms": dur(f_beg, f_end),
            "after_last_copy_ms": t(f_end[-1]) - t(r_in[-1]),
        }

    def run_layerwise_int8(self) -> Dict[str, float]:
        """Lynx-INT8 layer-wise pipelining: layer l's complete planes, then
        its full attention (overlapping the next layer's copy)."""
        n = len(self.layers)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        start, landed, done = ev(), [ev() for _ in range(n)], [ev() for _ in range(n)]
        cur = torch.cuda.current_stream(self.device)
        torch.cuda.synchronize(self.device)
        start.record(cur)
        self.copy_stream.wait_event(start)
        self.compute_stream.wait_event(start)
        with torch.cuda.stream(self.copy_stream):
            for i, l in enumerate(self.layers):
                copy_planes(self.dev_k[i], l.host_k, True, True)
                copy_planes(self.dev_v[i], l.host_v, True, True)
                landed[i].record(self.copy_stream)
        with torch.cuda.stream(self.compute_stream):
            for i in range(n):
                self.compute_stream.wait_event(landed[i])
                self._attend(i, full=True)
                done[i].record(self.compute_stream)
        torch.cuda.synchronize(self.device)
        return {"first_layer_ms": start.elapsed_time(done[0]),
                "all_full_ms": start.elapsed_time(done[-1]),
                "all_landed_ms": start.elapsed_time(landed[-1])}

    # -- schedules on an emulated link -----------------------------------
    def paced_progressive(self, link: PacedLink) -> Dict[str, float]:
        """Anchor-first streaming over the emulated link; drafts run as each
        layer's anchors land, full attention as its residual lands."""
        n = len(self.layers)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        start, a_in, r_in = ev(), [ev() for _ in range(n)], [ev() for _ in range(n)]
        d_end, f_end = [ev() for _ in range(n)], [ev() for _ in range(n)]
        link.start(start)
        for phase, (anchor, residual, landed, done, full) in enumerate(
                ((True, False, a_in, d_end, False), (False, True, r_in, f_end, True))):
            for i, l in enumerate(self.layers):
                for d, h in ((self.dev_k[i], l.host_k), (self.dev_v[i], l.host_v)):
                    for dt, ht in zip(_planes_tensors(d, anchor, residual),
                                      _planes_tensors(h, anchor, residual)):
                        link.send(dt, ht)
                landed[i].record(self.copy_stream)
                self.compute_stream.wait_event(landed[i])
                self._attend(i, full=full)
                done[i].record(self.compute_stream)
        torch.cuda.synchronize(self.device)
        t = lambda e: start.elapsed_time(e)
        return {"first_draft_ms": t(d_end[0]), "all_drafts_ms": t(d_end[-1]),
                "anchors_landed_ms": t(a_in[-1]), "first_full_layer_ms": t(f_end[0]),
                "all_full_ms": t(f_end[-1]), "residuals_landed_ms": t(r_in[-1])}

    def paced_layerwise_int8(self, link: PacedLink) -> Dict[str, float]:
        """Lynx-INT8 layer-wise over the emulated link: each layer's complete
        planes, then its full attention."""
        n = len(self.layers)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        start, landed, done = ev(), [ev() for _ in range(n)], [ev() for _ in range(n)]
        link.start(start)
        for i, l in enumerate(self.layers):
            for d, h in ((self.dev_k[i], l.host_k), (self.dev_v[i], l.host_v)):
                for dt, ht in zip(_planes_tensors(d, True, True), _planes_tensors(h, True, True)):
                    link.send(dt, ht)
            landed[i].record(self.copy_stream)
            self.compute_stream.wait_event(landed[i])
            self._attend(i, full=True)
            done[i].record(self.compute_stream)
        torch.cuda.synchronize(self.device)
        return {"first_full_layer_ms": start.elapsed_time(done[0]),
                "all_full_ms": start.elapsed_time(done[-1])}

    def paced_bf16(self, link: PacedLink, host_layer: torch.Tensor,
                   dev_layer: torch.Tensor) -> Dict[str, float]:
        """The raw bf16 cache (K and V of one layer per step) over the
        emulated link; its attention is not part of this library."""
        n = len(self.layers)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        start, landed = ev(), [ev() for _ in range(n)]
        link.start(start)
        for i in range(n):
            link.send(dev_layer, host_layer)
            landed[i].record(self.copy_stream)
        torch.cuda.synchronize(self.device)
        return {"first_layer_landed_ms": start.elapsed_time(landed[0]),
                "all_landed_ms": start.elapsed_time(landed[-1])}

    def draft_full_topk_overlap(self, ks: Sequence[int] = (1, 16, 64)) -> Dict[int, float]:
        """Mean over layers and query heads of |top-k(draft) & top-k(full)| / k
        on the scaled logits (the planes must be resident)."""
        T = self.pages * lynx.PAGE
        sd = torch.empty((1, self.q_heads, T), dtype=torch.float32, device=self.device)
        sf = torch.empty_like(sd)
        acc = {k: 0.0 for k in ks}
        with torch.cuda.stream(self.compute_stream):
            for i in range(len(self.layers)):
                self._attend(i, full=False, scores=sd)
                self._attend(i, full=True, scores=sf)
                for k, v in topk_overlap(sd[0], sf[0], ks).items():
                    acc[k] += v
        torch.cuda.synchronize(self.device)
        return {k: acc[k] / len(self.layers) for k in ks}


def topk_overlap(a: torch.Tensor, b: torch.Tensor, ks: Sequence[int]) -> Dict[int, float]:
    """Mean over rows of |top-k(a_row) & top-k(b_row)| / k (rows = heads)."""
    out = {}
    for k in ks:
        ia = torch.topk(a, k, dim=-1).indices
        ib = torch.topk(b, k, dim=-1).indices
        hit = (ia.unsqueeze(-1) == ib.unsqueeze(-2)).any(-1).sum(-1).to(torch.float64)
        out[k] = float((hit / k).mean())
    return out


def build_layers(w, device="cuda", layers: Optional[int] = None, tokens: Optional[int] = None,
                 request: int = 0) -> List[Layer]:
    """Encode each layer's synthetic K and V on the device and keep the planes
    in pinned host memory (the cache as it arrives from prefill)."""
    from . import synth
    L = w.layers if layers is None else layers
    T = w.tokens if tokens is None else tokens
    out = []
    for layer in range(L):
        planes = []
        for tensor, role in ((0, lynx.ROLE_KEY), (1, lynx.ROLE_VALUE)):
            x = synth.device_kv_pages(w, layer, tensor, request, device=device, tokens=T)
            p = lynx.quantize_pages(x, role)
            h = pinned_like(p)
            for d, s in zip(_planes_tensors(h, True, True), _planes_tensors(p, True, True)):
                d.copy_(s)
            planes.append(h)
            del x, p
        q = torch.from_numpy(synth.queries(w, batch=1, first_request=request, layer=layer)
                             .view("int16")).to(device)
        out.append(Layer(planes[0], planes[1], q))
    torch.cuda.synchronize(device)
    return out
