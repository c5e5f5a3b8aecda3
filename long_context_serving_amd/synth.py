"""Seeded synthetic KV-cache and query generators.

These are the only inputs shared by the HIP path and the CPU oracle.  The
module holds no arithmetic of the quantization method: it draws numbers and
rounds them to bf16, nothing else.

The workloads stand in for the real KV caches the Lynx paper measures on
("Lynx: the KV cache does not have to arrive whole", sections 1-2: a small
subset of channels up to 100x larger than the rest, consistent in magnitude
within a channel; per-channel values otherwise Laplacian-like) and for its
context lengths (16K-128K, and the Qwen3-235B-A22B shape of section 1).
No dataset is used.

Recipe, per (config, layer, tensor K=0/V=1, request):
  z ~ Laplace(0, 1) i.i.d. over [T][H][D];
  per KV head, round(frac * D) outlier channels chosen without replacement,
  each with one multiplier for all tokens (fixed or uniform in a range);
  optional per-channel offsets N(0, sigma) on every channel;
  x = mult * z + offset, rounded to bf16 (round to nearest even).
Outlier channels and offsets are drawn per (layer, tensor) and shared by
every request of that layer, like a property of the model.

Queries (the pages fix no query statistics; this is a reading): Laplace(0, 1)
per channel, divided by the square root of the multiplier of the key channel
it meets (same layer, the KV head its query head reads), rounded to bf16.  A
100x key channel then outweighs an ordinary one tenfold in q.k, so outlier
channels dominate the scores, while the scaled logits keep a standard
deviation of about 3 and a top token holding tens of per cent of the softmax,
as in trained models.  Plain Laplace(0, 1) queries (key_aligned=False) make
the logits spread by ~20 and the softmax one-hot at 32K tokens: a stress case
in which no fp32 evaluation holds outputs to 1e-3.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

PAGE = 256


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    kv_heads: int
    head_dim: int
    tokens: int            # tokens per request (a multiple of 256)
    batch: int             # requests
    q_heads: int           # 0 = encode-only workload
    outlier_frac: float    # fraction of channels per head that are outliers
    outlier_count: Optional[int] = None  # exact count per head (overrides frac)
    mult_lo: float = 100.0
    mult_hi: float = 100.0  # == mult_lo: fixed multiplier
    offset_sigma: float = 0.0
    seed: int = 0
    cfg_id: int = 0
    notes: str = field(default="", compare=False)

    @property
    def pages(self) -> int:
        return self.tokens // PAGE

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads if self.q_heads else 0

    def n_outliers(self) -> int:
        if self.outlier_count is not None:
            return self.outlier_count
        return int(round(self.outlier_frac * self.head_dim))

    def elements(self) -> int:
        """K+V elements over all layers and requests."""
        return 2 * self.layers * self.batch * self.tokens * self.kv_heads * self.head_dim


WORKLOADS = {
    "tiny": Workload("tiny", layers=1, kv_heads=4, head_dim=128, tokens=1024, batch=1,
                     q_heads=32, outlier_frac=4 / 128, outlier_count=4, cfg_id=1,
                     notes="4 pages, 4 of 128 channels x100, GQA group 8"),
    "ctx32k": Workload("ctx32k", layers=1, kv_heads=8, head_dim=128, tokens=32768, batch=1,
                       q_heads=64, outlier_frac=0.02, mult_lo=30.0, mult_hi=100.0,
                       offset_sigma=0.5, cfg_id=2,
                       notes="2% channels x U(30,100), per-channel offsets N(0,0.5)"),
    "qwen3_235b_128k": Workload("qwen3_235b_128k", layers=94, kv_heads=4, head_dim=128,
                                tokens=131072, batch=1, q_heads=0, outlier_frac=0.03,
                                cfg_id=3, notes="encode only, 3% channels x100"),
    "batched64x16k": Workload("batched64x16k", layers=1, kv_heads=8, head_dim=128,
                              tokens=16384, batch=64, q_heads=64, outlier_frac=0.02,
                              cfg_id=4, notes="64 requests, 2% channels x100"),
    "progressive32x64k": Workload("progressive32x64k", layers=32, kv_heads=8, head_dim=128,
                                  tokens=65536, batch=1, q_heads=64, outlier_frac=0.02,
                                  cfg_id=5, notes="32 layers, 2% channels x100"),
}


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _channel_plan(w: Workload, layer: int, tensor: int):
    """Per-(layer, tensor) outlier multipliers and offsets, shape [H][D]."""
    rng = np.random.default_rng([w.seed, w.cfg_id, layer, tensor, 0xC4A7])
    mult = np.ones((w.kv_heads, w.head_dim), np.float64)
    n = w.n_outliers()
    for h in range(w.kv_heads):
        if n:
            ch = rng.choice(w.head_dim, size=n, replace=False)
            if w.mult_hi > w.mult_lo:
                mult[h, ch] = rng.uniform(w.mult_lo, w.mult_hi, size=n)
            else:
                mult[h, ch] = w.mult_lo
    off = np.zeros((w.kv_heads, w.head_dim), np.float64)
    if w.offset_sigma > 0:
        off = rng.normal(0.0, w.offset_sigma, size=(w.kv_heads, w.head_dim))
    return mult, off


def outlier_mask(w: Workload, layer: int = 0, tensor: int = 0) -> np.ndarray:
    """Boolean [H][D]: which channels carry an outlier multiplier."""
    mult, _ = _channel_plan(w, layer, tensor)
    return mult != 1.0


def kv_pages(w: Workload, layer: int, tensor: int, request: int,
             tokens: Optional[int] = None) -> np.ndarray:
    """bf16 bit patterns of one K (tensor=0) or V (tensor=1) cache of one
    request, paged: uint16 [tokens/256][256][H][D]."""
    T = w.tokens if tokens is None else tokens
    if T % PAGE:
        raise ValueError("tokens must be a multiple of 256")
    mult, off = _channel_plan(w, layer, tensor)
    rng = np.random.default_rng([w.seed, w.cfg_id, layer, tensor, request + 1])
    z = rng.laplace(0.0, 1.0, size=(T, w.kv_heads, w.head_dim))
    x = (z * mult[None] + off[None]).astype(np.float32)
    return float_to_bf16_bits(x).reshape(T // PAGE, PAGE, w.kv_heads, w.head_dim)


def device_kv_pages(w: Workload, layer: int, tensor: int, request: int, device="cuda",
                    tokens: Optional[int] = None):
    """kv_pages' recipe drawn on the device with torch's generator, for caches
    of many GB (the progressive-streaming harness).  Same distribution, same
    outlier channels and offsets, but not the same values as kv_pages:
    Laplace(0, 1) by inverse CDF from u uniform in (0, 1),
    z = -sign(u - 1/2) ln(1 - 2|u - 1/2|).  Returns bf16 bit patterns as int16
    [tokens/256][256][H][D] on the device."""
    import torch
    T = w.tokens if tokens is None else tokens
    if T % PAGE:
        raise ValueError("tokens must be a multiple of 256")
    mult, off = _channel_plan(w, layer, tensor)
    seed = int(np.random.SeedSequence([w.seed, w.cfg_id, layer, tensor, request + 1, 0xD7]).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    u = torch.rand((T, w.kv_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)
    c = u * (1.0 - 2.0 ** -24) + 2.0 ** -25 - 0.5          # u in (0, 1): |c| < 1/2
    z = -torch.sign(c) * torch.log1p(-2.0 * c.abs())
    x = z * torch.as_tensor(mult, dtype=torch.float32, device=device) + \
        torch.as_tensor(off, dtype=torch.float32, device=device)
    return x.to(torch.bfloat16).view(torch.int16).reshape(T // PAGE, PAGE, w.kv_heads, w.head_dim)


def queries(w: Workload, batch: Optional[int] = None, first_request: int = 0,
            layer: int = 0, key_aligned: bool = True) -> np.ndarray:
    """bf16 bit patterns of the decode queries of one layer: uint16 [B][Hq][D]."""
    B = w.batch if batch is None else batch
    div = np.ones((w.q_heads, w.head_dim), np.float64)
    if key_aligned:
        mult, _ = _channel_plan(w, layer, 0)
        div = np.sqrt(np.repeat(mult, w.group, axis=0))
    out = np.empty((B, w.q_heads, w.head_dim), np.uint16)
    for i in range(B):
        rng = np.random.default_rng([w.seed, w.cfg_id, 0x9E37, first_request + i])
        z = rng.laplace(0.0, 1.0, size=(w.q_heads, w.head_dim))
        out[i] = float_to_bf16_bits((z / div).astype(np.float32))
    return out


def laplace_pages(pages: int, heads: int, dim: int, seed: int,
                  scale_channels: Tuple[Tuple[int, int, float], ...] = ()) -> np.ndarray:
    """Small ad-hoc paged bf16 input for tests: Laplace(0,1) with optional
    (head, channel, multiplier) overrides.  uint16 [pages][256][heads][dim]."""
    rng = np.random.default_rng([seed, 0x51D])
    z = rng.laplace(0.0, 1.0, size=(pages * PAGE, heads, dim))
    for h, d, m in scale_channels:
        z[:, h, d] *= m
    return float_to_bf16_bits(z.astype(np.float32)).reshape(pages, PAGE, heads, dim)
