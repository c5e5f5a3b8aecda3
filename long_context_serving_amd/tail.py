"""Growing an encoded cache token by token: a bf16 tail per request,
quantized one whole page at a time.

Page "Lynx: the KV cache does not have to arrive whole", section 3: the
quantizer works on pages of 256 tokens, so the newest tokens of a request
stay in bf16 until their page is full; section 4: a draft proposes tokens on
the anchor stream and the refined cache verifies them, after which the
rejected ones are dropped.  This module keeps, per request, the tail of
tokens after its last full page and the pool pages it owns:

  * ``append`` adds token rows (the decoded token, or a block of speculative
    tokens before their verify pass) to the tail;
  * ``truncate`` drops rejected speculative tokens from the end of the tail;
  * ``commit`` encodes every full page at the front of the tail into the next
    free pool page (the encoder of liblynx, writing through a view of the
    pool) and extends the request's block table.

Everything here is bookkeeping, copies and calls into liblynx.
"""
import contextlib
from typing import List, Optional

import torch

from . import lynx


class TailCache:
    """Page pools (K and V), per-request block tables and bf16 tails."""

    def __init__(self, requests: int, heads: int, pool_pages: int, max_pages: int, device="cuda"):
        self.requests, self.heads, self.max_pages = requests, heads, max_pages
        self.device = torch.device(device)
        self.k_pool = lynx.alloc_planes(pool_pages, heads, lynx.ROLE_KEY, self.device)
        self.v_pool = lynx.alloc_planes(pool_pages, heads, lynx.ROLE_VALUE, self.device)
        self.tail_k = lynx.alloc_tail(requests, heads, self.device)
        self.tail_v = lynx.alloc_tail(requests, heads, self.device)
        self.tail_len = torch.zeros(requests, dtype=torch.int32, device=self.device)
        self.page_tokens = torch.zeros(requests, dtype=torch.int32, device=self.device)
        self.block_table = torch.full((requests, max_pages), -1, dtype=torch.int32, device=self.device)
        self._tail: List[int] = [0] * requests
        self._pages: List[List[int]] = [[] for _ in range(requests)]
        self._free: List[int] = list(range(pool_pages))

    # -- host view -----------------------------------------------------------
    def tail_tokens(self, r: int) -> int:
        return self._tail[r]

    def pages(self, r: int) -> List[int]:
        return list(self._pages[r])

    def _publish(self, r: int):
        self.tail_len[r] = self._tail[r]
        self.page_tokens[r] = lynx.PAGE * len(self._pages[r])

    # -- growth --------------------------------------------------------------
    def append(self, r: int, k_rows: torch.Tensor, v_rows: torch.Tensor):
        """Append token rows (bf16 [n][H][128], on the device) to request r's tail."""
        n = k_rows.shape[0]
        if tuple(k_rows.shape) != (n, self.heads, lynx.HEAD_DIM) or v_rows.shape != k_rows.shape:
            raise ValueError("rows must be [n][H][128]")
        t0 = self._tail[r]
        if t0 + n > lynx.TAIL_TOKENS:
            raise ValueError("tail overflow: commit full pages first")
        self.tail_k[r, t0:t0 + n].copy_(lynx._bf16_bits(k_rows).view(torch.int16))
        self.tail_v[r, t0:t0 + n].copy_(lynx._bf16_bits(v_rows).view(torch.int16))
        self._tail[r] = t0 + n
        self._publish(r)

    def truncate(self, r: int, n: int):
        """Drop the last n tokens of request r's tail (rejected speculation)."""
        if n < 0 or n > self._tail[r]:
            raise ValueError("cannot drop %d of %d tail tokens" % (n, self._tail[r]))
        self._tail[r] -= n
        self._publish(r)

    def commit(self, r: int, stream: Optional[torch.cuda.Stream] = None) -> int:
        """Encode the full pages at the front of request r's tail; returns
        the number of pages written."""
        written = 0
        cur = torch.cuda.current_stream()
        side = stream is not None and stream != cur
        if side and self._tail[r] >= lynx.PAGE:
            # the tail rows were written by append() on the current stream
            stream.wait_stream(cur)
        while self._tail[r] >= lynx.PAGE:
            if not self._free:
                raise RuntimeError("page pool exhausted")
            if len(self._pages[r]) >= self.max_pages:
                raise RuntimeError("request %d has max_pages pages" % r)
            p = self._free.pop(0)
            # K and V of the page in one launch, then both tails shift down
            lynx.quantize_kv_pages(self.tail_k[r, :lynx.PAGE].unsqueeze(0),
                                   self.tail_v[r, :lynx.PAGE].unsqueeze(0),
                                   out_k=lynx.planes_view(self.k_pool, p, 1),
                                   out_v=lynx.planes_view(self.v_pool, p, 1), stream=stream)
            rest = self._tail[r] - lynx.PAGE
            # the shift and the block-table entry go on the encoder's stream,
            # so the shift cannot overwrite tokens before the encoder reads them
            with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
                if rest:
                    for tail in (self.tail_k, self.tail_v):
                        tail[r, :rest].copy_(tail[r, lynx.PAGE:lynx.PAGE + rest].clone())
                self.block_table[r, len(self._pages[r])] = p
            self._tail[r] -= lynx.PAGE
            self._pages[r].append(p)
            written += 1
        if side and written:
            # tail lengths, page counts and every later attention call run on
            # the current stream: they follow the shift and the table write
            cur.wait_stream(stream)
        self._publish(r)
        return written

    # -- attention -----------------------------------------------------------
    def attention(self, q: torch.Tensor, full: bool = True, sm_scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
        """Attention of every request's q.shape[1] newest tokens (the last
        tail tokens) over its pages and tail; full=False is the draft."""
        return lynx.verify_attention(q, self.k_pool, self.v_pool, self.max_pages, self.tail_k,
                                     self.tail_v, self.tail_len, full=full,
                                     block_table=self.block_table, page_tokens=self.page_tokens,
                                     sm_scale=sm_scale, out=out, workspace=workspace, stream=stream)
