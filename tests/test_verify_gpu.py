"""Parity of the verify and draft attention over pages plus a bf16 tail (through
the C ABI) with the oracle, and of quantize-on-append.

Bar: |gpu - oracle| <= 2e-3 + 1e-5 |oracle| per element (the same bar as
the single-query decode attention); pages written by quantize-on-append are
byte-identical to the same tokens encoded directly.
"""
import math

import numpy as np
import pytest

import oracle
from long_context_serving_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3
RTOL_ATTN = 1e-5
SM = float(np.float32(1.0 / math.sqrt(128.0)))
TAIL = 320


@pytest.fixture(scope="module")
def lynx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx as mod
    return mod


def to_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def check(got, ref, label):
    err = np.abs(got - ref)
    bound = ATOL_ATTN + RTOL_ATTN * np.abs(ref)
    print("%s: max abs err %.3g (max |out| %.1f), max err/bound %.3f" %
          (label, err.max(), np.abs(ref).max(), (err / bound).max()), flush=True)
    assert (err <= bound).all(), label


def pool_and_oracle(lynx, P, H, seed, k_shift=None):
    """Encoded K and V pools on the GPU and the oracle's dequantized pages
    (full and draft) of the same inputs; the GPU codes must equal the oracle's
    outside the flagged near-boundary elements, which are checked elsewhere --
    here the oracle dequantizes its own codes and the GPU reads its own."""
    xk = synth.laplace_pages(P, H, 128, seed=seed, scale_channels=((0, 3, 90.0),))
    if k_shift is not None:  # applied to the float values, then rounded to bf16 again
        xk = synth.float_to_bf16_bits(k_shift((xk.astype(np.uint32) << 16).view(np.float32)))
    xv = synth.laplace_pages(P, H, 128, seed=seed + 1, scale_channels=((H - 1, 77, 60.0),))
    pk = lynx.quantize_pages(to_dev(xk), lynx.ROLE_KEY)
    pv = lynx.quantize_pages(to_dev(xv), lynx.ROLE_VALUE)
    deq = {}
    for name, x in (("k", xk), ("v", xv)):
        enc = oracle.encode(x)
        a, r = oracle.split(enc["codes"])
        deq[name, True] = oracle.dequant(a, r, enc)
        deq[name, False] = oracle.dequant(a, None, enc)
    return pk, pv, deq


def tails(B, H, seed):
    x = synth.laplace_pages(2 * B, H, 128, seed=seed, scale_channels=((0, 5, 40.0),))
    return x.reshape(B, 2 * 256, H, 128)[:, :TAIL].copy()


def run_case(lynx, H, Hq, tq, page_lists, tail_len, P_pool, seed, full, max_pages=4,
             contiguous=False, k_shift=None):
    """contiguous: no block table; request b reads pool pages
    b * max_pages .. b * max_pages + len(page_lists[b]) - 1."""
    B = len(page_lists)
    if contiguous:
        assert all(pl == list(range(b * max_pages, b * max_pages + len(pl)))
                   for b, pl in enumerate(page_lists))
    pk, pv, deq = (pool_and_oracle(lynx, P_pool, H, seed, k_shift) if P_pool
                   else (None, None, None))
    if P_pool == 0:
        pk = lynx.alloc_planes(1, H, lynx.ROLE_KEY)
        pv = lynx.alloc_planes(1, H, lynx.ROLE_VALUE)
        import dataclasses
        pk, pv = dataclasses.replace(pk, num_pages=0), dataclasses.replace(pv, num_pages=0)
    tk, tv = tails(B, H, seed + 7), tails(B, H, seed + 9)
    rng = np.random.default_rng(seed)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (B, tq, Hq, 128)).astype(np.float32))
    bt = np.full((B, max_pages), -1, np.int32)
    for b, pl in enumerate(page_lists):
        bt[b, :len(pl)] = pl
    page_tokens = np.array([256 * len(pl) for pl in page_lists], np.int32)
    print("verify case H=%d Hq=%d tq=%d pages=%s tail=%s full=%s" %
          (H, Hq, tq, page_lists, tail_len, full), flush=True)
    got = lynx.verify_attention(to_dev(q), pk, pv, max_pages, to_dev(tk), to_dev(tv),
                                torch.tensor(tail_len, dtype=torch.int32, device="cuda"), full=full,
                                block_table=None if contiguous else torch.from_numpy(bt).cuda(),
                                page_tokens=torch.from_numpy(page_tokens).cuda(), sm_scale=SM)
    torch.cuda.synchronize()
    # a block-table entry outside the pool is skipped by the kernels
    present = [[p for p in pl if 0 <= p < P_pool] for pl in page_lists]
    pages_k = [np.concatenate([deq["k", full][p] for p in pl]).astype(np.float64) if pl else
               np.zeros((0, H, 128)) for pl in present]
    pages_v = [np.concatenate([deq["v", full][p] for p in pl]).astype(np.float64) if pl else
               np.zeros((0, H, 128)) for pl in present]
    ref = oracle.verify_attention(q, pages_k, pages_v, tk, tv, tail_len, SM)
    check(got.cpu().numpy().astype(np.float64), ref,
          "H=%d Hq=%d tq=%d full=%s" % (H, Hq, tq, full))


@pytest.mark.parametrize("full", [True, False])
def test_verify_group8_ragged_pages_and_tails(lynx, full):
    # matrix-core page kernel (group 8); a request with no full page
    # tq 5 and 16: one column group per wave (16 rows per block); 17, 37 and
    # 64: two (32 rows per block), 17 leaving row 16 alone in wave 4 and 37
    # the second block one row in wave 1
    for tq, tail_len in ((1, [1, 200, 320]), (5, [5, 64, 319]), (16, [16, 17, 272]),
                         (17, [17, 260, 300]), (37, [37, 100, 320]), (64, [64, 300, 320])):
        run_case(lynx, 2, 16, tq, [[4, 1, 6], [], [0, 2, 5, 3]], tail_len, 7, 101 + tq, full)


@pytest.mark.parametrize("full", [True, False])
def test_verify_group8_absent_pages_and_a_partial_row_group(lynx, full):
    # 20 tokens: one block of 32 rows with 20 of them (waves 5-7 without a
    # row, wave 4 with 4); entries 9 and -4 lie outside the pool of 7 pages
    # and are skipped
    run_case(lynx, 2, 16, 20, [[4, 9, 1], [2, -4, 6, 0]], [20, 150], 7, 211, full)


def test_verify_merge_of_many_parts_per_row(lynx):
    # one request of 32 pages in a reversed block table, 2 KV heads, 64
    # speculative tokens: 128 (row, KV head) pairs whose runs split into 32
    # parts plus the tail's, so the per-row merge reads 16 parts ahead of
    # the weights, 16 in groups of four and the last one alone
    pages = list(range(31, -1, -1))
    run_case(lynx, 2, 16, 64, [pages], [90], 32, 808, True, max_pages=32)


def _offset_keys(x):
    """Key channel (head 0, channel 7) on a DC offset of 300 (the page
    minimum then dwarfs the range) and channel (1, 20) raised by 40 in every
    other 32-token chunk (the chunk means then dwarf the chunk deviations)."""
    x = x.copy()
    x[:, :, 0, 7] += 300.0
    t = np.arange(x.shape[1])
    x[:, ((t // 32) % 2) == 1, 1, 20] += 40.0
    return x


@pytest.mark.parametrize("full", [True, False])
def test_verify_keys_with_offset_and_shifted_chunks(lynx, full):
    # the page minimum enters the scores through the fp64 page bias, the
    # chunk offset rg * mu through the fp32 key operand: both stay inside
    # the bar for one column group per wave (tq 5) and two (tq 64)
    for tq, tail_len in ((5, [5, 200]), (64, [64, 320])):
        run_case(lynx, 2, 16, tq, [[3, 0, 5], [1, 4, 2, 6]], tail_len, 7, 303 + tq, full,
                 k_shift=_offset_keys)


@pytest.mark.parametrize("full", [True, False])
def test_verify_group16_valu_path(lynx, full):
    run_case(lynx, 2, 32, 7, [[3, 5], [1], [6, 0, 2]], [7, 100, 256], 7, 303, full)


@pytest.mark.parametrize("Hq", [16, 32])
def test_verify_without_block_table(lynx, Hq):
    # no block table: request b owns pool pages b * max_pages ..; several
    # query tokens per request, so every row must read its request's pages
    # (group 8: matrix-core page kernel; group 16: the other kernel)
    run_case(lynx, 2, Hq, 6, [[0, 1], [3], [6, 7, 8]], [6, 40, 100], 9, 606, True, max_pages=3,
             contiguous=True)


@pytest.mark.parametrize("H,Hq", [(4, 8), (2, 10)])
def test_verify_small_groups_tails_across_slabs(lynx, H, Hq):
    # groups of 2 and 5 query heads (a wave with one head, waves with none);
    # tails that end just before, on and just after 64-token slab edges
    run_case(lynx, H, Hq, 3, [[2], [], [0, 1], [3]], [63, 64, 65, 131], 4, 404 + Hq, True)


def test_verify_pool_of_zero_pages(lynx):
    # the tail is the whole context
    run_case(lynx, 1, 8, 3, [[], []], [3, 250], 0, 505, True)


def test_verify_at_ctx32k_shape(lynx):
    # one request, 128 pages of 8 KV heads, 64 speculative tokens of 64 query heads
    run_case(lynx, 8, 64, 64, [list(range(128))], [100], 128, 707, True, max_pages=128)


def test_append_commit_writes_the_pages_directly_encoded(lynx):
    from long_context_serving_amd.tail import TailCache
    H = 2
    cache = TailCache(requests=2, heads=H, pool_pages=4, max_pages=3)
    x = synth.laplace_pages(2, H, 128, seed=909, scale_channels=((1, 9, 70.0),))  # 512 tokens
    y = synth.laplace_pages(2, H, 128, seed=910)
    xk, xv = x.reshape(512, H, 128), y.reshape(512, H, 128)
    # request 1: 100 + 150 + 50 rows, then a commit: one page, 44 tokens left
    for a, b in ((0, 100), (100, 250), (250, 300)):
        cache.append(1, to_dev(xk[a:b]), to_dev(xv[a:b]))
    assert cache.tail_tokens(1) == 300
    assert cache.commit(1) == 1
    assert cache.tail_tokens(1) == 44 and cache.pages(1) == [0]
    direct_k = lynx.quantize_pages(to_dev(xk[:256][None]), lynx.ROLE_KEY)
    direct_v = lynx.quantize_pages(to_dev(xv[:256][None]), lynx.ROLE_VALUE)
    page_k = lynx.planes_view(cache.k_pool, 0, 1)
    page_v = lynx.planes_view(cache.v_pool, 0, 1)
    for got, want in ((page_k, direct_k), (page_v, direct_v)):
        for f in ("anchor", "residual", "page_min", "page_range", "chunk_mean", "chunk_maxabs"):
            assert torch.equal(getattr(got, f), getattr(want, f)), f
    assert np.array_equal(cache.tail_k[1, :44].cpu().numpy().view(np.uint16), xk[256:300])
    # a speculative round: 8 tokens appended, scored, 5 rejected
    cache.append(1, to_dev(xk[300:308]), to_dev(xv[300:308]))
    rng = np.random.default_rng(11)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (2, 8, 16, 128)).astype(np.float32))
    cache.append(0, to_dev(xk[:8]), to_dev(xv[:8]))  # request 0: tail only
    out = cache.attention(to_dev(q), full=True, sm_scale=SM)
    torch.cuda.synchronize()
    enc_k, enc_v = oracle.encode(xk[:256][None]), oracle.encode(xv[:256][None])
    ak, rk = oracle.split(enc_k["codes"])
    av, rv = oracle.split(enc_v["codes"])
    pk = oracle.dequant(ak, rk, enc_k).reshape(256, H, 128)
    pv = oracle.dequant(av, rv, enc_v).reshape(256, H, 128)
    tail_bits_k = np.stack([xk[:TAIL], np.concatenate([xk[256:308], np.zeros((TAIL - 52, H, 128), np.uint16)])])
    tail_bits_v = np.stack([xv[:TAIL], np.concatenate([xv[256:308], np.zeros((TAIL - 52, H, 128), np.uint16)])])
    ref = oracle.verify_attention(q, [np.zeros((0, H, 128)), pk], [np.zeros((0, H, 128)), pv],
                                  tail_bits_k, tail_bits_v, [8, 52], SM)
    check(out.cpu().numpy().astype(np.float64), ref, "append + verify")
    cache.truncate(1, 5)
    assert cache.tail_tokens(1) == 47
    assert int(cache.tail_len[1].item()) == 47


def test_commit_on_a_side_stream(lynx):
    """Rows appended on the current stream, pages committed on a side
    stream, attention on the current stream: the commit orders itself after
    the appends and the attention after the commit."""
    from long_context_serving_amd.tail import TailCache
    H = 2
    cache = TailCache(requests=1, heads=H, pool_pages=3, max_pages=3)
    x = synth.laplace_pages(2, H, 128, seed=919, scale_channels=((0, 4, 50.0),))
    y = synth.laplace_pages(2, H, 128, seed=920)
    xk, xv = x.reshape(512, H, 128), y.reshape(512, H, 128)
    side = torch.cuda.Stream()
    cache.append(0, to_dev(xk[:300]), to_dev(xv[:300]))
    assert cache.commit(0, stream=side) == 1
    cache.append(0, to_dev(xk[300:306]), to_dev(xv[300:306]))
    rng = np.random.default_rng(12)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (1, 6, 16, 128)).astype(np.float32))
    out = cache.attention(to_dev(q), full=True, sm_scale=SM)
    torch.cuda.synchronize()
    enc_k, enc_v = oracle.encode(xk[:256][None]), oracle.encode(xv[:256][None])
    ak, rk = oracle.split(enc_k["codes"])
    av, rv = oracle.split(enc_v["codes"])
    pk = oracle.dequant(ak, rk, enc_k).reshape(256, H, 128)
    pv = oracle.dequant(av, rv, enc_v).reshape(256, H, 128)
    tk = np.concatenate([xk[256:306], np.zeros((TAIL - 50, H, 128), np.uint16)])[None]
    tv = np.concatenate([xv[256:306], np.zeros((TAIL - 50, H, 128), np.uint16)])[None]
    ref = oracle.verify_attention(q, [pk], [pv], tk, tv, [50], SM)
    check(out.cpu().numpy().astype(np.float64), ref, "commit on a side stream")
