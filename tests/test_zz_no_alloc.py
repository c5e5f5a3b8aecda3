"""lynx_decode_attention_full_static (the call that allocates nothing: its
split partials live in the library's static scratch) against
lynx_decode_attention_full with a caller workspace: two calls in a row on
one GPU, the second over a smaller input, each bitwise equal to the
workspace call (the same kernels), which the other tests hold to the
oracle's bar."""
import dataclasses
import math

import numpy as np
import pytest

from long_context_serving_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SM = float(np.float32(1.0 / math.sqrt(128.0)))


@pytest.fixture(scope="module")
def lynx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx as mod
    return mod


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def planes(lynx, w):
    k = to_dev(synth.kv_pages(w, 0, 0, 0))
    v = to_dev(synth.kv_pages(w, 0, 1, 0))
    return lynx.quantize_kv_pages(k, v)


def both(lynx, q, pk, pv, max_pages, **kw):
    ref = lynx.decode_attention(q, pk, pv, max_pages, full=True, sm_scale=SM, **kw)
    got = torch.full_like(ref, float("nan"))
    lynx.decode_attention_full_static(q, pk, pv, max_pages, sm_scale=SM, out=got, **kw)
    torch.cuda.synchronize()
    return got, ref


def test_static_scratch_call_equals_the_workspace_call(lynx):
    # 1: one request of 64 pages x 8 KV heads, 64 query heads: 32 splits per
    # (request, head), so the partials fill the scratch
    w1 = dataclasses.replace(synth.WORKLOADS["ctx32k"], tokens=64 * 256)
    pk, pv = planes(lynx, w1)
    q = to_dev(synth.queries(w1, key_aligned=False))
    print("static scratch call 1: %d pages x %d heads, %d query heads" %
          (w1.pages, w1.kv_heads, w1.q_heads), flush=True)
    got, ref = both(lynx, q, pk, pv, w1.pages)
    assert torch.equal(got, ref)
    # 2: a smaller input right after, with a block table and ragged lengths:
    # 3 requests over a pool of 6 pages of 2 KV heads, 16 query heads
    w2 = dataclasses.replace(synth.WORKLOADS["tiny"], kv_heads=2, tokens=6 * 256, q_heads=16)
    pk2, pv2 = planes(lynx, w2)
    rng = np.random.default_rng(3)
    q2 = to_dev(synth.float_to_bf16_bits(rng.laplace(0, 1, (3, 16, 128)).astype(np.float32)))
    bt = torch.tensor([[5, 1, 3], [0, -1, 2], [4, 2, 1]], dtype=torch.int32, device="cuda")
    sl = torch.tensor([768, 512, 256], dtype=torch.int32, device="cuda")
    print("static scratch call 2: 3 requests, pool of 6 pages x 2 heads", flush=True)
    got2, ref2 = both(lynx, q2, pk2, pv2, 3, block_table=bt, seq_lens=sl)
    assert torch.equal(got2, ref2)
    # 3: group 16 (the other page kernel and its combine)
    w3 = dataclasses.replace(synth.WORKLOADS["tiny"], kv_heads=2, tokens=4 * 256, q_heads=32)
    pk3, pv3 = planes(lynx, w3)
    q3 = to_dev(synth.queries(w3, key_aligned=False))
    print("static scratch call 3: group 16", flush=True)
    got3, ref3 = both(lynx, q3, pk3, pv3, w3.pages)
    assert torch.equal(got3, ref3)


def test_static_scratch_call_refuses_a_shape_beyond_the_scratch(lynx):
    w = dataclasses.replace(synth.WORKLOADS["tiny"], kv_heads=1, q_heads=8, tokens=256)
    pk, pv = planes(lynx, w)
    big = 16384
    q = torch.zeros((big, 8, 128), dtype=torch.int16, device="cuda")
    out = torch.empty((big, 8, 128), dtype=torch.float32, device="cuda")
    bt = torch.zeros((big, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(lynx.LynxError):
        lynx.decode_attention_full_static(q, pk, pv, 1, block_table=bt, out=out)
