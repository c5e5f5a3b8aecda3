"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar (element by element, same seeded inputs):
  codes       bit-exact, except +-1 on elements the oracle flags as lying
              within 2^-20 of a rounding boundary;
  scales      bit-exact (page min/range, chunk mean/max-abs);
  dequant     |gpu - oracle| <= 1e-3 |oracle|, or <= 1e-6 * page range where
              the reconstruction cancels to ~0;
  attention   |gpu - oracle| <= 2e-3 + 1e-5 |oracle| per element (oracle in
              fp64 over its own dequantized K and V), for key-aligned and for
              plain Laplace queries alike.  The 2e-3 is the stated bar
              against fp32; the 1e-5 relative part covers the fp32 value
              sums of outputs of several hundred.  A plain fp32 evaluation
              of the same attention misses this bar on plain Laplace queries
              (one-hot softmax over scores of a few hundred); the kernel's
              scores are exact integer products, so it does not.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from long_context_serving_amd import synth
from planes_layout import unpack_codes

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL_ATTN = 2e-3
RTOL_ATTN = 1e-5
RTOL_DQ = 1e-3
FLOOR_DQ = 1e-6
SM = float(np.float32(1.0 / math.sqrt(128.0)))


@pytest.fixture(scope="module")
def lynx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx as mod
    return mod


def to_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def gpu_codes(pl, P, H, role):
    a = pl.anchor.cpu().numpy()
    r = pl.residual.cpu().numpy()
    return unpack_codes(a, r, P, H, role)


def check_encode(lynx, x_bits, role, enc=None, pl=None):
    P, _, H, _ = x_bits.shape
    print("encode parity P=%d H=%d role=%d" % (P, H, role), flush=True)
    if enc is None:
        enc = oracle.encode(x_bits)
    if pl is None:
        pl = lynx.quantize_pages(to_dev(x_bits), role)
    torch.cuda.synchronize()
    a, r, code = gpu_codes(pl, P, H, role)
    ref = enc["codes"]
    assert not (enc["flags"] & oracle.FLAG_SUM_INEXACT).any(), "input breaks the exact-sum precondition"
    near = (enc["flags"] & oracle.FLAG_NEAR_HALF) != 0
    mism = code != ref
    n_mism, n_near = int(mism.sum()), int(near.sum())
    print("  codes: %d mismatches, %d elements flagged near a half-level" % (n_mism, n_near), flush=True)
    assert not (mism & ~near).any(), "unflagged code mismatches: %d" % int((mism & ~near).sum())
    assert (np.abs(code.astype(np.int16) - ref.astype(np.int16))[mism] <= 1).all()
    # The bar allows +-1 on flagged elements; the kernel's level thresholds
    # are the oracle's own rounding points (checked for every fp32 u on the
    # host and on the device), so none is used.
    assert n_mism == 0, "flagged code mismatches: %d" % n_mism
    for name in ("page_min", "page_range", "chunk_mean", "chunk_maxabs"):
        got = getattr(pl, name).cpu().numpy().reshape(enc[name].shape)
        assert np.array_equal(got.view(np.uint32), enc[name].view(np.uint32)), name
    return pl, enc, (a, r, code), n_mism


def check_dequant(lynx, pl, enc, gpu_code, full):
    a_ref, r_ref = oracle.split(enc["codes"])
    ref = oracle.dequant(a_ref, r_ref if full else None, enc)
    got = lynx.dequantize(pl, full=full).cpu().numpy().astype(np.float64)
    same = gpu_code == enc["codes"] if full else (gpu_code >> 4) == (enc["codes"] >> 4)
    rg = np.broadcast_to(enc["page_range"][:, None].astype(np.float64), ref.shape)
    err = np.abs(got - ref)
    ok = (err <= RTOL_DQ * np.abs(ref)) | (err <= FLOOR_DQ * rg)
    assert ok[same].all(), "dequant mismatch: max rel %g" % float((err / np.maximum(np.abs(ref), 1e-30))[same & ~ok].max())


def oracle_attention_for(enc_k, enc_v, q_bits, page_lists, full, want_logits=False):
    """Oracle attention for requests whose logical pages are page_lists[b] (pool indices)."""
    ak, rk = oracle.split(enc_k["codes"])
    av, rv = oracle.split(enc_v["codes"])
    kh = oracle.dequant(ak, rk if full else None, enc_k)
    vh = oracle.dequant(av, rv if full else None, enc_v)
    q = oracle.bf16_bits_to_float(q_bits).astype(np.float64)
    outs, logits = [], []
    for b, pages in enumerate(page_lists):
        H, D = kh.shape[2], kh.shape[3]
        kk = kh[pages].reshape(1, -1, H, D)
        vv = vh[pages].reshape(1, -1, H, D)
        res = oracle.attention(q[b:b + 1], kk, vv, SM, want_logits=want_logits)
        if want_logits:
            outs.append(res[0][0])
            logits.append(res[1][0])
        else:
            outs.append(res[0])
    return (np.stack(outs), logits) if want_logits else np.stack(outs)


def check_attention(got, ref, label, fp32_err=None):
    """The attention bar, on both query classes.  fp32_err, printed for
    comparison only: the max-abs error of a plain fp32 evaluation of the
    same attention (with plain Laplace queries the softmax is one-hot over
    scores of a few hundred, and fp32 alone misses the bar)."""
    err = np.abs(got - ref)
    bound = ATOL_ATTN + RTOL_ATTN * np.abs(ref)
    print("%s: max abs err %.3g (max |out| %.1f), max err/bound %.3f%s" %
          (label, err.max(), np.abs(ref).max(), (err / bound).max(),
           "" if fp32_err is None else ", plain fp32 evaluation %.3g" % fp32_err), flush=True)
    assert (err <= bound).all(), label


def fp32_attention(enc_k, enc_v, q_bits, full):
    """Plain fp32 evaluation (torch on the CPU) of one request's attention
    over the oracle's dequantized K and V: the precision the bar refers to."""
    ak, rk = oracle.split(enc_k["codes"])
    av, rv = oracle.split(enc_v["codes"])
    kh = oracle.dequant(ak, rk if full else None, enc_k)
    vh = oracle.dequant(av, rv if full else None, enc_v)
    H, D = kh.shape[2], kh.shape[3]
    k = torch.from_numpy(kh.reshape(-1, H, D).astype(np.float32)).permute(1, 2, 0).contiguous()
    v = torch.from_numpy(vh.reshape(-1, H, D).astype(np.float32)).permute(1, 0, 2).contiguous()
    q = torch.from_numpy(oracle.bf16_bits_to_float(q_bits).astype(np.float32)).reshape(H, -1, D)
    p = torch.softmax(torch.bmm(q, k) * SM, dim=-1)
    return torch.bmm(p, v).reshape(1, -1, D).numpy().astype(np.float64)


def run_gpu_attention(lynx, q_bits, pk, pv, max_pages, full, block_table=None, seq_lens=None,
                      scores=None):
    q = to_dev(q_bits)
    bt = None if block_table is None else torch.from_numpy(np.asarray(block_table, np.int32)).cuda()
    sl = None if seq_lens is None else torch.from_numpy(np.asarray(seq_lens, np.int32)).cuda()
    out = lynx.decode_attention(q, pk, pv, max_pages, full=full, block_table=bt, seq_lens=sl,
                                sm_scale=SM, scores=scores)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def encode_pair(lynx, w, layer=0, request=0, tokens=None):
    xk = synth.kv_pages(w, layer, 0, request, tokens=tokens)
    xv = synth.kv_pages(w, layer, 1, request, tokens=tokens)
    pk, ek, ck, _ = check_encode(lynx, xk, 0)
    pv, ev, cv, _ = check_encode(lynx, xv, 1)
    return pk, ek, ck, pv, ev, cv


# ---------------------------------------------------------------------------
# Tiny workload: 4 pages, 4 KV heads, 32 query heads
# ---------------------------------------------------------------------------
def test_tiny_encode_dequant_attention(lynx):
    w = synth.WORKLOADS["tiny"]
    pk, ek, ck, pv, ev, cv = encode_pair(lynx, w)
    for full in (False, True):
        check_dequant(lynx, pk, ek, ck[2], full)
        check_dequant(lynx, pv, ev, cv[2], full)
    for aligned in (True, False):
        q = synth.queries(w, key_aligned=aligned)
        for full in (False, True):
            ref = oracle_attention_for(ek, ev, q, [list(range(w.pages))], full)
            got = run_gpu_attention(lynx, q, pk, pv, w.pages, full)
            e32 = None if aligned else float(np.abs(fp32_attention(ek, ev, q, full) - ref).max())
            check_attention(got, ref, "tiny full=%s aligned=%s" % (full, aligned), e32)


def test_anchor_calls_never_need_the_residual(lynx):
    w = synth.WORKLOADS["tiny"]
    pk, ek, ck, pv, ev, cv = encode_pair(lynx, w)
    q = synth.queries(w)
    with_res = run_gpu_attention(lynx, q, pk, pv, w.pages, False)
    without = run_gpu_attention(lynx, q, pk.without_residual(), pv.without_residual(), w.pages, False)
    assert np.array_equal(with_res, without)
    d1 = lynx.dequantize(pk.without_residual(), full=False).cpu().numpy()
    d2 = lynx.dequantize(pk, full=False).cpu().numpy()
    assert np.array_equal(d1, d2)
    with pytest.raises(lynx.LynxError):
        lynx.dequantize(pk.without_residual(), full=True)


# ---------------------------------------------------------------------------
# 32K context (the benchmark workload), full size
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def ctx32k(lynx):
    return encode_pair(lynx, synth.WORKLOADS["ctx32k"])


def test_ctx32k_full_size(lynx, ctx32k):
    w = synth.WORKLOADS["ctx32k"]
    pk, ek, ck, pv, ev, cv = ctx32k
    check_dequant(lynx, pk, ek, ck[2], True)
    check_dequant(lynx, pv, ev, cv[2], False)
    q = synth.queries(w)
    T = w.tokens
    for full in (False, True):
        scores = torch.empty((1, w.q_heads, T), dtype=torch.float32, device="cuda")
        ref, logits = oracle_attention_for(ek, ev, q, [list(range(w.pages))], full, want_logits=True)
        got = run_gpu_attention(lynx, q, pk, pv, w.pages, full, scores=scores)
        check_attention(got, ref, "ctx32k full=%s" % full)
        sc = scores.cpu().numpy()[0].astype(np.float64)
        lg = logits[0]
        assert np.abs(sc - lg).max() <= 1e-4 * max(1.0, np.abs(lg).max())
        # top-1 token per head agrees unless the oracle's top-2 gap is tiny
        srt = np.sort(lg, axis=1)
        clear = (srt[:, -1] - srt[:, -2]) > 1e-3
        assert np.array_equal(sc.argmax(1)[clear], lg.argmax(1)[clear])


def test_ctx32k_plain_laplace_queries(lynx, ctx32k):
    w = synth.WORKLOADS["ctx32k"]
    pk, ek, ck, pv, ev, cv = ctx32k
    q = synth.queries(w, key_aligned=False)
    for full in (False, True):
        ref = oracle_attention_for(ek, ev, q, [list(range(w.pages))], full)
        got = run_gpu_attention(lynx, q, pk, pv, w.pages, full)
        e32 = float(np.abs(fp32_attention(ek, ev, q, full) - ref).max())
        check_attention(got, ref, "ctx32k plain queries full=%s" % full, e32)


# ---------------------------------------------------------------------------
# Batched decode: 64 requests x 16K; the GPU runs the full batch, the oracle
# checks sampled requests (the others are copies, which must agree bitwise)
# ---------------------------------------------------------------------------
def test_batched_64x16k_sampled(lynx):
    w = synth.WORKLOADS["batched64x16k"]
    sampled = [0, 1]
    P = w.pages
    xk = [synth.kv_pages(w, 0, 0, r) for r in sampled]
    xv = [synth.kv_pages(w, 0, 1, r) for r in sampled]
    ek = [oracle.encode(x) for x in xk]
    ev = [oracle.encode(x) for x in xv]
    # pool: request b uses the pages of sampled request b % 2, laid out in a
    # permuted order through the block table
    pool_k = np.concatenate([xk[b % 2] for b in range(w.batch)])
    pool_v = np.concatenate([xv[b % 2] for b in range(w.batch)])
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.batch * P)              # logical page -> pool slot
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    pk = lynx.quantize_pages(to_dev(pool_k[inv]), 0)
    pv = lynx.quantize_pages(to_dev(pool_v[inv]), 1)
    block_table = perm.reshape(w.batch, P).astype(np.int32)
    for aligned in (True, False):
        q_all = synth.queries(w, key_aligned=aligned)
        q = np.stack([q_all[b % 2] if b >= 2 else q_all[b] for b in range(w.batch)])
        for full in (False, True):
            got = run_gpu_attention(lynx, q, pk, pv, P, full, block_table=block_table)
            for i, r in enumerate(sampled):
                ref = oracle_attention_for(ek[i], ev[i], q[r:r + 1], [list(range(P))], full)
                e32 = None if aligned else float(
                    np.abs(fp32_attention(ek[i], ev[i], q[r:r + 1], full) - ref).max())
                check_attention(got[r], ref[0], "batched request %d full=%s aligned=%s" %
                                (r, full, aligned), e32)
            for b in range(2, w.batch):
                assert np.array_equal(got[b], got[b % 2])


# The benchmark's launch configuration: 64 distinct requests drawn on the
# device into contiguous K and V pools (no block table), encoded by one
# launch, one decode launch per variant over the whole batch; the first,
# a middle and the last request checked against the oracle.
def test_batched_64x16k_bench_configuration_sampled(lynx):
    w = synth.WORKLOADS["batched64x16k"]
    P = w.pages
    shape = (w.batch * P, 256, w.kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.int16, device="cuda")
    v = torch.empty(shape, dtype=torch.int16, device="cuda")
    for r in range(w.batch):
        k[r * P:(r + 1) * P] = synth.device_kv_pages(w, 0, 0, r)
        v[r * P:(r + 1) * P] = synth.device_kv_pages(w, 0, 1, r)
    pk, pv = lynx.quantize_kv_pages(k, v)
    torch.cuda.synchronize()
    sampled = (0, w.batch // 2 - 1, w.batch - 1)
    encs = {}
    for r in sampled:
        sl = slice(r * P, (r + 1) * P)
        print("batched request %d: encode parity" % r, flush=True)
        _, ek, _, _ = check_encode(lynx, k[sl].cpu().numpy().view(np.uint16), 0,
                                   pl=lynx.planes_view(pk, r * P, P))
        _, ev, _, _ = check_encode(lynx, v[sl].cpu().numpy().view(np.uint16), 1,
                                   pl=lynx.planes_view(pv, r * P, P))
        encs[r] = (ek, ev)
    del k, v
    for aligned in (True, False):
        q = synth.queries(w, key_aligned=aligned)
        for full in (False, True):
            got = run_gpu_attention(lynx, q, pk, pv, P, full)
            for r in sampled:
                ek, ev = encs[r]
                ref = oracle_attention_for(ek, ev, q[r:r + 1], [list(range(P))], full)
                check_attention(got[r], ref[0], "batched (bench layout) request %d full=%s aligned=%s"
                                % (r, full, aligned))
    del pk, pv
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Qwen3-235B-A22B shape: encode of one layer (512 pages x 4 heads), K and V
# ---------------------------------------------------------------------------
def test_qwen3_235b_layer_encode(lynx):
    w = synth.WORKLOADS["qwen3_235b_128k"]
    for tensor, role in ((0, 0), (1, 1)):
        x = synth.kv_pages(w, 47, tensor, 0)
        check_encode(lynx, x, role)


# The same shape at full size in the benchmark's launch configuration: the
# 94 layers' pages in one K and one V pool drawn on the device (12.6 GB
# each), encoded by one launch; pages of the first, middle and last layers
# (and a few drawn at random) checked against the oracle one by one.
def test_qwen3_235b_all_layers_one_launch_sampled_pages(lynx):
    w = synth.WORKLOADS["qwen3_235b_128k"]
    P = w.pages
    shape = (w.layers * P, 256, w.kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.int16, device="cuda")
    v = torch.empty(shape, dtype=torch.int16, device="cuda")
    for layer in range(w.layers):
        k[layer * P:(layer + 1) * P] = synth.device_kv_pages(w, layer, 0, 0)
        v[layer * P:(layer + 1) * P] = synth.device_kv_pages(w, layer, 1, 0)
    print("qwen3 pools drawn: %d pages" % (w.layers * P), flush=True)
    pk, pv = lynx.quantize_kv_pages(k, v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    picks = [(0, 0), (0, P - 1), (w.layers // 2, P // 2), (w.layers - 1, 0), (w.layers - 1, P - 1)]
    picks += [(int(a), int(b)) for a, b in zip(rng.integers(0, w.layers, 3), rng.integers(0, P, 3))]
    for layer, page in picks:
        g = layer * P + page
        for x_dev, pl, role in ((k, pk, 0), (v, pv, 1)):
            print("qwen3 layer %d page %d role %d" % (layer, page, role), flush=True)
            x = x_dev[g:g + 1].cpu().numpy().view(np.uint16)
            check_encode(lynx, x, role, pl=lynx.planes_view(pl, g, 1))
    del k, v, pk, pv
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Progressive-arrival shape: one layer of 64K context, both variants
# ---------------------------------------------------------------------------
def test_progressive_layer_attention(lynx):
    w = synth.WORKLOADS["progressive32x64k"]
    pk, ek, ck, pv, ev, cv = encode_pair(lynx, w, layer=5)
    for aligned in (True, False):
        q = synth.queries(w, layer=5, key_aligned=aligned)
        for full in (False, True):
            ref = oracle_attention_for(ek, ev, q, [list(range(w.pages))], full)
            got = run_gpu_attention(lynx, q, pk, pv, w.pages, full)
            e32 = None if aligned else float(np.abs(fp32_attention(ek, ev, q, full) - ref).max())
            check_attention(got, ref, "progressive layer 5 full=%s aligned=%s" % (full, aligned), e32)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
def test_degenerate_channels_and_chunks(lynx):
    x = synth.laplace_pages(3, 2, 128, seed=91, scale_channels=((0, 5, 100.0), (1, 77, 100.0)))
    xf = oracle.bf16_bits_to_float(x).copy()
    xf[:, :, 0, 3] = 1.5                         # constant channel (range 0)
    xf[1, 64:96, 1, 9] = xf[1, 70, 1, 9]         # constant chunk (max-abs 0)
    xf[2, :, 1, 10] = np.arange(256) * 0.25      # exact ramp
    xf[0, :, 0, 11] = np.float32(2.0 ** -20) * np.sign(xf[0, :, 0, 11])  # two-valued channel
    x = synth.float_to_bf16_bits(xf)
    for role in (0, 1):
        pl, enc, codes, _ = check_encode(lynx, x, role)
        check_dequant(lynx, pl, enc, codes[2], True)
        check_dequant(lynx, pl, enc, codes[2], False)


def test_chunks_outside_the_exact_sum_precondition(lynx):
    """A nonzero normalised value below 2^-24 next to a large page range:
    the kernel's double-precision chunk sum may round there (the header's
    contract), so its mean is within one ulp of the oracle's exactly rounded
    one, codes within +-1 and the max-abs within the ulp that moves; every
    other chunk and every page statistic stays bit-exact."""
    rng = np.random.default_rng(3)
    xf = np.zeros((2, 256, 2, 128), np.float32)
    xf[:] = rng.laplace(0, 1, xf.shape).astype(np.float32)
    for d in range(0, 128, 3):
        base = np.float32(-(2.0 ** -(20 + d % 9)))
        xf[0, :, 1, d] = base * (1 + rng.integers(0, 128, 256) / np.float32(128.0))
        xf[0, 200, 1, d] = np.float32(96.0 * (d + 1))
    x = synth.float_to_bf16_bits(xf)
    enc = oracle.encode(x)
    flagged_chunk = ((enc["flags"] & oracle.FLAG_SUM_INEXACT) != 0).reshape(2, 8, 32, 2, 128).any(axis=2)
    assert flagged_chunk.any()
    fc = np.transpose(flagged_chunk, (0, 2, 1, 3))                   # [P][H][8][D]
    for role in (0, 1):
        pl = lynx.quantize_pages(to_dev(x), role)
        torch.cuda.synchronize()
        _, _, code = gpu_codes(pl, 2, 2, role)
        for name in ("page_min", "page_range"):
            got = getattr(pl, name).cpu().numpy().reshape(enc[name].shape)
            assert np.array_equal(got.view(np.uint32), enc[name].view(np.uint32)), name
        mu = pl.chunk_mean.cpu().numpy().reshape(enc["chunk_mean"].shape)
        sd = pl.chunk_maxabs.cpu().numpy().reshape(enc["chunk_maxabs"].shape)
        assert np.array_equal(mu[~fc].view(np.uint32), enc["chunk_mean"][~fc].view(np.uint32))
        assert np.array_equal(sd[~fc].view(np.uint32), enc["chunk_maxabs"][~fc].view(np.uint32))
        ulp_mu = np.spacing(np.abs(enc["chunk_mean"][fc]))
        assert np.all(np.abs(mu[fc] - enc["chunk_mean"][fc]) <= ulp_mu)
        ulp_s = np.spacing(np.abs(enc["chunk_maxabs"][fc]))
        assert np.all(np.abs(sd[fc] - enc["chunk_maxabs"][fc]) <= ulp_mu + 2 * ulp_s)
        el = np.repeat(flagged_chunk, 32, axis=1).reshape(2, 256, 2, 128)
        ref = enc["codes"]
        assert np.array_equal(code[~el], ref[~el])
        assert np.all(np.abs(code[el].astype(np.int16) - ref[el].astype(np.int16)) <= 1)
        print("role %d: %d flagged chunks, %d chunk means differ by one ulp, %d codes by one" %
              (role, int(fc.sum()), int((mu[fc] != enc["chunk_mean"][fc]).sum()),
               int((code[el] != ref[el]).sum())), flush=True)


def test_empty_inputs(lynx):
    x = np.zeros((0, 256, 2, 128), np.uint16)
    pl = lynx.alloc_planes(1, 2, 0)
    out = lynx.quantize_pages(to_dev(x), 0, out=pl)
    torch.cuda.synchronize()
    assert out is pl
    q = to_dev(np.zeros((0, 16, 128), np.uint16))
    o = lynx.decode_attention(q, pl, pl, 1, full=True)
    assert o.shape == (0, 16, 128)
    # requests over an empty pool: every block-table entry is skipped, the
    # context is empty and the output is zero (group 8: matrix-core kernel;
    # group 16: the other kernel)
    empty = dataclasses.replace(pl, num_pages=0)  # valid pointers, pool of 0 pages
    for Hq in (16, 32):
        q = to_dev(synth.float_to_bf16_bits(np.ones((3, Hq, 128), np.float32)))
        bt = torch.full((3, 2), -1, dtype=torch.int32, device="cuda")
        for full in (False, True):
            o = lynx.decode_attention(q, empty, empty, 2, full=full, block_table=bt,
                                      out=torch.full((3, Hq, 128), 7.0, device="cuda"))
            torch.cuda.synchronize()
            assert torch.count_nonzero(o).item() == 0, (Hq, full)


def test_ragged_lengths_group_sizes_and_skipped_pages(lynx):
    rng = np.random.default_rng(13)
    for H, Hq in ((2, 32), (4, 4), (1, 8)):
        P_pool = 9
        x_k = synth.laplace_pages(P_pool, H, 128, seed=H * 100 + 1, scale_channels=((0, 2, 80.0),))
        x_v = synth.laplace_pages(P_pool, H, 128, seed=H * 100 + 2, scale_channels=((H - 1, 100, 90.0),))
        pk, ek, _, _ = check_encode(lynx, x_k, 0)
        pv, ev, _, _ = check_encode(lynx, x_v, 1)
        max_pages = 4
        lengths = [1, 4, 3]
        bt = np.full((3, max_pages), -1, np.int32)
        pages = []
        for b, n in enumerate(lengths):
            pg = rng.choice(P_pool, size=n, replace=False)
            bt[b, :n] = pg
            pages.append(list(pg))
        # an out-of-range entry inside a request's length is skipped
        bt[1, 2] = P_pool + 7
        pages[1] = [p for i, p in enumerate(pages[1]) if i != 2]
        q = synth.float_to_bf16_bits(rng.laplace(0, 1, (3, Hq, 128)).astype(np.float32))
        for full in (False, True):
            ref = oracle_attention_for(ek, ev, q, pages, full)
            got = run_gpu_attention(lynx, q, pk, pv, max_pages, full, block_table=bt,
                                    seq_lens=[256 * n for n in lengths])
            check_attention(got, ref, "ragged H=%d Hq=%d full=%s" % (H, Hq, full))


@pytest.mark.parametrize("H,Hq", [(2, 16), (1, 16)])
def test_keys_with_offset_and_shifted_chunks(lynx, H, Hq):
    """Key channel (head 0, channel 7) on a DC offset of 300, so the page
    minimum dwarfs the range, and channel (H - 1, 20) raised by 40 in every
    other 32-token chunk, so the chunk means dwarf the chunk deviations:
    encode parity (both roles), both dequantizers, and decode attention
    within the bar for the matrix-core kernel (group 8) and the other one
    (group 16)."""
    rng = np.random.default_rng(29)
    P_pool = 6
    x = synth.laplace_pages(P_pool, H, 128, seed=H * 10 + 3, scale_channels=((0, 3, 90.0),))
    xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
    xf[:, :, 0, 7] += 300.0
    t = np.arange(xf.shape[1])
    xf[:, ((t // 32) % 2) == 1, H - 1, 20] += 40.0
    x_k = synth.float_to_bf16_bits(xf)
    x_v = synth.laplace_pages(P_pool, H, 128, seed=H * 10 + 4, scale_channels=((0, 9, 60.0),))
    pk, ek, kcodes, _ = check_encode(lynx, x_k, 0)
    pv, ev, _, _ = check_encode(lynx, x_v, 1)
    for full in (True, False):
        check_dequant(lynx, pk, ek, kcodes[2], full)
    # the same keys under the value role, dequantized
    pkv, ekv, kvcodes, _ = check_encode(lynx, x_k, 1)
    for full in (True, False):
        check_dequant(lynx, pkv, ekv, kvcodes[2], full)
    pages = [[4, 0, 2], [5, 1, 3]]
    bt = np.array(pages, np.int32)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (2, Hq, 128)).astype(np.float32))
    for full in (False, True):
        ref = oracle_attention_for(ek, ev, q, pages, full)
        got = run_gpu_attention(lynx, q, pk, pv, 3, full, block_table=bt)
        check_attention(got, ref, "offset keys H=%d Hq=%d full=%s" % (H, Hq, full))


@pytest.mark.parametrize("Hq", [8, 4])
def test_most_splits_per_head(lynx, Hq):
    """One request and one KV head over 256 pages: one page per block, so the
    split combine merges 256 parts per head (the most attention_shape makes),
    past the parts a combine thread preloads, for GQA groups 8 and 4."""
    H, P = 1, 256
    x_k = synth.laplace_pages(P, H, 128, seed=81, scale_channels=((0, 3, 90.0),))
    x_v = synth.laplace_pages(P, H, 128, seed=82, scale_channels=((0, 77, 50.0),))
    pk, ek, _, _ = check_encode(lynx, x_k, 0)
    pv, ev, _, _ = check_encode(lynx, x_v, 1)
    rng = np.random.default_rng(83)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (1, Hq, 128)).astype(np.float32))
    for full in (False, True):
        print("most splits Hq=%d full=%s" % (Hq, full), flush=True)
        ref = oracle_attention_for(ek, ev, q, [list(range(P))], full)
        got = run_gpu_attention(lynx, q, pk, pv, P, full)
        check_attention(got, ref, "256 splits Hq=%d full=%s" % (Hq, full))


def test_uneven_runs_across_the_pairs_of_a_block(lynx):
    """Runs of 3 pages per block, so each of a block's 8 K/V wave pairs takes
    3 chunks; the last block of request 1 (2 pages left by its length) gives
    pairs 0-4 three chunks, pair 5 one and pairs 6-7 none, and the block's
    step count follows pair 0.  Request 0 is 150 pages long, request 1 149
    (no block table: each owns 150 contiguous pool pages)."""
    H, Hq, max_pages = 2, 16, 150
    x_k = synth.laplace_pages(2 * max_pages, H, 128, seed=71, scale_channels=((1, 5, 70.0),))
    x_v = synth.laplace_pages(2 * max_pages, H, 128, seed=72, scale_channels=((0, 9, 60.0),))
    pk, ek, _, _ = check_encode(lynx, x_k, 0)
    pv, ev, _, _ = check_encode(lynx, x_v, 1)
    lengths = [150, 149]
    pages = [list(range(0, 150)), list(range(150, 150 + 149))]
    rng = np.random.default_rng(73)
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (2, Hq, 128)).astype(np.float32))
    for full in (False, True):
        print("uneven runs full=%s" % full, flush=True)
        ref, logits = oracle_attention_for(ek, ev, q, pages, full, want_logits=True)
        scores = torch.empty((2, Hq, 256 * max_pages), dtype=torch.float32, device="cuda")
        got = run_gpu_attention(lynx, q, pk, pv, max_pages, full,
                                seq_lens=[256 * n for n in lengths], scores=scores)
        check_attention(got, ref, "uneven pair runs full=%s" % full)
        sc = scores.cpu().numpy().astype(np.float64)
        for b, n in enumerate(lengths):
            lg = logits[b]
            assert np.abs(sc[b, :, :256 * n] - lg).max() <= 1e-4 * max(1.0, np.abs(lg).max())


@pytest.mark.parametrize("H,Hq,B", [(8, 64, 16), (16, 32, 8)])
def test_merge_of_many_rows_one_block_per_row_and_head(lynx, H, Hq, B):
    """B requests x H KV heads = 128 (row, KV head) pairs of up to 4 pages,
    so each run splits in two and the split merge takes one block per pair
    (GQA groups 8 and 2: threads past the group idle); ragged lengths leave
    some requests one part (no block table: request b owns pool pages
    4b .. 4b + 3)."""
    max_pages = 4
    x_k = synth.laplace_pages(B * max_pages, H, 128, seed=81, scale_channels=((2, 7, 50.0),))
    x_v = synth.laplace_pages(B * max_pages, H, 128, seed=82, scale_channels=((1, 3, 40.0),))
    pk, ek, _, _ = check_encode(lynx, x_k, 0)
    pv, ev, _, _ = check_encode(lynx, x_v, 1)
    rng = np.random.default_rng(83)
    lengths = [int(n) for n in rng.integers(1, max_pages + 1, B)]
    lengths[0] = max_pages
    pages = [list(range(b * max_pages, b * max_pages + n)) for b, n in enumerate(lengths)]
    q = synth.float_to_bf16_bits(rng.laplace(0, 1, (B, Hq, 128)).astype(np.float32))
    for full in (False, True):
        print("many-row merge H=%d Hq=%d full=%s lengths=%s" % (H, Hq, full, lengths), flush=True)
        ref = oracle_attention_for(ek, ev, q, pages, full)
        got = run_gpu_attention(lynx, q, pk, pv, max_pages, full, seq_lens=[256 * n for n in lengths])
        check_attention(got, ref, "many-row merge H=%d Hq=%d full=%s" % (H, Hq, full))


@pytest.mark.parametrize("P,H", [(1, 1), (3, 5), (128, 8)])
def test_kv_encode_in_one_launch_equals_one_launch_per_tensor(lynx, P, H):
    # lynx_quantize_kv_pages: every byte of both tensors' planes as written by
    # lynx_quantize_pages per tensor; the small shapes also against the oracle
    w = dataclasses.replace(synth.WORKLOADS["ctx32k"], kv_heads=H, tokens=P * 256)
    xk, xv = synth.kv_pages(w, 0, 0, 0), synth.kv_pages(w, 0, 1, 0)
    print("kv encode P=%d H=%d" % (P, H), flush=True)
    k, v = to_dev(xk), to_dev(xv)
    pk1 = lynx.quantize_pages(k, lynx.ROLE_KEY)
    pv1 = lynx.quantize_pages(v, lynx.ROLE_VALUE)
    pk2, pv2 = lynx.quantize_kv_pages(k, v)
    torch.cuda.synchronize()
    for one, two in ((pk1, pk2), (pv1, pv2)):
        for name in ("anchor", "residual", "page_min", "page_range", "chunk_mean", "chunk_maxabs"):
            assert torch.equal(getattr(one, name), getattr(two, name)), name
    if P * H <= 16:
        check_encode(lynx, xk, lynx.ROLE_KEY, pl=pk2)
        check_encode(lynx, xv, lynx.ROLE_VALUE, pl=pv2)


def test_repeat_runs_are_bitwise_identical(lynx):
    w = synth.WORKLOADS["tiny"]
    x = synth.kv_pages(w, 0, 0, 0)
    t = to_dev(x)
    p1 = lynx.quantize_pages(t, 1)
    p2 = lynx.quantize_pages(t, 1)
    torch.cuda.synchronize()
    assert torch.equal(p1.anchor, p2.anchor) and torch.equal(p1.residual, p2.residual)
    q = to_dev(synth.queries(w))
    o1 = lynx.decode_attention(q, lynx.quantize_pages(t, 0), p1, w.pages)
    o2 = lynx.decode_attention(q, lynx.quantize_pages(t, 0), p2, w.pages)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("one_launch", [False, True])
def test_graph_replays_match_eager(lynx, one_launch):
    """The calls of one step captured in a HIP graph (K and V encoded by one
    launch or one launch each): every replay, with other eager work on the
    device in between, is bitwise the eager result."""
    w = synth.WORKLOADS["tiny"]
    xk, xv = to_dev(synth.kv_pages(w, 0, 0, 0)), to_dev(synth.kv_pages(w, 0, 1, 0))
    other = to_dev(synth.kv_pages(w, 0, 0, 3))
    q = to_dev(synth.queries(w))
    pk = lynx.alloc_planes(w.pages, w.kv_heads, 0)
    pv = lynx.alloc_planes(w.pages, w.kv_heads, 1)
    po = lynx.alloc_planes(w.pages, w.kv_heads, 0)
    ws = lynx.alloc_workspace(1, w.kv_heads, w.q_heads, w.pages)
    oa = torch.empty((1, w.q_heads, 128), dtype=torch.float32, device="cuda")
    of = torch.empty_like(oa)

    def step():
        if one_launch:
            lynx.quantize_kv_pages(xk, xv, out_k=pk, out_v=pv)
        else:
            lynx.quantize_pages(xk, 0, out=pk)
            lynx.quantize_pages(xv, 1, out=pv)
        lynx.decode_attention(q, pk, pv, w.pages, full=False, sm_scale=SM, out=oa, workspace=ws)
        lynx.decode_attention(q, pk, pv, w.pages, full=True, sm_scale=SM, out=of, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pk.anchor, pk.residual, pv.anchor, pv.residual, pk.chunk_maxabs, oa, of)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (pk.anchor, pv.residual, oa, of, ws):
            t.zero_()
        lynx.quantize_pages(other, 0, out=po)
        g.replay()
        torch.cuda.synchronize()
        got = (pk.anchor, pk.residual, pv.anchor, pv.residual, pk.chunk_maxabs, oa, of)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d differs" % rep


def test_code_map_fast_path_is_exact_for_every_fp32_in_unit_interval(lynx):
    """Exhaustive: all 1,065,353,217 fp32 values u in [0, 1], and every u in
    (1, 2), which rounding can produce and which must take level 127."""
    assert lynx.selftest_code_map(0, 0x3F800001) == 0
    assert lynx.selftest_code_map(0x3F800001, 0x40000000) == 0
