"""Quality harness checks (tests/quality_harness.py).

CPU: the harness's unablated quantizer agrees with the oracle, and the
orderings the study reports hold on a small synthetic case.
GPU: the library's kernels (encoder + fused decode attention) reproduce the
harness's attention-output NMSE of Lynx full and anchor-only.
"""
import math

import numpy as np
import pytest

import oracle
import quality_harness as qh

SM = 1.0 / math.sqrt(128.0)


@pytest.fixture(scope="module")
def case():
    w, cases = qh.synthetic_cases(tokens=2048, requests=2)
    return w, cases


def _oracle_reconstruction(x_f64, anchor_only):
    bits = (x_f64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    enc = oracle.encode(bits)
    a, r = oracle.split(enc["codes"])
    return oracle.dequant(a, None if anchor_only else r, enc)


def test_unablated_harness_quantizer_matches_the_oracle(case):
    _, cases = case
    xk, xv, q = cases[0]
    for anchor_only in (False, True):
        for x in (xk, xv):
            got, _ = qh.lynx_reconstruct(x, anchor_only=anchor_only)
            ref = _oracle_reconstruction(x, anchor_only)
            rg = x.max(axis=1, keepdims=True) - x.min(axis=1, keepdims=True)
            close = np.abs(got - ref) <= 1e-5 * np.broadcast_to(rg, x.shape) + 1e-12
            # the harness takes its statistics in float64, the oracle in the
            # named fp32 operations: a code may move by one level at a boundary
            assert close.mean() > 0.999, (anchor_only, close.mean())
        P, T, H, D = xk.shape
        flat = lambda a: a.reshape(P * T, H, D)
        ref_out = qh.attention(q, flat(xk), flat(xv), SM)
        e_h = qh.nmse(qh.attention(q, flat(qh.lynx_reconstruct(xk, anchor_only=anchor_only)[0]),
                                   flat(qh.lynx_reconstruct(xv, anchor_only=anchor_only)[0]), SM),
                      ref_out)
        e_o = qh.nmse(qh.attention(q, flat(_oracle_reconstruction(xk, anchor_only)),
                                   flat(_oracle_reconstruction(xv, anchor_only)), SM), ref_out)
        assert abs(e_h - e_o) <= 0.05 * e_o, (anchor_only, e_h, e_o)


def test_uniform_grid_matches_the_oracles_grid():
    rng = np.random.default_rng(3)
    x = rng.laplace(0, 1, (2, 256, 2, 128))
    got, bits = qh.uniform_reconstruct(x, 4, "token")
    rows = x.reshape(-1, 128).astype(np.float32)
    codes = oracle.uniform_codes(rows, 4)
    lo = rows.min(axis=1, keepdims=True).astype(np.float64)
    step = (rows.max(axis=1, keepdims=True).astype(np.float64) - lo) / 15
    np.testing.assert_allclose(got.reshape(-1, 128), lo + codes * step, rtol=0, atol=1e-6)
    assert bits == 4 + 32 / 128


def test_study_orderings_on_synthetic_kv(case):
    _, cases = case
    r = qh.study(cases, SM, chunks=(8, 32, 64), alphas=())
    n = {k: v["nmse"] for k, v in r.items()}
    print({k: "%.3g" % v for k, v in n.items()}, flush=True)
    # per-token uniform grids are crushed by the outlier channels
    assert n["lynx_full"] < n["uniform_int8_per_token"] / 10
    assert n["lynx_anchor"] < n["uniform_int4_per_token"] / 3
    # the +7 midpoint and the chunking both help the anchor-only draft
    assert n["anchor_no_midpoint"] > 1.3 * n["lynx_anchor"]
    assert n["anchor_no_chunking"] > 1.3 * n["lynx_anchor"]
    # smaller chunks help the draft
    assert n["anchor_chunk_8"] < n["anchor_chunk_64"]
    # sign awareness only changes the draft: the full code keeps every sign
    assert n["full_no_sign_aware"] == n["lynx_full"]
    # the scales cost 2.25 bits per coordinate (fp32, C = 32)
    assert r["lynx_full"]["bits"] == 10.25 and r["lynx_anchor"]["bits"] == 6.25


@pytest.mark.gpu
def test_gpu_kernels_reproduce_the_quality_metric(case):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx
    _, cases = case
    num = {True: 0.0, False: 0.0}
    num_o = {True: 0.0, False: 0.0}
    den = 0.0
    for xk, xv, q in cases:
        P, T, H, D = xk.shape
        flat = lambda a: a.reshape(P * T, H, D)
        ref = qh.attention(q, flat(xk), flat(xv), SM)
        den += float((ref ** 2).sum())
        to_dev = lambda x: torch.from_numpy(
            (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).cuda()
        pk = lynx.quantize_pages(to_dev(xk), lynx.ROLE_KEY)
        pv = lynx.quantize_pages(to_dev(xv), lynx.ROLE_VALUE)
        qd = to_dev(q[None])
        for full in (True, False):
            out = lynx.decode_attention(qd, pk, pv, P, full=full, sm_scale=float(np.float32(SM)))
            torch.cuda.synchronize()
            num[full] += float(((out.cpu().numpy()[0].astype(np.float64) - ref) ** 2).sum())
            o_or = qh.attention(q, flat(_oracle_reconstruction(xk, not full)),
                                flat(_oracle_reconstruction(xv, not full)), SM)
            num_o[full] += float(((o_or - ref) ** 2).sum())
    for full in (True, False):
        e_gpu, e_or = num[full] / den, num_o[full] / den
        print("full=%s: NMSE gpu %.4g oracle %.4g" % (full, e_gpu, e_or), flush=True)
        assert abs(e_gpu - e_or) <= 0.02 * e_or
