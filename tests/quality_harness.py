"""Quality harness (test infrastructure): normalised MSE of the attention
output for Lynx, its stage ablations and uniform INT8/INT4, on seeded
synthetic KV.

Page "Lynx: the KV cache does not have to arrive whole", section 5 reports
the normalised mean squared error of the attention output (the full
reconstruction about 25x below uniform INT8, the 4-bit variant about 35x
below uniform INT4, on LLaMA 8B keys and values); section 7 notes that the
quantizer's stages were only ever evaluated as a bundle and that the chunk
size was never swept.  This module measures both on the synthetic
Laplacian-plus-outlier caches that stand in for the pages' workloads.

The quantizer below restates section 3 in numpy (float64 statistics) with
switches that turn one stage off at a time; it is used for the study only.
Its unablated configuration is checked against the oracle and the GPU
kernels in tests/test_quality.py.  Readings:
  * NMSE = sum over query heads of |o_hat - o|^2 / sum of |o|^2, with o the
    float64 attention over the bf16 cache and o_hat the same attention over
    the reconstruction;
  * the 4-bit Lynx variant is the anchor plane alone (the draft);
  * uniform INT-B: an asymmetric grid of 2^B levels between the minimum and
    the maximum, per token (over the 128 channels of one head) or per
    channel (over the 256 tokens of one page);
  * bits per coordinate include the scales: Lynx stores 2 fp32 per channel
    per page and 2 per channel per chunk, the uniform grids 2 fp16 per group;
  * alpha (the curvature of the map, not given by the pages) is also swept.
"""
from typing import Dict

import numpy as np

ALPHA = 255.0
PAGE = 256


def _map(u, alpha=ALPHA):
    return np.log1p(alpha * u) / np.log1p(alpha)


def _inv(v, alpha=ALPHA):
    return ((1.0 + alpha) ** v - 1.0) / alpha


def lynx_reconstruct(x: np.ndarray, chunk: int = 32, page_norm: bool = True, log_map: bool = True,
                     sign_aware: bool = True, midpoint: bool = True, anchor_only: bool = False,
                     alpha: float = ALPHA, anchor_bits: int = 4):
    """Reconstruction of x (float64 [P][256][H][D]) by the quantizer of
    section 3 with the given stages; returns (x_hat, bits per coordinate).
    anchor_bits splits the 8-bit code into that many high bits (the anchor)
    and 8 - anchor_bits low bits (the residual); the draft keeps the anchor
    and the round-half-down centre of the residual range."""
    P, T, H, D = x.shape
    if P > 1:  # pages are independent; page-sized temporaries stay in cache
        out = np.empty_like(x)
        for i in range(P):
            out[i:i + 1], bits = lynx_reconstruct(x[i:i + 1], chunk, page_norm, log_map, sign_aware,
                                                  midpoint, anchor_only, alpha, anchor_bits)
        return out, bits
    if page_norm:
        mn = x.min(axis=1, keepdims=True)
        rg = x.max(axis=1, keepdims=True) - mn
        xn = np.where(rg > 0, (x - mn) / np.where(rg > 0, rg, 1.0), 0.0)
    else:
        xn = x
    xc = xn.reshape(P, T // chunk, chunk, H, D)
    mu = xc.mean(axis=2, keepdims=True)
    d = xc - mu
    s = np.abs(d).max(axis=2, keepdims=True)
    y = np.clip(np.where(s > 0, d / np.where(s > 0, s, 1.0), 0.0), -1.0, 1.0)
    mag = np.abs(y)
    m = np.floor(127.0 * (_map(mag, alpha) if log_map else mag) + 0.5).astype(np.int64)
    neg = y < 0
    q = np.where(neg, -m - 1, m) if sign_aware else np.where(neg, -m, m)
    if anchor_only:
        rb = 8 - anchor_bits
        q = (q >> rb) * (1 << rb) + (((1 << rb) // 2 - 1) if midpoint and rb > 0 else 0)
    if sign_aware:
        mm, sgn = np.where(q < 0, -q - 1, q), np.where(q < 0, -1.0, 1.0)
    else:
        mm, sgn = np.abs(q), np.where(q < 0, -1.0, 1.0)
    yh = sgn * (_inv(mm / 127.0, alpha) if log_map else mm / 127.0)
    xr = (mu + s * yh).reshape(P, T, H, D)
    xh = mn + rg * xr if page_norm else xr
    bits = (float(anchor_bits) if anchor_only else 8.0) + 2 * 32.0 / chunk + \
        (2 * 32.0 / T if page_norm else 0.0)
    return xh, bits


def uniform_reconstruct(x: np.ndarray, bits: int, per: str):
    """Asymmetric uniform grid of 2^bits levels per token ('token': over the
    channels of one head) or per channel ('channel': over a page's tokens)."""
    axis = 3 if per == "token" else 1
    if x.shape[0] > 1:
        parts = [uniform_reconstruct(x[i:i + 1], bits, per) for i in range(x.shape[0])]
        return np.concatenate([p[0] for p in parts]), parts[0][1]
    lo = x.min(axis=axis, keepdims=True)
    hi = x.max(axis=axis, keepdims=True)
    step = np.where(hi > lo, (hi - lo) / (2 ** bits - 1), 1.0)
    code = np.clip(np.floor((x - lo) / step + 0.5), 0, 2 ** bits - 1)
    group = x.shape[3] if per == "token" else x.shape[1]
    return lo + code * step, bits + 2 * 16.0 / group


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm: float) -> np.ndarray:
    """float64 single-query GQA attention; q [Hq][D], k, v [T][H][D]."""
    Hq, D = q.shape
    T, H, _ = k.shape
    g = Hq // H
    out = np.empty((Hq, D))
    for h in range(H):
        s = q[h * g:(h + 1) * g] @ k[:, h].T * sm          # [g][T]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[h * g:(h + 1) * g] = p @ v[:, h]
    return out


def nmse(o_hat: np.ndarray, o: np.ndarray) -> float:
    return float(((o_hat - o) ** 2).sum() / (o ** 2).sum())


def study(cases, sm: float, chunks=(8, 16, 32, 64), alphas=(3, 15, 63),
          splits=(2, 3, 5, 6), pooled_parts: bool = False) -> Dict[str, Dict[str, float]]:
    """NMSE and bits per coordinate of every configuration, pooled over the
    cases (each a tuple xk, xv float64 [P][256][H][D] of one request and its
    queries q float64 [Hq][D]): the squared errors and the squared norms are
    summed over all cases before the ratio is taken."""
    configs = []
    lyn = lambda **kw: (lambda x: lynx_reconstruct(x, **kw))
    configs.append(("lynx_full", lyn()))
    configs.append(("lynx_anchor", lyn(anchor_only=True)))
    for b in (8, 4):
        for per in ("token", "channel"):
            configs.append(("uniform_int%d_per_%s" % (b, per),
                            lambda x, b=b, per=per: uniform_reconstruct(x, b, per)))
    for name, kw in (("no_page_norm", dict(page_norm=False)),
                     ("no_chunking", dict(chunk=PAGE)),
                     ("linear_map", dict(log_map=False)),
                     ("no_sign_aware", dict(sign_aware=False))):
        configs.append(("full_" + name, lyn(**kw)))
        configs.append(("anchor_" + name, lyn(anchor_only=True, **kw)))
    configs.append(("anchor_no_midpoint", lyn(anchor_only=True, midpoint=False)))
    for c in chunks:
        configs.append(("full_chunk_%d" % c, lyn(chunk=c)))
        configs.append(("anchor_chunk_%d" % c, lyn(anchor_only=True, chunk=c)))
    for a in alphas:
        configs.append(("full_alpha_%g" % a, lyn(alpha=a)))
        configs.append(("anchor_alpha_%g" % a, lyn(anchor_only=True, alpha=a)))
    for b in splits:  # the anchor of a b + (8 - b) split
        configs.append(("anchor_split_%d_%d" % (b, 8 - b), lyn(anchor_only=True, anchor_bits=b)))

    num = {name: 0.0 for name, _ in configs}
    bits = {}
    den = 0.0
    for xk, xv, q in cases:
        P, T, H, D = xk.shape
        flat = lambda a: a.reshape(P * T, H, D)
        ref = attention(q, flat(xk), flat(xv), sm)
        den += float((ref ** 2).sum())
        for name, f in configs:
            kh, bk = f(xk)
            vh, bv = f(xv)
            num[name] += float(((attention(q, flat(kh), flat(vh), sm) - ref) ** 2).sum())
            bits[name] = 0.5 * (bk + bv)
    if pooled_parts:  # the sums themselves, to pool over several processes
        out = {name: {"num": num[name], "bits": bits[name]} for name, _ in configs}
        out["__den"] = den
        return out
    return {name: {"nmse": num[name] / den, "bits": bits[name]} for name, _ in configs}


def synthetic_cases(workload: str = "ctx32k", tokens: int = 4096, requests: int = 1,
                    first_request: int = 0):
    """bf16 K, V pages and queries of requests first_request .. + requests of
    a workload, as float64 (xk, xv [P][256][H][D], q [Hq][D]) per request."""
    from long_context_serving_amd import synth
    w = synth.WORKLOADS[workload]
    to_f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qs = to_f(synth.queries(w, batch=requests, first_request=first_request))
    rs = range(first_request, first_request + requests)
    return w, [(to_f(synth.kv_pages(w, 0, 0, r, tokens=tokens)),
                to_f(synth.kv_pages(w, 0, 1, r, tokens=tokens)), qs[i]) for i, r in enumerate(rs)]


def _one_request(args):
    tokens, r = args
    _, cases = synthetic_cases(tokens=tokens, requests=1, first_request=r)
    return study(cases, 1.0 / np.sqrt(128.0), pooled_parts=True)


if __name__ == "__main__":
    import json
    import multiprocessing
    import sys
    tokens = int(sys.argv[1]) if len(sys.argv) > 1 else 8192
    requests = int(sys.argv[2]) if len(sys.argv) > 2 else 8
    workers = int(sys.argv[3]) if len(sys.argv) > 3 else 4
    with multiprocessing.Pool(workers) as pool:
        parts = pool.map(_one_request, [(tokens, r) for r in range(requests)])
    den = sum(p["__den"] for p in parts)
    res = {k: {"nmse": sum(p[k]["num"] for p in parts) / den, "bits": parts[0][k]["bits"]}
           for k in parts[0] if k != "__den"}
    print(json.dumps({"workload": "ctx32k", "tokens": tokens, "requests": requests,
                      "results": res}, indent=1))
