"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test names the passage it pins.  Page references are to
"Lynx: the KV cache does not have to arrive whole" (sections 1-3) unless
stated.  None of these tests runs the HIP path.
"""
import functools
import json
import math
import os

import numpy as np
import pytest

import oracle
from long_context_serving_amd import synth

ALPHA = 255.0
HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))


def G(v):
    """Closed-form inverse of the alpha-law curve: ((1+alpha)^v - 1)/alpha."""
    return (np.power(1.0 + ALPHA, v) - 1.0) / ALPHA


def f32(x):
    return np.float32(x)


# ---------------------------------------------------------------------------
# Page constants (golden fixture: values printed on the page, cited there)
# ---------------------------------------------------------------------------
def test_page_constants_shape_the_oracle():
    """256-token pages, C = 32 chunks, 127 magnitude levels, 4 + 4 bits.

    Section 3.  Checked through behaviour: the number of chunk statistics per
    page, the set of magnitude levels reached, and the nibble ranges.
    """
    P, H, D = 2, 1, 8
    x = synth.laplace_pages(P, H, D, seed=3)
    enc = oracle.encode(x)
    assert x.shape[1] == GOLD["page_tokens"]["value"]
    assert enc["chunk_mean"].shape[2] * GOLD["chunk_tokens"]["value"] == GOLD["page_tokens"]["value"]
    # magnitude levels 0..127: every u in [0, 1] maps into them, 0 -> 0, 1 -> 127
    u = np.linspace(0.0, 1.0, 200001, dtype=np.float32)
    q, _ = oracle.codes(u)
    assert q.min() == 0 and q.max() == GOLD["magnitude_levels"]["value"]
    assert len(np.unique(q)) == GOLD["magnitude_levels"]["value"] + 1
    codes = np.arange(-128, 128)
    a, r = oracle.split(codes)
    assert a.min() == -(1 << (GOLD["anchor_bits"]["value"] - 1))
    assert a.max() == (1 << (GOLD["anchor_bits"]["value"] - 1)) - 1
    assert r.min() == 0 and r.max() == (1 << GOLD["residual_bits"]["value"]) - 1
    assert GOLD["anchor_bits"]["value"] + GOLD["residual_bits"]["value"] == GOLD["total_bits"]["value"]
    # the draft code is the +7 point of the anchor's 16-code interval
    assert np.array_equal(oracle.join(a) - 16 * a.astype(np.int32),
                          np.full(256, GOLD["round_half_down_bias"]["value"]))


# ---------------------------------------------------------------------------
# Pin 1: effective bin count 2^B * m_i / m (section 2)
# ---------------------------------------------------------------------------
def test_effective_bins_uniform_grid_vs_lynx():
    """A uniform 8-bit grid shared by all channels spans 2^B m_i/m codes on a
    normal channel when a few channels are 100x larger (section 2); Lynx's
    per-channel page normalisation and chunk scaling restore the full code
    range on the same channels (section 3)."""
    ratio = GOLD["outlier_ratio"]["value"]
    B = GOLD["grid_bits"]["value"]
    D = 128
    outl = (5, 40, 77, 101)
    x = synth.laplace_pages(1, 1, D, seed=11, scale_channels=tuple((0, d, float(ratio)) for d in outl))
    xf = oracle.bf16_bits_to_float(x)[0, :, 0, :].copy()     # [256][D]
    # channel 0's outlier twin: exactly 100x channel 0, so m_0 / m = 1/100
    xf[:, outl[0]] = xf[:, 0] * np.float32(ratio)
    xf = oracle.bf16_bits_to_float(synth.float_to_bf16_bits(xf))
    twin_is_extreme = xf[:, outl[0]].max() >= xf.max() and xf[:, outl[0]].min() <= xf.min()
    grid = oracle.uniform_codes(xf.reshape(1, -1), B).reshape(xf.shape)   # one grid per page
    m = float(xf.max()) - float(xf.min())
    steps = (1 << B) - 1
    for d in range(D):
        if d in outl:
            continue
        mi = float(xf[:, d].max()) - float(xf[:, d].min())
        span = int(grid[:, d].max() - grid[:, d].min()) + 1
        lo = math.floor(steps * mi / m) + 1
        hi = math.ceil(steps * mi / m) + 1
        assert lo <= span <= hi, (d, span, lo, hi)
    # the formula at a 100x ratio: 2^8/100 = 2.56 bins = 1.36 bits ("about 1.5")
    bits100 = math.log2((1 << B) / ratio)
    assert abs(bits100 - GOLD["effective_bits_at_100x"]["value"]) < 0.2
    if twin_is_extreme:
        m0 = float(xf[:, 0].max()) - float(xf[:, 0].min())
        assert abs(m0 / m - 1.0 / ratio) < 1e-2 / ratio
        span0 = int(grid[:, 0].max() - grid[:, 0].min()) + 1
        assert span0 in (2, 3, 4)          # 2.56 bins, +1 for straddling
    enc = oracle.encode(synth.float_to_bf16_bits(xf)[None, :, None, :])
    q = enc["codes"][0, :, 0, :]
    for d in range(D):
        # 256 tokens over 8 chunks: well over 64 distinct codes on every channel
        assert len(np.unique(q[:, d])) >= 64, d


# ---------------------------------------------------------------------------
# Pin 2: monotone code map, exhaustive over all fp32 u in [0, 1]
# ---------------------------------------------------------------------------
@pytest.mark.slow
def test_code_map_exhaustive_monotone_and_thresholds():
    """y -> q is non-decreasing on [0, 1] (section 3, logarithmic map onto
    127 levels); level k starts at the first fp32 u >= G((k - 1/2)/127),
    the closed-form inverse, up to the 2^-20 flag window."""
    top = int(np.float32(1.0).view(np.uint32))      # 0x3F800000
    block = 1 << 24
    prev_last = -1
    first_u = {}
    flagged = 0
    for start in range(0, top + 1, block):
        bits = np.arange(start, min(start + block, top + 1), dtype=np.uint32)
        u = bits.view(np.float32)
        q, flag = oracle.codes(u)
        flagged += int(flag.sum())
        qi = q.astype(np.int16)
        assert qi[0] >= prev_last
        assert np.all(np.diff(qi) >= 0)
        prev_last = int(qi[-1])
        steps = np.nonzero(np.diff(qi))[0] + 1
        for i in steps:
            assert int(qi[i]) - int(qi[i - 1]) == 1        # no level is skipped
            first_u[int(qi[i])] = (float(u[i - 1]), float(u[i]), int(flag[i]) | int(flag[i - 1]))
    assert prev_last == 127
    assert sorted(first_u) == list(range(1, 128))
    # every flagged u of [0, 1] lies in the windows around the 127 boundaries
    assert flagged == near_half_flag_count()
    for k, (below, at, flagged) in first_u.items():
        t = G((k - 0.5) / 127.0)
        if not flagged:
            assert below < t <= at or math.isclose(at, t, rel_tol=1e-6), (k, below, at, t)


# ---------------------------------------------------------------------------
# The near-half flag: set exactly where tau = 127 F(u) lies within 2^-20 of
# a rounding boundary k + 1/2 (the window in which the spec bar lets a
# code differ by one), with tau evaluated here in 40-digit decimal
# arithmetic, independently of the oracle's double-precision log1p.
# ---------------------------------------------------------------------------
_WINDOW = 64        # fp32 steps scanned on each side of every boundary


def _tau_decimal(u):
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    return 127 * (1 + 255 * Decimal(float(u))).ln() / Decimal(256).ln()


@functools.lru_cache(maxsize=1)
def _near_half_windows():
    """Per boundary k + 1/2 (k = 0..126): the fp32 bit patterns of u within
    _WINDOW steps of the first u with tau >= k + 1/2, and whether each lies
    within 2^-20 of the boundary (None where that is closer to 1e-12 than
    decimal vs double evaluation can decide)."""
    from decimal import Decimal
    band = Decimal(2) ** -20
    out = []
    for k in range(127):
        half = Decimal(k) + Decimal(1) / 2
        lo, hi = 0, 0x3F800000                       # tau(0) < half <= tau(1)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if _tau_decimal(np.uint32(mid).view(np.float32)) >= half:
                hi = mid
            else:
                lo = mid
        bits = np.arange(hi - _WINDOW, hi + _WINDOW + 1, dtype=np.uint32)
        want = []
        for b in bits:
            dist = abs(_tau_decimal(b.view(np.float32)) - half)
            want.append(None if abs(dist - band) < Decimal("1e-12") else dist < band)
        out.append((k, bits, want))
    return out


def test_near_half_flag_is_set_exactly_within_two_to_minus_20_of_a_boundary():
    total = 0
    for k, bits, want in _near_half_windows():
        _, flag = oracle.codes(bits.view(np.float32))
        assert not flag[0] and not flag[-1], k          # the band lies inside the window
        for f, w in zip(flag, want):
            if w is not None:
                assert bool(f) == w, (k, f, w)
        total += int(flag.sum())
    assert total > 0
    # away from the boundaries the flag is never set
    rng = np.random.default_rng(11)
    u = rng.random(200000).astype(np.float32)
    tau = oracle.tau(u)
    _, flag = oracle.codes(u)
    far = np.abs(tau - np.floor(tau) - 0.5) > 2.0 ** -19
    assert not flag[far].any()


def near_half_flag_count():
    """Number of fp32 u in [0, 1] the windows above flag."""
    total = 0
    for _, bits, _ in _near_half_windows():
        total += int(oracle.codes(bits.view(np.float32))[1].sum())
    return total


def test_yhat_monotone_and_closed_form():
    """q -> yhat is non-decreasing over the 256 codes and 1 + alpha |yhat| is
    (1 + alpha)^(m/127): reconstructed magnitude grows geometrically with the
    level (section 3, the cut)."""
    q = np.arange(-128, 128)
    y = oracle.yhat(q)
    dy = np.diff(y)
    assert np.all(dy >= 0)
    # strictly increasing except between -1 and 0, the two level-0 codes
    assert np.array_equal(np.nonzero(dy == 0)[0], [127])
    assert np.signbit(y[127]) and not np.signbit(y[128])
    m = np.where(q >= 0, q, -q - 1)
    np.testing.assert_allclose(1.0 + ALPHA * np.abs(y), np.power(256.0, m / 127.0), rtol=1e-14)
    assert y[q == 127][0] == 1.0 and y[q == -128][0] == -1.0
    assert y[q == 0][0] == 0.0 and y[q == -1][0] == 0.0


# ---------------------------------------------------------------------------
# Pin 3: sign preservation for small negatives (section 3)
# ---------------------------------------------------------------------------
def test_small_negatives_keep_their_sign_in_the_draft():
    half0 = G(0.5 / 127.0)                                  # 8.6555e-5
    assert abs(half0 - 8.6555e-5) < 1e-9
    u = np.geomspace(1e-9, half0 * 0.999, 50).astype(np.float32)
    q, _ = oracle.codes(u, np.ones(u.shape, np.uint8))
    assert np.all(q == -1)
    qp, _ = oracle.codes(u, np.zeros(u.shape, np.uint8))
    assert np.all(qp == 0)
    a, r = oracle.split(q)
    assert np.all(a == -1) and np.all(r == 15)
    draft = oracle.yhat(oracle.join(a))
    np.testing.assert_allclose(draft, -G(8 / 127.0), rtol=1e-14)
    assert np.all(draft < 0) and abs(draft[0] + 1.63952e-3) < 1e-8
    # a sign-agnostic cut would have drafted +G(7/127) = +1.40193e-3
    assert abs(G(7 / 127.0) - 1.40193e-3) < 1e-8


# ---------------------------------------------------------------------------
# Pin 4: the anchor names a geometric interval (section 3, the cut)
# ---------------------------------------------------------------------------
def test_anchor_interval_is_geometric():
    a = np.repeat(np.arange(-8, 8), 16).astype(np.int8)
    r = np.tile(np.arange(16), 16).astype(np.uint8)
    full = oracle.yhat(oracle.join(a, r))
    draft = oracle.yhat(oracle.join(a))
    ap = np.where(a >= 0, a, ~a).astype(np.float64)          # interval index
    lo, hi = G(16 * ap / 127.0), G((16 * ap + 15) / 127.0)
    for y in (full, draft):
        assert np.all(np.abs(y) >= lo * (1 - 1e-15)) and np.all(np.abs(y) <= hi * (1 + 1e-15))
        assert not np.signbit(y[a >= 0]).any() and np.signbit(y[a < 0]).all()
    # interval ends step by (1 + alpha)^(16/127) in the 1 + alpha|y| domain
    k = np.arange(8)
    ratio = (1 + ALPHA * G(16 * (k + 1) / 127.0)) / (1 + ALPHA * G(16 * k / 127.0))
    np.testing.assert_allclose(ratio, 256.0 ** (16 / 127.0), rtol=1e-13)
    assert abs(256.0 ** (16 / 127.0) - 2.010946) < 1e-6


# ---------------------------------------------------------------------------
# Pins 5 and 6: lossless recombination, centred residual (section 3)
# ---------------------------------------------------------------------------
def test_recombination_and_centring():
    q = np.arange(-128, 128).astype(np.int8)
    a, r = oracle.split(q)
    assert np.array_equal(oracle.join(a, r), q.astype(np.int32))
    assert np.array_equal(((a.astype(np.int32) << 4) | r), q.astype(np.int32))
    assert np.array_equal(oracle.yhat(oracle.join(a, r)), oracle.yhat(q))
    e = r.astype(np.int32) - GOLD["round_half_down_bias"]["value"]
    assert e.min() == -7 and e.max() == 8
    draft, full = oracle.join(a), oracle.join(a, r)
    assert np.array_equal(draft == full, r == 7)


def test_dequant_full_equals_8bit_decode_on_encoded_pages():
    x = synth.laplace_pages(2, 2, 16, seed=5, scale_channels=((1, 3, 100.0),))
    enc = oracle.encode(x)
    a, r = oracle.split(enc["codes"])
    full = oracle.dequant(a, r, enc)
    P, T, H, D = x.shape
    c = np.arange(T) // 32
    pm = enc["page_min"][:, None].astype(np.float64)
    pr = enc["page_range"][:, None].astype(np.float64)
    cm = np.transpose(enc["chunk_mean"], (0, 2, 1, 3))[:, c].astype(np.float64)
    cs = np.transpose(enc["chunk_maxabs"], (0, 2, 1, 3))[:, c].astype(np.float64)
    direct = pm + pr * (cm + cs * oracle.yhat(enc["codes"]))
    assert np.array_equal(full, direct)


# ---------------------------------------------------------------------------
# Pin 7: closed forms and the reconstruction error bound (sections 2-3)
# ---------------------------------------------------------------------------
def _stats_per_element(enc, T):
    c = np.arange(T) // 32
    pm = enc["page_min"][:, None].astype(np.float64)
    pr = enc["page_range"][:, None].astype(np.float64)
    cm = np.transpose(enc["chunk_mean"], (0, 2, 1, 3))[:, c].astype(np.float64)
    cs = np.transpose(enc["chunk_maxabs"], (0, 2, 1, 3))[:, c].astype(np.float64)
    return pm, pr, cm, cs


def test_reconstruction_error_bound_full_and_draft():
    """|x - xhat| <= range * maxabs * (half a level width of the map), plus the
    fp32 pipeline's rounding: the full code is a nearest level of a monotone
    map; the draft stays inside the anchor's interval."""
    x = synth.laplace_pages(3, 2, 32, seed=9, scale_channels=((0, 1, 100.0), (1, 30, 60.0)))
    enc = oracle.encode(x)
    a, r = oracle.split(enc["codes"])
    xf = oracle.bf16_bits_to_float(x).astype(np.float64)
    pm, pr, cm, cs = _stats_per_element(enc, x.shape[1])
    q = enc["codes"].astype(np.int32)
    m = np.where(q >= 0, q, -q - 1).astype(np.float64)
    halfw = np.maximum(G(np.minimum(m + 0.5, 127) / 127.0) - G(m / 127.0),
                       G(m / 127.0) - G(np.maximum(m - 0.5, 0) / 127.0))
    slack = 4 * 2.0 ** -23 * pr      # fp32 normalisation rounding, in x units
    full = oracle.dequant(a, r, enc)
    assert np.all(np.abs(full - xf) <= pr * cs * halfw + slack)
    draft = oracle.dequant(a, None, enc)
    ap = np.where(a >= 0, a, ~a).astype(np.float64)
    width = G((16 * ap + 15) / 127.0) - G(16 * ap / 127.0)
    assert np.all(np.abs(draft - xf) <= pr * cs * (width + halfw) + slack)


def test_maxabs_element_and_degenerate_channels():
    x = synth.laplace_pages(1, 2, 8, seed=21)
    x[0, :, 0, 2] = synth.float_to_bf16_bits(np.float32(3.25))      # constant channel: range 0
    blk = oracle.bf16_bits_to_float(x[0, :, 1, 5]).copy()
    blk[64:96] = blk[70]                                             # constant chunk 2: maxabs 0
    x[0, :, 1, 5] = synth.float_to_bf16_bits(blk)
    enc = oracle.encode(x)
    a, r = oracle.split(enc["codes"])
    full = oracle.dequant(a, r, enc)
    # range 0: all codes 0, exact reconstruction of the constant
    assert enc["page_range"][0, 0, 2] == 0.0
    assert np.all(enc["codes"][0, :, 0, 2] == 0)
    assert np.all(full[0, :, 0, 2] == 3.25)
    # maxabs 0 in one chunk: codes 0 there, xhat = min + range * mean
    assert enc["chunk_maxabs"][0, 1, 2, 5] == 0.0
    assert np.all(enc["codes"][0, 64:96, 1, 5] == 0)
    want = float(enc["page_min"][0, 1, 5]) + float(enc["page_range"][0, 1, 5]) * float(enc["chunk_mean"][0, 1, 2, 5])
    assert np.all(full[0, 64:96, 1, 5] == want)
    # every element whose deviation equals the chunk max-abs has |y| = 1 up
    # to the rounding of |d| / s (at most one ulp below 1), so lands on
    # level 127 (the closed form |y| = 1 -> 127 -> yhat = +-1)
    q = enc["codes"].astype(np.int32)
    m = np.where(q >= 0, q, -q - 1)
    xn, _ = _fp32_chain(x)
    for c in range(8):
        for h in range(2):
            for d in range(8):
                s = enc["chunk_maxabs"][0, h, c, d]
                if s > 0:
                    dev = np.abs((xn[0, 32 * c:32 * c + 32, h, d] -
                                  enc["chunk_mean"][0, h, c, d]).astype(np.float32))
                    top = dev == s
                    assert top.any()
                    assert np.all(m[0, 32 * c:32 * c + 32, h, d][top] == 127)
                    y = (dev[top] * np.float32(1.0 / np.float64(s))).astype(np.float32)
                    assert np.all(y >= np.float32(1.0) - np.float32(2.0 ** -23))


def test_ramp_pages_closed_form_codes():
    """Exact ramps give page and chunk statistics in closed form, so codes
    are known per token: m = round(127 F(|2(t - 32c) - 31| / 31)).  The ramp
    counts 0..255 with a step skipped after 127 (values t + [t >= 128], times
    2^k, or reversed), so the page range is 256 * 2^k and x' = value / 256
    exactly.  Different heads/channels carry different ramps, pinning the
    oracle's page, chunk, head and channel indexing."""
    H, D = 3, 8
    x = np.empty((2, 256, H, D), np.float32)
    t = np.arange(256, dtype=np.float32)
    tp = t + (t >= 128)                       # 0 .. 127, 129 .. 256
    for p in range(2):
        for h in range(H):
            for d in range(D):
                k = (d + 2 * h + p) % 6 - 2
                ramp = tp if (d + h + p) % 2 == 0 else 256.0 - tp
                x[p, :, h, d] = ramp * np.float32(2.0 ** k) - np.float32(2.0 ** (k + 5)) * h
    xb = synth.float_to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_float(xb), x)   # exactly representable
    enc = oracle.encode(xb)
    tl = np.arange(256) % 32
    u = np.abs(2.0 * tl - 31.0) / 31.0
    tau = 127.0 * np.log1p(ALPHA * u) / np.log1p(ALPHA)
    want_m = np.floor(tau + 0.5).astype(np.int32)
    safe = np.abs(tau - np.floor(tau) - 0.5) > 1e-3
    c = np.arange(8)
    up_mu = (32 * c + 15.5 + (c >= 4)) / 256.0
    for p in range(2):
        for h in range(H):
            for d in range(D):
                rev = (d + h + p) % 2 == 1
                neg = (tl < 15.5) if not rev else (tl > 15.5)
                want = np.where(neg, -want_m - 1, want_m)
                got = enc["codes"][p, :, h, d].astype(np.int32)
                assert np.array_equal(got[safe], want[safe]), (p, h, d)
                k = (d + 2 * h + p) % 6 - 2
                assert enc["page_range"][p, h, d] == np.float32(256.0 * 2.0 ** k)
                want_mu = up_mu if not rev else 1.0 - up_mu
                assert np.array_equal(enc["chunk_mean"][p, h, :, d], want_mu.astype(np.float32))
                assert np.all(enc["chunk_maxabs"][p, h, :, d] == np.float32(15.5 / 256.0))


def _fp32_chain(x_bits):
    """x' = RN32(RN32(x - min) * RN32(1/range)) per page and channel, with
    numpy's IEEE float32 operations: ([P][256][H][D], range [P][H][D])."""
    xf = oracle.bf16_bits_to_float(x_bits)
    mn = xf.min(axis=1, keepdims=True)
    rg = (xf.max(axis=1, keepdims=True) - mn).astype(np.float32)
    with np.errstate(divide="ignore"):  # degenerate channels take 0 below
        inv = np.where(rg > 0, (1.0 / rg.astype(np.float64)).astype(np.float32), np.float32(0.0))
    return ((xf - mn).astype(np.float32) * inv).astype(np.float32), rg[:, 0]


def _rn32(fr):
    """Round an exact rational to the nearest fp32 (ties to even)."""
    from fractions import Fraction
    f = np.float32(float(fr))             # within one ulp of the answer
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1)
    return min(cands, key=key)


def test_scales_are_plain_fp32_range_mean_and_maxabs():
    """Section 3: the page range is the page's max minus min (one fp32
    subtraction), the chunk mean the exact mean of the chunk's 32
    normalised values rounded once to fp32 (exact rational arithmetic here),
    and the chunk max-abs the largest |x' - mean| -- no extra rounding of
    any scale."""
    from fractions import Fraction
    x = synth.laplace_pages(2, 2, 16, seed=52, scale_channels=((1, 4, 100.0),))
    enc = oracle.encode(x)
    xn, rg = _fp32_chain(x)
    assert np.array_equal(enc["page_range"].view(np.uint32), rg.view(np.uint32))
    P, _, H, D = x.shape
    for p in range(P):
        for h in range(H):
            for c in range(8):
                for d in range(D):
                    vals = xn[p, 32 * c:32 * c + 32, h, d]
                    mu = _rn32(sum(Fraction(float(v)) for v in vals) / 32)
                    assert enc["chunk_mean"][p, h, c, d] == mu, (p, h, c, d)
                    s = np.abs((vals - mu).astype(np.float32)).max()
                    assert enc["chunk_maxabs"][p, h, c, d] == s, (p, h, c, d)


def test_chunk_mean_is_exact_when_a_double_sum_would_round():
    """Values far below the page range (nonzero x' under 2^-24) next to a
    large one: a plain double-precision sum of such a chunk can round; the
    oracle's mean is still the exactly rounded one, and exactly those chunks
    are flagged."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    xf = np.zeros((1, 256, 1, 8), np.float32)
    for d in range(8):
        base = np.float32(-(2.0 ** -(20 + d)))
        xf[0, :, 0, d] = base * (1 + rng.integers(0, 128, 256) / np.float32(128.0))
        xf[0, 200, 0, d] = np.float32(96.0 * (d + 1))       # sets the range
    xb = synth.float_to_bf16_bits(xf)
    enc = oracle.encode(xb)
    xn, _ = _fp32_chain(xb)
    tiny = (xn != 0) & (xn < 2.0 ** -24)
    assert tiny[0, :192].any()
    for c in range(8):
        for d in range(8):
            vals = xn[0, 32 * c:32 * c + 32, 0, d]
            assert enc["chunk_mean"][0, 0, c, d] == _rn32(sum(Fraction(float(v)) for v in vals) / 32)
            chunk_tiny = tiny[0, 32 * c:32 * c + 32, 0, d].any()
            flags = enc["flags"][0, 32 * c:32 * c + 32, 0, d]
            assert np.all(((flags & oracle.FLAG_SUM_INEXACT) != 0) == chunk_tiny)


# ---------------------------------------------------------------------------
# Pin 8: exact power-of-two invariance (section 3: an extreme channel sets
# only its own scale)
# ---------------------------------------------------------------------------
def test_power_of_two_channel_scaling_is_exact():
    x = synth.laplace_pages(2, 2, 16, seed=31)
    enc = oracle.encode(x)
    xs = oracle.bf16_bits_to_float(x).copy()
    xs[:, :, 1, 7] *= np.float32(64.0)
    xs[:, :, 0, 3] *= np.float32(0.125)
    enc2 = oracle.encode(synth.float_to_bf16_bits(xs))
    assert np.array_equal(enc["codes"], enc2["codes"])
    assert np.array_equal(enc["chunk_mean"], enc2["chunk_mean"])
    assert np.array_equal(enc["chunk_maxabs"], enc2["chunk_maxabs"])
    assert np.array_equal(enc2["page_min"][:, 1, 7], enc["page_min"][:, 1, 7] * 64)
    assert np.array_equal(enc2["page_range"][:, 0, 3], enc["page_range"][:, 0, 3] * np.float32(0.125))


# ---------------------------------------------------------------------------
# Pin 9: stage order -- codes equal the exact-arithmetic chain
# ---------------------------------------------------------------------------
def test_stage_order_matches_exact_arithmetic():
    """In exact arithmetic y = (x - (min + range*mean)) / (range*maxabs).  The
    oracle's fp32 chain agrees except within the pipeline's rounding of a
    level boundary."""
    x = synth.laplace_pages(2, 2, 64, seed=41, scale_channels=((0, 9, 100.0),))
    enc = oracle.encode(x)
    xf = oracle.bf16_bits_to_float(x).astype(np.float64)
    pm, pr, cm, cs = _stats_per_element(enc, x.shape[1])
    y = (xf - (pm + pr * cm)) / (pr * cs)
    y = np.clip(y, -1.0, 1.0)
    tau = 127.0 * np.log1p(ALPHA * np.abs(y)) / np.log1p(ALPHA)
    m = np.floor(tau + 0.5).astype(np.int32)
    want = np.where(y < 0, -m - 1, m)
    got = enc["codes"].astype(np.int32)
    # error of y from the fp32 chain, in level units, bounded by slope * eps / maxabs
    eps = 8 * 2.0 ** -24 / cs * 5840.2
    near = np.abs(tau - np.floor(tau) - 0.5) <= eps
    tiny = np.abs(y) * 5840.2 < eps        # sign of |y| ~ ulp may flip
    ok = (got == want) | near | tiny
    assert ok.all()
    assert (got == want).mean() > 0.995


# ---------------------------------------------------------------------------
# Pin 10: brute-force attention against torch's SDPA (float64, CPU)
# ---------------------------------------------------------------------------
def test_attention_matches_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    B, T, H, g, D = 2, 300, 2, 4, 16
    q = rng.standard_normal((B, H * g, D))
    k = rng.standard_normal((B, T, H, D)) * 3
    v = rng.standard_normal((B, T, H, D))
    sc = 1.0 / math.sqrt(D)
    out, logits = oracle.attention(q, k, v, sc, want_logits=True)
    qt = torch.from_numpy(q)[:, :, None, :]                          # [B][Hq][1][D]
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sc)[:, :, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12, rtol=1e-12)
    ref_logits = torch.einsum("bjd,bjtd->bjt", torch.from_numpy(q), kt).numpy() * sc
    np.testing.assert_allclose(logits, ref_logits, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    D = 8
    v = rng.standard_normal((1, 5, 1, D))
    # one token: the output is that token's value
    out = oracle.attention(rng.standard_normal((1, 2, D)), rng.standard_normal((1, 1, 1, D)),
                           v[:, :1], 0.3)
    np.testing.assert_array_equal(out[0, 0], v[0, 0, 0])
    # identical keys, or a zero query: the plain mean of the values
    kk = np.repeat(rng.standard_normal((1, 1, 1, D)), 5, axis=1)
    out = oracle.attention(rng.standard_normal((1, 1, D)), kk, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, :, 0].mean(axis=0), atol=1e-14)
    out = oracle.attention(np.zeros((1, 1, D)), rng.standard_normal((1, 5, 1, D)), v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, :, 0].mean(axis=0), atol=1e-14)
    # GQA: query head j reads KV head j // g
    k2 = rng.standard_normal((1, 5, 2, D))
    v2 = rng.standard_normal((1, 5, 2, D))
    q2 = rng.standard_normal((1, 4, D))
    out = oracle.attention(q2, k2, v2, 0.5)
    for j in range(4):
        solo = oracle.attention(q2[:, j:j + 1], k2[:, :, j // 2:j // 2 + 1], v2[:, :, j // 2:j // 2 + 1], 0.5)
        np.testing.assert_array_equal(out[0, j], solo[0, 0])


# ---------------------------------------------------------------------------
# Pin 9b: other cuts of the 8-bit code (b + (8 - b))
# ---------------------------------------------------------------------------
def test_other_cuts_split_join_and_draft_centre():
    q = np.arange(-128, 128).astype(np.int8)
    for b in range(1, 9):
        a, r = oracle.split_bits(q, b)
        rb = 8 - b
        # a lossless cut: anchor and residual give the code back
        np.testing.assert_array_equal(oracle.join_bits(a, r, b), q.astype(np.int32))
        assert a.min() == -(1 << (b - 1)) and a.max() == (1 << (b - 1)) - 1
        assert r.max() == (1 << rb) - 1
        # the draft is the round-half-down centre of the anchor's codes
        lo = a.astype(np.int64) * (1 << rb)
        hi = lo + (1 << rb) - 1
        d = oracle.join_bits(a, None, b)
        np.testing.assert_array_equal(d, np.floor((lo + hi) / 2).astype(np.int64))
        assert (np.diff(d) >= 0).all()
    # b = 4 is the page's cut (+7 centre)
    a4, r4 = oracle.split(q)
    a, r = oracle.split_bits(q, 4)
    np.testing.assert_array_equal(a, a4)
    np.testing.assert_array_equal(r, r4)
    np.testing.assert_array_equal(oracle.join_bits(a, None, 4), 16 * a4.astype(np.int32) + 7)


def test_other_cuts_dequant():
    x = synth.laplace_pages(2, 2, 16, seed=31, scale_channels=((1, 3, 60.0),))
    enc = oracle.encode(x)
    a4, r4 = oracle.split(enc["codes"])
    full = oracle.dequant(a4, r4, enc)
    draft4 = oracle.dequant(a4, None, enc)
    for b in range(1, 9):
        a, r = oracle.split_bits(enc["codes"], b)
        # the full reconstruction does not depend on the cut
        np.testing.assert_array_equal(oracle.dequant_bits(a, r, b, enc), full)
        d = oracle.dequant_bits(a, None, b, enc)
        if b == 4:
            np.testing.assert_array_equal(d, draft4)
        if b == 8:
            np.testing.assert_array_equal(d, full)
    # more anchor bits, closer drafts (mean squared error against the full code)
    err = [float(((oracle.dequant_bits(*oracle.split_bits(enc["codes"], b)[:1], None, b, enc) - full) ** 2).mean())
           for b in range(1, 8)]
    assert all(err[i + 1] < err[i] for i in range(6)), err


# ---------------------------------------------------------------------------
# Pin 10b: several query tokens over prefixes of the cache (the verify pass)
# against torch's SDPA with an explicit mask (float64, CPU)
# ---------------------------------------------------------------------------
def test_prefix_attention_matches_masked_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    B, Tq, T, H, g, D = 2, 5, 40, 2, 3, 16
    q = rng.standard_normal((B, Tq, H * g, D))
    k = rng.standard_normal((B, T, H, D)) * 3
    v = rng.standard_normal((B, T, H, D))
    vis = np.array([[36, 37, 38, 39, 40], [1, 2, 17, 30, 40]])
    sc = 1.0 / math.sqrt(D)
    out = oracle.prefix_attention(q, k, v, vis, sc)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()                 # [B][Hq][Tq][D]
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    mask = torch.from_numpy(np.arange(T)[None, None, :] < vis[:, :, None])[:, None]  # [B][1][Tq][T]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sc)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=1e-12)


def test_prefix_attention_special_cases():
    rng = np.random.default_rng(18)
    B, Tq, T, H, D = 1, 3, 12, 1, 8
    q = rng.standard_normal((B, Tq, 2, D))
    k = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, D))
    vis = np.array([[1, 6, 12]])
    out = oracle.prefix_attention(q, k, v, vis, 0.4)
    # one visible token: its value
    np.testing.assert_array_equal(out[0, 0, 0], v[0, 0, 0])
    # tokens past a query's prefix do not reach it
    k2, v2 = k.copy(), v.copy()
    k2[0, 6:] += 50.0
    v2[0, 6:] -= 7.0
    out2 = oracle.prefix_attention(q, k2, v2, vis, 0.4)
    np.testing.assert_array_equal(out2[0, :2], out[0, :2])
    assert not np.allclose(out2[0, 2], out[0, 2])
    # the whole sequence visible: the single-query attention
    full = oracle.attention(q[:, 2], k, v, 0.4)
    np.testing.assert_allclose(out[0, 2], full[0], atol=1e-15)


def test_verify_attention_sees_pages_and_tail_up_to_itself():
    rng = np.random.default_rng(19)
    H, D, Tq = 1, 8, 3
    pages = rng.standard_normal((256, H, D))
    tail = rng.standard_normal((10, H, D)).astype(np.float32)
    tail_bits = (tail.view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16
    tail_f = oracle.bf16_bits_to_float(tail_bits).astype(np.float64)
    q_bits = (rng.standard_normal((1, Tq, 2, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = oracle.verify_attention(q_bits, [pages], [pages * 0.5], [tail_bits], [tail_bits], [7], 0.3)
    # token i (of the Tq = 3 newest of 7 tail tokens) sees 256 + 5 + i tokens
    k = np.concatenate([pages, tail_f[:7]])[None]
    v = np.concatenate([pages * 0.5, tail_f[:7]])[None]
    qf = oracle.bf16_bits_to_float(q_bits).astype(np.float64)
    for i in range(Tq):
        ref = oracle.attention(qf[:, i], k[:, :256 + 5 + i], v[:, :256 + 5 + i], 0.3)
        np.testing.assert_allclose(out[0, i], ref[0], atol=1e-15)


# ---------------------------------------------------------------------------
# Pin 11: the size arithmetic of section 1
# ---------------------------------------------------------------------------
def test_qwen3_235b_kv_size():
    g = GOLD["qwen3_235b_a22b"]
    nbytes = g["layers"] * 2 * g["kv_heads"] * g["head_dim"] * g["tokens"] * 2
    assert nbytes == 25_232_932_864 == 23.5 * 2 ** 30
    assert abs(nbytes / 1e9 - g["bf16_gb_approx"]) < 2.0         # "roughly 23.5 GB"
    assert abs(nbytes * 8 / 100e9 - g["seconds_at_100gbps_approx"]) < 0.05
    assert nbytes * 8 / 400e9 > g["seconds_at_400gbps_min"]
    w = synth.WORKLOADS["qwen3_235b_128k"]
    assert w.elements() * 2 == nbytes


# ---------------------------------------------------------------------------
# Pin 12: generator shape (section 2: values cluster near the centre)
# ---------------------------------------------------------------------------
def test_generator_laplacian_shape_and_outliers():
    w = synth.WORKLOADS["ctx32k"]
    x = oracle.bf16_bits_to_float(synth.kv_pages(w, 0, 0, 0, tokens=256 * 64))
    mask = synth.outlier_mask(w)
    assert mask.sum(axis=1).tolist() == [round(0.02 * 128)] * w.kv_heads
    spans = []
    for p in range(0, 64, 4):
        for h in range(w.kv_heads):
            for d in np.nonzero(~mask[h])[0][:16]:
                col = x[p, :, h, d]
                q25, q75 = np.quantile(col, [0.25, 0.75])
                spans.append((q75 - q25) / (col.max() - col.min()))
    # Laplace(0,1) pages of 256: the middle half spans ~13% of the range
    # (the page reports 17% on real KV)
    assert 0.10 < float(np.mean(spans)) < 0.17
    big = np.abs(x[..., mask]).mean() / np.abs(x[..., ~mask]).mean()
    assert 20 < big < 120


def test_oracle_is_thread_count_invariant():
    x = synth.laplace_pages(3, 2, 16, seed=77, scale_channels=((0, 0, 100.0),))
    e1 = oracle.encode(x, nthreads=1)
    e4 = oracle.encode(x, nthreads=4)
    for key in e1:
        assert np.array_equal(e1[key], e4[key])
