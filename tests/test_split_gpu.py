"""Parity of the b + (8 - b) cuts (through the C ABI) with the oracle.

Bar: the streams are bit-exact against the oracle's cut of the same codes,
packed in the documented order; the full reconstruction from the streams is
bit-identical to the 4 + 4 dequantizer; the draft is within 1e-3 relative of
the oracle's draft wherever the GPU and oracle codes agree (as for the 4 + 4
dequantizer).
"""
import numpy as np
import pytest

import oracle
from long_context_serving_amd import synth
from planes_layout import unpack_codes

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

RTOL_DQ = 1e-3
FLOOR_DQ = 1e-6


@pytest.fixture(scope="module")
def lynx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx as mod
    return mod


def stream_codes(pl, P, H):
    """Codes in stream order (the nibble order of the 4-bit planes): [P*H][32768] int8."""
    a = pl.anchor.cpu().numpy().reshape(P * H, -1)
    r = pl.residual.cpu().numpy().reshape(P * H, -1)
    nib = lambda b: np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[0], -1)
    return ((nib(a).astype(np.uint8) << 4) | nib(r).astype(np.uint8)).view(np.int8)


def pack_bits(values, bits):
    """LSB-first bit stream of `bits` bits per value, per row."""
    v = values.astype(np.int64) & ((1 << bits) - 1)
    b = ((v[..., None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(v.shape[0], -1)
    return np.packbits(b, axis=1, bitorder="little")


@pytest.mark.parametrize("role", [0, 1])
def test_cuts_streams_full_and_draft(lynx, role):
    P, H = 3, 2
    x = synth.laplace_pages(P, H, 128, seed=41 + role, scale_channels=((1, 5, 70.0),))
    pl = lynx.quantize_pages(torch.from_numpy(x.view(np.int16)).cuda(), role)
    torch.cuda.synchronize()
    codes = stream_codes(pl, P, H)
    full4 = lynx.dequantize(pl, full=True).cpu().numpy()
    enc = oracle.encode(x)
    _, _, gpu_code = unpack_codes(pl.anchor.cpu().numpy(), pl.residual.cpu().numpy(), P, H, role)
    same = gpu_code == enc["codes"]
    rg = np.broadcast_to(enc["page_range"][:, None].astype(np.float64), x.shape)
    for b in range(1, 8):
        print("cut %d + %d role %d" % (b, 8 - b, role), flush=True)
        sa, sr = lynx.split_planes(pl, b)
        torch.cuda.synchronize()
        a, r = oracle.split_bits(codes, b)
        np.testing.assert_array_equal(sa.cpu().numpy().reshape(P * H, -1), pack_bits(a, b))
        np.testing.assert_array_equal(sr.cpu().numpy().reshape(P * H, -1), pack_bits(r, 8 - b))
        # the full code does not depend on the cut
        full = lynx.dequantize_split(sa, sr, b, pl).cpu().numpy()
        np.testing.assert_array_equal(full, full4)
        # draft against the oracle's draft of its own codes
        got = lynx.dequantize_split(sa, None, b, pl).cpu().numpy().astype(np.float64)
        oa, _ = oracle.split_bits(enc["codes"], b)
        ref = oracle.dequant_bits(oa, None, b, enc)
        err = np.abs(got - ref)
        ok = (err <= RTOL_DQ * np.abs(ref)) | (err <= FLOOR_DQ * rg)
        assert ok[same].all(), (b, float(err[same & ~ok].max()))


def test_cut_4_draft_equals_the_anchor_dequantizer(lynx):
    P, H = 2, 3
    x = synth.laplace_pages(P, H, 128, seed=77)
    for role in (0, 1):
        pl = lynx.quantize_pages(torch.from_numpy(x.view(np.int16)).cuda(), role)
        sa, _ = lynx.split_planes(pl, 4)
        torch.cuda.synchronize()
        # the 4-bit anchor stream is the anchor plane itself
        assert torch.equal(sa, pl.anchor)
        d = lynx.dequantize_split(sa, None, 4, pl)
        assert torch.equal(d, lynx.dequantize(pl, full=False))


def test_empty_cut_is_a_noop(lynx):
    pl = lynx.alloc_planes(0, 2, 0)
    a, r = lynx.split_planes(pl, 3)
    assert a.numel() == 0 and r.numel() == 0
