"""Progressive plane streaming (anchor planes first, residual planes after).

CPU: the top-k overlap report against a brute-force count.
GPU: a 3-layer, 4K-token run of the streaming schedule.  The streamed
device planes must equal the pinned host planes, and the drafts and full
outputs computed on arrival must equal direct calls bit for bit.  Layer 0's
planes must match the oracle's codes and scales, and its attention must
meet the attention bar.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

SM = float(np.float32(1.0 / math.sqrt(128.0)))


def test_topk_overlap_matches_brute_force():
    from long_context_serving_amd.stream import topk_overlap
    g = torch.Generator().manual_seed(3)
    a = torch.randn((6, 500), generator=g)
    b = a + 0.3 * torch.randn((6, 500), generator=g)
    got = topk_overlap(a, b, (1, 5, 40))
    for k, v in got.items():
        hits = [len(set(np.argsort(-a[i].numpy())[:k]) & set(np.argsort(-b[i].numpy())[:k]))
                for i in range(6)]
        assert abs(v - np.mean(hits) / k) < 1e-12
    assert topk_overlap(a, a, (7,))[7] == 1.0


@pytest.mark.gpu
def test_progressive_stream_small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from long_context_serving_amd import lynx, stream, synth
    from planes_layout import unpack_codes

    w = synth.WORKLOADS["progressive32x64k"]
    L, T = 3, 4096
    print("progressive stream: %d layers x %d tokens" % (L, T), flush=True)
    layers = stream.build_layers(w, device="cuda", layers=L, tokens=T)
    ps = stream.ProgressiveStream(layers, device="cuda", sm_scale=SM)
    t = ps.run_progressive()
    assert 0 < t["anchors_landed_ms"] <= t["residuals_landed_ms"]
    assert t["first_draft_layer_ms"] <= t["all_drafts_ms"] <= t["all_full_ms"]
    assert t["all_full_ms"] >= t["residuals_landed_ms"]

    for i, l in enumerate(layers):
        for dv, hv in ((ps.dev_k[i], l.host_k), (ps.dev_v[i], l.host_v)):
            for a, b in zip(stream._planes_tensors(dv, True, True), stream._planes_tensors(hv, True, True)):
                assert torch.equal(a.cpu(), b)
        for full, got in ((False, ps.out_draft[i]), (True, ps.out_full[i])):
            k, v = ps.dev_k[i], ps.dev_v[i]
            if not full:
                k, v = k.without_residual(), v.without_residual()
            ref = lynx.decode_attention(l.q, k, v, ps.pages, full=full, sm_scale=SM)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), "layer %d full=%s" % (i, full)

    i8 = ps.run_layerwise_int8()
    assert i8["first_layer_ms"] <= i8["all_full_ms"]
    for i, l in enumerate(layers):
        ref = lynx.decode_attention(l.q, ps.dev_k[i], ps.dev_v[i], ps.pages, full=True, sm_scale=SM)
        torch.cuda.synchronize()
        assert torch.equal(ps.out_full[i], ref)

    # layer 0 against the oracle: the same device-drawn bf16 input
    P, H = T // 256, w.kv_heads
    encs = []
    for tensor, role, host in ((0, 0, layers[0].host_k), (1, 1, layers[0].host_v)):
        x = synth.device_kv_pages(w, 0, tensor, 0, device="cuda", tokens=T).cpu().numpy().view(np.uint16)
        enc = oracle.encode(x)
        _, _, code = unpack_codes(host.anchor.numpy(), host.residual.numpy(), P, H, role)
        near = (enc["flags"] & oracle.FLAG_NEAR_HALF) != 0
        mism = code != enc["codes"]
        assert not (mism & ~near).any()
        for f in stream.SCALE_FIELDS:
            assert np.array_equal(getattr(host, f).numpy().reshape(enc[f].shape).view(np.uint32),
                                  enc[f].view(np.uint32)), f
        encs.append(enc)
    q = oracle.bf16_bits_to_float(layers[0].q.cpu().numpy().view(np.uint16)).astype(np.float64)
    for full, got in ((False, ps.out_draft[0]), (True, ps.out_full[0])):
        ak, rk = oracle.split(encs[0]["codes"])
        av, rv = oracle.split(encs[1]["codes"])
        kh = oracle.dequant(ak, rk if full else None, encs[0]).reshape(1, T, H, 128)
        vh = oracle.dequant(av, rv if full else None, encs[1]).reshape(1, T, H, 128)
        ref = oracle.attention(q, kh, vh, SM)
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
        print("layer 0 full=%s: max abs err %.3g" % (full, err.max()), flush=True)
        assert (err <= 2e-3 + 1e-5 * np.abs(ref)).all()

    ov = ps.draft_full_topk_overlap((1, 16))
    assert all(0.0 <= v <= 1.0 for v in ov.values())


@pytest.mark.gpu
def test_paced_link_timeline():
    """Throttled link (10 Gbps): the planes land when the link would have
    delivered them, in the order of each schedule, and arrive intact."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_serving_amd import lynx, stream, synth

    w = synth.WORKLOADS["progressive32x64k"]
    L, T, gbps = 3, 4096, 10.0
    print("paced link: %d layers x %d tokens at %.0f Gbps" % (L, T, gbps), flush=True)
    layers = stream.build_layers(w, device="cuda", layers=L, tokens=T)
    ps = stream.ProgressiveStream(layers, device="cuda", sm_scale=SM)
    link = stream.PacedLink(gbps, ps.copy_stream, piece_bytes=1 << 20)
    rate = gbps * 1e9 / 8 / 1e3  # bytes per ms
    ab, rb = ps.anchor_bytes(), ps.residual_bytes()
    # the start event runs on the GPU a little after the host starts the
    # link's clock, so lower bounds get a small allowance
    lo = lambda nbytes: 0.98 * nbytes / rate - 0.3

    p = ps.paced_progressive(link)
    print("progressive:", p, flush=True)
    # the anchors of every layer take ab / rate on the link, then the residuals
    assert lo(ab) <= p["anchors_landed_ms"] <= 1.25 * ab / rate + 3.0
    assert lo(ab + rb) <= p["residuals_landed_ms"] <= 1.25 * (ab + rb) / rate + 3.0
    assert p["first_draft_ms"] <= p["all_drafts_ms"] <= p["first_full_layer_ms"] <= p["all_full_ms"]
    for i, l in enumerate(layers):
        ref = lynx.decode_attention(l.q, ps.dev_k[i], ps.dev_v[i], ps.pages, full=True, sm_scale=SM)
        torch.cuda.synchronize()
        assert torch.equal(ps.out_full[i], ref)

    i8 = ps.paced_layerwise_int8(link)
    print("int8 layer-wise:", i8, flush=True)
    assert lo((ab + rb) / L) <= i8["first_full_layer_ms"] <= i8["all_full_ms"]
    assert lo(ab + rb) <= i8["all_full_ms"]

    bf16_layer = 2 * T * w.kv_heads * 128 * 2
    hb = torch.zeros(bf16_layer, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(bf16_layer, dtype=torch.uint8, device="cuda")
    bf = ps.paced_bf16(link, hb, db)
    print("bf16 layer-wise:", bf, flush=True)
    assert lo(L * bf16_layer) <= bf["all_landed_ms"] <= 1.25 * L * bf16_layer / rate + 3.0
    # the first draft needs a layer's anchors, the first full INT8 layer its
    # whole planes, the first bf16 layer twice the INT8 bytes and more
    assert p["first_draft_ms"] < i8["first_full_layer_ms"] < bf["first_layer_landed_ms"]
