#!/usr/bin/env python3
"""Benchmark of the Lynx hot path on one MI355X.

One step = encode of the whole K and V cache of the workload (page/chunk
statistics, alpha-law codes, anchor/residual planes), then anchor-only and
full fused-dequant single-query decode attention.  Inputs are seeded
synthetic Laplacian KV with outlier channels (long_context_serving_amd/synth.py),
resident in HBM before timing starts.  A step encodes K and V of one buffer
set and runs anchor-only and full decode over it.  To keep the 256 MB
Infinity Cache from serving the data, S distinct buffer sets (>= 1.5 GB in
total) are used; steps run in rounds of S, each phase of a round one HIP
graph of back-to-back launches, with events on the launch stream between
the phases giving every kernel's time inside the timed region.

Prints ONE JSON line.  Throughput counts algorithmic bytes: encode
3.28125 B per K/V element (2 read, 0.5 + 0.5 + 0.03125 + 0.25 written; one
launch encodes K and V),
full decode 1.28125 B and anchor-only decode 0.78125 B per element (plus
query and output).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode GB/s + fused-dequant decode-attn GB/s (% of HBM peak), 1×MI355X"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
ENCODER_SOURCE = os.path.join(ROOT, "long_context_serving_amd", "csrc", "lynx_encode.hip")
TRAFFIC_SUMMARY = os.path.join(PROFILES, "encode_kv_kernel_ctx32k_hbm_traffic.txt")
COPY_PROBE_BYTES = 256 << 20


def source_sha1(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha1(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per encoder launch from the committed counter summary, or
    None when the summary is missing or was taken on another encoder source."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    if kv.get("encoder_source_sha1", "").strip() != source_sha1(ENCODER_SOURCE):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize(kind, db_dir, out_path, command):
    """Write a short text summary of rocprofv3 output (kernel trace with
    --stats, FETCH_SIZE / WRITE_SIZE counter runs, or a run of SQ counters
    and derived metrics) under profiles/."""
    import glob
    import sqlite3

    def dbs(d):
        return sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))

    def short(name):
        name = name.replace("lynx::(anonymous namespace)::", "").replace("void ", "")
        return name.split("(")[0]

    lines = ["command: %s" % command]
    if kind == "sq":
        # per kernel: the average of every collected counter over its dispatches
        per = {}
        for db in dbs(db_dir):
            con = sqlite3.connect(db)
            for name, ctr, val in con.execute(
                    "select kernel_name, counter_name, value from counters_collection"):
                per.setdefault(short(name), {}).setdefault(ctr, []).append(val)
        ctrs = sorted({c for d in per.values() for c in d})
        lines.append("")
        lines.append("per dispatch, averaged over the kernel's dispatches; VALU/wave = "
                     "SQ_INSTS_VALU / SQ_WAVES (instructions per wave)")
        lines.append("%-40s %s %10s" % ("kernel", " ".join("%16s" % c[:16] for c in ctrs), "VALU/wave"))
        for k in sorted(per):
            avg = {c: sum(v) / len(v) for c, v in per[k].items()}
            vpw = (avg["SQ_INSTS_VALU"] / avg["SQ_WAVES"]
                   if avg.get("SQ_WAVES") and "SQ_INSTS_VALU" in avg else float("nan"))
            lines.append("%-40s %s %10.1f" % (k[:40], " ".join(
                "%16.4g" % avg.get(c, float("nan")) for c in ctrs), vpw))
    elif kind == "kt":
        lines.append("")
        lines.append("%-44s %7s %11s %13s %6s" % ("kernel", "calls", "avg_us", "total_us", "pct"))
        for db in dbs(db_dir):
            con = sqlite3.connect(db)
            for name, calls, total, avg, pct in con.execute(
                    "select name, total_calls, total_duration, average, percentage from top_kernels"):
                # the top_kernels view reports microseconds
                lines.append("%-44s %7d %11.2f %13.1f %6.1f" % (short(name)[:44], calls, avg, total,
                                                               pct))
    else:
        # kind == "pmc": db_dir = "<fetch dir>,<write dir>"
        fetch_dir, write_dir = db_dir.split(",")
        per = {}
        probe = {}
        for d, ctr in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
            for db in dbs(d):
                con = sqlite3.connect(db)
                for name, val in con.execute(
                        "select kernel_name, value from counters_collection where counter_name = ?",
                        (ctr,)):
                    per.setdefault(short(name), {}).setdefault(ctr, []).append(val)
                    # the 256 MiB probe copy runs as one or a few large blit
                    # dispatches; the other copies of a run (input uploads,
                    # slices of a pool) move at most 64 MiB each
                    if "copyBuffer" in name and val > 65536.0:
                        probe[ctr] = probe.get(ctr, 0.0) + val
        avg = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in per.items()}
        if "FETCH_SIZE" not in probe or "WRITE_SIZE" not in probe:
            raise SystemExit("no copy-probe dispatch in the counter runs (run bench.py --copy-probe)")
        exp_kib = COPY_PROBE_BYTES / 1024.0
        f_fetch = exp_kib / probe["FETCH_SIZE"]
        f_write = exp_kib / probe["WRITE_SIZE"]
        # a copy of N bytes reads and writes N bytes: counters that miss it by
        # more than 4x mean other large copies were taken for the probe
        if not (0.25 <= f_fetch <= 4.0 and 0.25 <= f_write <= 4.0):
            raise SystemExit("copy probe counters off by more than 4x (fetch scale %.3g, write "
                             "scale %.3g): was another large copy in the run?" % (f_fetch, f_write))
        enc = [k for k in avg if k.startswith("encode_kv_kernel")]
        enc_fetch = sum(avg[k]["FETCH_SIZE"] for k in enc) / len(enc) if enc else float("nan")
        enc_write = sum(avg[k]["WRITE_SIZE"] for k in enc) / len(enc) if enc else float("nan")
        traffic = (enc_fetch * f_fetch + enc_write * f_write) * 1024.0
        scaled = {k: (v.get("FETCH_SIZE", 0.0) * f_fetch + v.get("WRITE_SIZE", 0.0) * f_write) * 1024.0
                  for k, v in avg.items()}
        lines += [
            "encoder_source_sha1: %s" % source_sha1(ENCODER_SOURCE),
            "copy_probe: device copy of %d bytes; FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB in total" % (
                COPY_PROBE_BYTES, probe["FETCH_SIZE"], probe["WRITE_SIZE"]),
            "fetch_scale: %.4f" % f_fetch,
            "write_scale: %.4f" % f_write,
            "encode_fetch_kib_per_dispatch: %.1f" % enc_fetch,
            "encode_write_kib_per_dispatch: %.1f" % enc_write,
            "traffic_bytes_per_launch: %.0f" % traffic,
            "",
            "%-44s %16s %16s %18s" % ("kernel", "FETCH_SIZE KiB", "WRITE_SIZE KiB",
                                      "HBM bytes (scaled)"),
        ]
        for k in sorted(avg):
            lines.append("%-44s %16.1f %16.1f %18.0f" % (k[:44], avg[k].get("FETCH_SIZE", float("nan")),
                                                         avg[k].get("WRITE_SIZE", float("nan")), scaled[k]))
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COPY_CEILING_BYTES = 1 << 30


def copy_ceiling(dev, stream):
    """Measured device-copy ceiling after the timed region: a 1 GiB
    device-to-device copy, read + write bytes over the average time of 5
    copies."""
    import torch
    a = torch.ones(COPY_CEILING_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            b.copy_(a)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del a, b
    return {"GBps": 2 * COPY_CEILING_BYTES / (ms * 1e-3) / 1e9, "bytes_per_copy": 2 * COPY_CEILING_BYTES,
            "how": "torch device copy of 1 GiB (read + write bytes), average of 5 after the timed region"}


def algorithmic_bytes(w):
    """Per-launch algorithmic bytes of each kernel for workload w (one layer)."""
    per_tensor = w.batch * w.tokens * w.kv_heads * w.head_dim
    qo = w.batch * w.q_heads * w.head_dim * (2 + 4)
    return {
        "encode": 2 * per_tensor * 3.28125,             # K and V in one launch
        "decode_full": 2 * per_tensor * 1.28125 + qo,
        "decode_anchor": 2 * per_tensor * 0.78125 + qo,
        "elements_per_tensor": per_tensor,
    }


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(w, xk, xv, qb, pages, sm, nthreads, min_seconds):
    """One timing leg of the CPU oracle: encode K and V, then anchor and full
    dequantization of K and V, then brute-force attention for every query
    head over both reconstructions, repeated until min_seconds have passed.
    Rates use the GPU's algorithmic-byte accounting (dequantization counted
    with fp32 output)."""
    import oracle
    xk, xv = xk[:pages], xv[:pages]
    q = oracle.bf16_bits_to_float(qb).astype(np.float64)
    t = {"encode": 0.0, "dequant": 0.0, "attention": 0.0}
    passes = 0
    while passes == 0 or sum(t.values()) < min_seconds:
        t0 = time.perf_counter()
        ek, ev = oracle.encode(xk, nthreads), oracle.encode(xv, nthreads)
        t1 = time.perf_counter()
        ak, rk = oracle.split(ek["codes"])
        av, rv = oracle.split(ev["codes"])
        recon = {}
        for full in (False, True):
            recon[full] = (oracle.dequant(ak, rk if full else None, ek, nthreads),
                           oracle.dequant(av, rv if full else None, ev, nthreads))
        t2 = time.perf_counter()
        for full in (False, True):
            kh, vh = (r.reshape(1, -1, w.kv_heads, w.head_dim) for r in recon[full])
            oracle.attention(q[:1], kh, vh, sm, nthreads=nthreads)
        t3 = time.perf_counter()
        t["encode"] += t1 - t0
        t["dequant"] += t2 - t1
        t["attention"] += t3 - t2
        passes += 1
    elems = 2 * pages * 256 * w.kv_heads * w.head_dim          # K and V
    qo = w.q_heads * w.head_dim * 6
    nbytes = {"encode": elems * 3.28125,
              "dequant": elems * (1.28125 + 4.0) + elems * (0.78125 + 4.0),
              "attention": elems * (1.28125 + 0.78125) + 2 * qo}
    total = sum(t.values())
    leg = {"threads": nthreads, "pages": pages, "passes": passes, "seconds": total,
           "GBps": passes * sum(nbytes.values()) / total / 1e9}
    for k in t:
        leg[k] = {"s_per_pass": t[k] / passes, "GBps": passes * nbytes[k] / t[k] / 1e9,
                  "elements_per_s": passes * elems / t[k]}
    return leg


def cpu_baseline(w, xk, xv, qb, sm, pages_all=32, pages_one=4):
    """The CPU oracle, as it stands, on bounded samples of the same workload,
    on all host cores and on one core.  value: the all-cores rate of the
    whole step (encode, anchor and full reconstruction, attention) in the
    step's byte accounting."""
    import oracle
    nt = oracle.max_threads()
    allc = cpu_leg(w, xk, xv, qb, min(pages_all, w.pages), sm, nt, 8.0)
    one = cpu_leg(w, xk, xv, qb, min(pages_one, w.pages), sm, 1, 4.0)
    return {
        "value": allc["GBps"], "unit": "GB/s", "cores": nt, "kind": "oracle",
        "cpu_model": cpu_model(), "nproc": os.cpu_count(),
        "sample": "the first %d (all cores) and %d (one core) of the %d pages of one request of %s, "
                  "K and V: encode, anchor and full dequant, brute-force attention of all %d "
                  "query heads over both, repeated for at least 8 s / 4 s" % (
                      allc["pages"], one["pages"], w.pages, w.name, w.q_heads),
        "all_cores": allc, "one_core": one,
    }


def time_graph(calls, stream, reps=3):
    """Average time (ms) of one replay of a HIP graph of the given calls,
    measured with events on the launch stream over `reps` replays after one
    untimed replay."""
    import torch
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def tiny_leg(dev, stream, launches=64):
    """Latency of every call on the tiny workload (1 layer, 4 KV heads, 1024
    tokens, 32 query heads): graphs of `launches` back-to-back launches."""
    import torch
    from long_context_serving_amd import lynx, synth
    w = synth.WORKLOADS["tiny"]
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    k, v = to_dev(synth.kv_pages(w, 0, 0, 0)), to_dev(synth.kv_pages(w, 0, 1, 0))
    q = to_dev(synth.queries(w))
    pk = lynx.alloc_planes(w.pages, w.kv_heads, lynx.ROLE_KEY, dev)
    pv = lynx.alloc_planes(w.pages, w.kv_heads, lynx.ROLE_VALUE, dev)
    out = torch.empty((1, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    deq = torch.empty((w.pages, 256, w.kv_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = lynx.alloc_workspace(1, w.kv_heads, w.q_heads, w.pages, dev)
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    calls = {
        "encode_kv": lambda: lynx.quantize_kv_pages(k, v, out_k=pk, out_v=pv),
        "dequant_anchor_k": lambda: lynx.dequantize(pk, full=False, out=deq),
        "dequant_full_k": lambda: lynx.dequantize(pk, full=True, out=deq),
        "decode_anchor": lambda: lynx.decode_attention(q, pk, pv, w.pages, full=False, sm_scale=sm,
                                                       out=out, workspace=ws),
        "decode_full": lambda: lynx.decode_attention(q, pk, pv, w.pages, full=True, sm_scale=sm,
                                                     out=out, workspace=ws),
    }
    calls["encode_kv"]()
    res = {}
    for name, c in calls.items():
        res[name + "_us"] = time_graph([c] * launches, stream) / launches * 1e3
    return {"workload": w.name, "latency": res,
            "timing": "events around replays of a HIP graph of %d back-to-back launches of one call "
                      "(inputs cache-resident: a launch-bound shape)" % launches}


def qwen3_leg(dev, stream, reps=3):
    """Streaming encode of the Qwen3-235B-A22B-shaped request: 94 layers x
    K and V of 4 KV heads x 128K tokens (25.2 GB of bf16) into planes resident
    in HBM (16.2 GB).  The layers' pages sit in one K and one V page pool, as
    in a paged cache, so one lynx_quantize_kv_pages launch encodes every
    layer (pages are independent); the per-layer launches (94, one per
    layer's slice of the pools) are timed too.  Inputs are drawn on the
    device (synth.device_kv_pages), so the timed regions hold only encodes."""
    import torch
    from long_context_serving_amd import lynx, synth
    w = synth.WORKLOADS["qwen3_235b_128k"]
    log("bench: qwen3 shape: drawing %d layers of K and V on the device" % w.layers)
    t0 = time.perf_counter()
    P = w.pages
    shape = (w.layers * P, 256, w.kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.int16, device=dev)
    v = torch.empty(shape, dtype=torch.int16, device=dev)
    for layer in range(w.layers):
        k[layer * P:(layer + 1) * P] = synth.device_kv_pages(w, layer, 0, 0, device=dev)
        v[layer * P:(layer + 1) * P] = synth.device_kv_pages(w, layer, 1, 0, device=dev)
    pk = lynx.alloc_planes(w.layers * P, w.kv_heads, lynx.ROLE_KEY, dev)
    pv = lynx.alloc_planes(w.layers * P, w.kv_heads, lynx.ROLE_VALUE, dev)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    ms = time_graph([lambda: lynx.quantize_kv_pages(k, v, out_k=pk, out_v=pv)], stream, reps)
    layer_calls = [lambda l=l: lynx.quantize_kv_pages(
        k[l * P:(l + 1) * P], v[l * P:(l + 1) * P], out_k=lynx.planes_view(pk, l * P, P),
        out_v=lynx.planes_view(pv, l * P, P)) for l in range(w.layers)]
    ms_layers = time_graph(layer_calls, stream, reps)
    E = w.elements()
    nbytes = E * 3.28125
    del k, v, pk, pv, layer_calls
    torch.cuda.empty_cache()
    return {"workload": w.name, "layers": w.layers, "kv_heads": w.kv_heads, "tokens": w.tokens,
            "bf16_in_bytes": 2 * E, "encoded_bytes": int(E * 1.28125),
            "ms_all_layers": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "pct_of_hbm_peak": 100.0 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "kv_tokens_per_s": w.tokens * w.layers / (ms * 1e-3),
            "per_layer_launches": {"ms_all_layers": ms_layers,
                                   "GBps": nbytes / (ms_layers * 1e-3) / 1e9},
            "algorithmic_bytes": nbytes, "inputs_drawn_s": gen_s,
            "timing": "events around %d replays of a HIP graph of one encode launch over the %d "
                      "layers' pages (per_layer_launches: a graph of %d launches); inputs 25 GB: "
                      "no cache reuse" % (reps, w.layers, w.layers)}


def batched_leg(dev, stream, reps=5):
    """One decode step over the 64 x 16K batch (8 KV heads, 64 query heads):
    full and anchor-only fused attention over all requests, one launch each.
    K and V are drawn on the device and encoded (also timed) beforehand."""
    import torch
    from long_context_serving_amd import lynx, synth
    w = synth.WORKLOADS["batched64x16k"]
    log("bench: batched 64 x 16K: drawing and encoding the pool")
    P = w.pages
    shape = (w.batch * P, 256, w.kv_heads, w.head_dim)
    k = torch.empty(shape, dtype=torch.int16, device=dev)
    v = torch.empty(shape, dtype=torch.int16, device=dev)
    for r in range(w.batch):
        k[r * P:(r + 1) * P] = synth.device_kv_pages(w, 0, 0, r, device=dev)
        v[r * P:(r + 1) * P] = synth.device_kv_pages(w, 0, 1, r, device=dev)
    pk = lynx.alloc_planes(w.batch * P, w.kv_heads, lynx.ROLE_KEY, dev)
    pv = lynx.alloc_planes(w.batch * P, w.kv_heads, lynx.ROLE_VALUE, dev)
    q = torch.from_numpy(synth.queries(w).view(np.int16)).to(dev)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = lynx.alloc_workspace(w.batch, w.kv_heads, w.q_heads, P, dev)
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    enc_ms = time_graph([lambda: lynx.quantize_kv_pages(k, v, out_k=pk, out_v=pv)], stream, reps)
    del k, v
    torch.cuda.empty_cache()
    ab = algorithmic_bytes(w)
    res = {"workload": w.name, "batch": w.batch, "tokens": w.tokens, "kv_heads": w.kv_heads,
           "q_heads": w.q_heads,
           "encode": {"us_per_launch": enc_ms * 1e3, "GBps": ab["encode"] / (enc_ms * 1e-3) / 1e9}}
    for full, name in ((True, "decode_full"), (False, "decode_anchor")):
        ms = time_graph([lambda: lynx.decode_attention(q, pk, pv, P, full=full, sm_scale=sm,
                                                       out=out, workspace=ws)], stream, reps)
        res[name] = {"us_per_call": ms * 1e3, "GBps": ab[name] / (ms * 1e-3) / 1e9,
                     "decode_tokens_per_s": w.batch / (ms * 1e-3),
                     "kv_tokens_per_s": w.batch * w.tokens / (ms * 1e-3)}
    for key in ("encode", "decode_full", "decode_anchor"):
        res[key]["pct_of_hbm_peak"] = 100.0 * res[key]["GBps"] / HBM_PEAK_GBPS
    res["timing"] = "events around %d replays of a HIP graph of one launch (2.75 GB of planes: " \
                    "no cache reuse)" % reps
    del pk, pv
    torch.cuda.empty_cache()
    return res


def progressive_leg(dev):
    """One progressive-streaming run of the 32-layer 64K workload (planes in
    pinned host memory, anchors first): times to all drafts and all full
    attention, against the Lynx-INT8 layer-wise schedule; one warm-up run."""
    import torch
    from long_context_serving_amd import stream, synth
    w = synth.WORKLOADS["progressive32x64k"]
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    t0 = time.perf_counter()
    ps = stream.ProgressiveStream(stream.build_layers(w, device=dev), device=dev, sm_scale=sm)
    build_s = time.perf_counter() - t0
    ps.run_progressive()
    prog = ps.run_progressive()
    int8 = ps.run_layerwise_int8()
    ab, rb = ps.anchor_bytes(), ps.residual_bytes()
    res = {"workload": w.name, "layers": w.layers, "tokens": w.tokens,
           "all_drafts_ms": prog["all_drafts_ms"], "all_full_ms": prog["all_full_ms"],
           "first_draft_ms": prog["first_draft_layer_ms"],
           "draft_attention_ms": prog["draft_attention_ms"],
           "full_attention_ms": prog["full_attention_ms"],
           "h2d_anchor_GBps": ab / (prog["anchors_landed_ms"] * 1e-3) / 1e9,
           "h2d_residual_GBps": rb / ((prog["residuals_landed_ms"] - prog["anchors_landed_ms"]) * 1e-3) / 1e9,
           "lynx_int8_layerwise_first_layer_ms": int8["first_layer_ms"],
           "lynx_int8_layerwise_all_ms": int8["all_full_ms"],
           "build_s": build_s,
           "timing": "one run after one warm-up run; bench.py --progressive runs the full harness"}
    del ps
    torch.cuda.empty_cache()
    return res


def progressive_main(args):
    """Progressive plane streaming of the 32-layer 64K workload (anchor
    planes first, residual planes after; drafts start as anchors land).
    Prints one JSON line; link rates are PCIe host-to-device rates."""
    import statistics
    import torch
    from long_context_serving_amd import lynx, stream, synth

    w = synth.WORKLOADS["progressive32x64k"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    log("bench: encoding %d layers of %d tokens into pinned host planes" % (w.layers, w.tokens))
    t0 = time.perf_counter()
    ps = stream.ProgressiveStream(stream.build_layers(w, device=dev), device=dev, sm_scale=sm)
    log("bench: built in %.1f s" % (time.perf_counter() - t0))
    runs = max(1, args.stream_runs)
    prog = [ps.run_progressive() for _ in range(runs + 1)][1:]
    int8 = [ps.run_layerwise_int8() for _ in range(runs + 1)][1:]
    med = lambda rs, key: statistics.median(r[key] for r in rs)
    # bf16 comparison: the raw cache of one layer (K and V) copied once per layer
    bf16_layer = 2 * w.tokens * w.kv_heads * w.head_dim * 2
    hb = torch.empty(bf16_layer, dtype=torch.uint8, pin_memory=True)
    db = torch.empty(bf16_layer, dtype=torch.uint8, device=dev)
    bf16_ms = []
    for _ in range(runs + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(w.layers):
            db.copy_(hb, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        bf16_ms.append(e0.elapsed_time(e1))
    bf16_all = statistics.median(bf16_ms[1:])
    overlap = ps.draft_full_topk_overlap((1, 16, 64))
    ab, rb = ps.anchor_bytes(), ps.residual_bytes()
    # the same schedules on an emulated inter-server link (one run per rate)
    paced = {}
    for gbps in [float(x) for x in args.link_gbps.split(",") if x]:
        log("bench: emulated link at %g Gbps" % gbps)
        link = stream.PacedLink(gbps, ps.copy_stream)
        lp = ps.paced_progressive(link)
        li = ps.paced_layerwise_int8(link)
        lb = ps.paced_bf16(link, hb, db)
        paced["%g" % gbps] = {
            "lynx": lp, "lynx_int8_layerwise": li, "bf16_layerwise": lb,
            "first_draft_vs_int8_first_layer": li["first_full_layer_ms"] / lp["first_draft_ms"],
            "first_draft_vs_bf16_first_layer": lb["first_layer_landed_ms"] / lp["first_draft_ms"],
            "all_drafts_vs_int8_all_layers": li["all_full_ms"] / lp["all_drafts_ms"],
        }
    a_ms, r_ms = med(prog, "anchors_landed_ms"), med(prog, "residuals_landed_ms")
    result = {
        "metric": "progressive plane streaming: time to all drafts / all full attention (ms), 1xMI355X",
        "value": med(prog, "all_drafts_ms"),
        "unit": "ms",
        "higher_is_better": False,
        "n_gpus": 1,
        "runs": runs,
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": w.kv_heads,
                   "tokens": w.tokens, "q_heads": w.q_heads},
        "anchor_bytes": ab, "residual_bytes": rb, "bf16_bytes": bf16_layer * w.layers,
        "h2d_anchor_GBps": ab / (a_ms * 1e-3) / 1e9,
        "h2d_residual_GBps": rb / ((r_ms - a_ms) * 1e-3) / 1e9,
        "lynx": {k: med(prog, k) for k in prog[0]},
        "lynx_int8_layerwise": {k: med(int8, k) for k in int8[0]},
        "bf16_copy_all_layers_ms": bf16_all,
        "draft_vs_full_topk_overlap": {str(k): v for k, v in overlap.items()},
        "emulated_link": {"pacing": "pieces of 4 MiB released on the host at cumulative bytes / rate; "
                                    "times from an event at the link's start",
                          "by_gbps": paced},
    }
    print(json.dumps(result), flush=True)


def dequant_leg(w, sets, stream):
    """The standalone 4 + 4 dequantizers after the timed region: draft
    (anchor plane) and full (both planes) reconstruction of K and of V into
    fp32, one call per buffer set in turn (cache-cold), graph replays."""
    import torch
    from long_context_serving_amd import lynx
    elems = w.batch * w.tokens * w.kv_heads * w.head_dim
    out = torch.empty((w.pages * w.batch, 256, w.kv_heads, w.head_dim), dtype=torch.float32,
                      device=sets[0]["pk"].anchor.device)
    res = {}
    for tensor, key in (("K", "pk"), ("V", "pv")):
        for full in (False, True):
            calls = [lambda e=e: lynx.dequantize(e[key], full=full, out=out) for e in sets]
            for c in calls:
                c()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for c in calls:
                    c()
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(4):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (4 * len(sets))
            nbytes = elems * ((1.28125 if full else 0.78125) + 4.0)  # planes and scales in, fp32 out
            res["%s_%s" % (tensor, "full" if full else "draft")] = {
                "us_per_call": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9,
                "pct_of_hbm_peak": 100.0 * nbytes / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9)}
    return {"tensor": "one tensor of one buffer set per call, all %d sets in turn" % len(sets),
            "timing": "events around 4 replays of a HIP graph of one call per set, after the timed region",
            "by_call": res}


def cuts_leg(args, w, sets, stream, q, out_attn, ws, sm):
    """The b + (8 - b) cuts after the timed region: encoding one tensor
    straight into the two streams, re-cutting its 4 + 4 planes into them,
    the draft reconstruction from the anchor stream, the fused draft
    decode attention over the K and V anchor streams and the fused full
    decode attention over both streams, each cycled over the
    buffer sets (cache-cold)."""
    import torch
    from long_context_serving_amd import lynx
    elems = w.batch * w.tokens * w.kv_heads * w.head_dim
    scale_bytes = 0.28125  # fp32 page and chunk scales per element
    res = {}
    for b in (2, 3, 5, 6):
        streams = [lynx.split_planes(e["pk"], b) for e in sets]
        outs = torch.empty((w.pages * w.batch, 256, w.kv_heads, w.head_dim), dtype=torch.float32,
                           device=sets[0]["pk"].anchor.device)
        split_calls = [lambda e=e: lynx.split_planes(e["pk"], b) for e in sets]
        enc_out = lynx.alloc_cut_planes(w.pages * w.batch, w.kv_heads, lynx.ROLE_KEY, b,
                                        sets[0]["pk"].anchor.device)
        enc_calls = [lambda e=e: lynx.quantize_pages_split(e["k"], lynx.ROLE_KEY, b, out=enc_out)
                     for e in sets]
        draft_calls = [lambda e=e, st=st: lynx.dequantize_split(st[0], None, b, e["pk"], out=outs)
                       for e, st in zip(sets, streams)]
        cut_k = [lynx.cut_planes(e["pk"], b) for e in sets]
        cut_v = [lynx.cut_planes(e["pv"], b) for e in sets]
        attn_calls = [lambda ck=ck, cv=cv: lynx.decode_attention_split(
            q, ck, cv, b, w.pages, full=False, sm_scale=sm, out=out_attn, workspace=ws)
            for ck, cv in zip(cut_k, cut_v)]
        full_calls = [lambda ck=ck, cv=cv: lynx.decode_attention_split(
            q, ck, cv, b, w.pages, full=True, sm_scale=sm, out=out_attn, workspace=ws)
            for ck, cv in zip(cut_k, cut_v)]
        times = []
        for calls in (split_calls, draft_calls, attn_calls, enc_calls, full_calls):
            for c in calls:
                c()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for c in calls:
                    c()
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                for _ in range(4):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / (4 * len(sets)))  # one call per set per replay
        split_bytes = elems * 2.0                    # 4 + 4 planes in, both streams out
        draft_bytes = elems * (b / 8.0 + scale_bytes + 4.0)
        attn_bytes = 2 * elems * (b / 8.0 + scale_bytes)  # K and V anchor streams and scales
        full_bytes = 2 * elems * (1.0 + scale_bytes)      # both streams of K and V and scales
        res["%d+%d" % (b, 8 - b)] = {
            "encode_direct_us": times[3] * 1e3,
            "encode_direct_GBps": elems * 3.28125 / (times[3] * 1e-3) / 1e9,
            "draft_attention_us": times[2] * 1e3,
            "draft_attention_GBps": attn_bytes / (times[2] * 1e-3) / 1e9,
            "full_attention_us": times[4] * 1e3,
            "full_attention_GBps": full_bytes / (times[4] * 1e-3) / 1e9,
            "split_us": times[0] * 1e3, "split_GBps": split_bytes / (times[0] * 1e-3) / 1e9,
            "draft_dequant_us": times[1] * 1e3,
            "draft_dequant_GBps": draft_bytes / (times[1] * 1e-3) / 1e9,
            "anchor_stream_bytes_per_elem": b / 8.0}
    return {"tensor": "K of one buffer set per call, all %d sets in turn" % len(sets),
            "timing": "events around 4 replays of a HIP graph of one call per set, after the "
                      "timed region",
            "by_cut": res}


def verify_leg(args, w, sets, dev, sm, stream, tq):
    """Verify pass after the timed region: the newest tq tokens of the
    request (its speculative tokens) attend to the full planes of every
    buffer set in turn (cache-cold) plus a bf16 tail of tq + 36 tokens."""
    import torch
    from long_context_serving_amd import lynx, synth
    tail_len = tq + 36
    rng = np.random.default_rng(4242)
    tail = lambda: torch.from_numpy(synth.float_to_bf16_bits(
        rng.laplace(0, 1, (w.batch, lynx.TAIL_TOKENS, w.kv_heads, w.head_dim)).astype(np.float32))
        .view(np.int16)).to(dev)
    tk, tv = tail(), tail()
    tl = torch.full((w.batch,), tail_len, dtype=torch.int32, device=dev)
    qv = torch.from_numpy(synth.float_to_bf16_bits(
        rng.laplace(0, 1, (w.batch, tq, w.q_heads, w.head_dim)).astype(np.float32)).view(np.int16)).to(dev)
    out = torch.empty((w.batch, tq, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = lynx.alloc_verify_workspace(w.batch, tq, w.kv_heads, w.q_heads, w.pages, dev)
    calls = [lambda e=e: lynx.verify_attention(qv, e["pk"], e["pv"], w.pages, tk, tv, tl, full=True,
                                               sm_scale=sm, out=out, workspace=ws) for e in sets]
    for c in calls:
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.verify_reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (args.verify_reps * len(calls))
    ctx = w.tokens + tail_len - tq  # cached tokens before the speculative ones
    # score and value products of every query row with every visible token
    flops = 4.0 * w.batch * w.q_heads * w.head_dim * sum(ctx + i + 1 for i in range(tq))
    plane_bytes = algorithmic_bytes(w)["decode_full"]
    return {"tq": tq, "tail_tokens": tail_len, "us_per_call": ms * 1e3,
            "speculative_tokens_per_s": w.batch * tq / (ms * 1e-3),
            "algorithmic_TFLOPs": flops / (ms * 1e-3) / 1e12,
            "frac_of_fp16_mfma_peak": flops / (ms * 1e-3) / 2.5e15,
            "plane_GBps": plane_bytes / (ms * 1e-3) / 1e9,
            "timing": "events around graph replays of one call per buffer set, after the timed region"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="ctx32k")
    ap.add_argument("--sets", type=int, default=8, help="distinct buffer sets cycled per step")
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the other workloads (tiny latency, 94-layer encode, 64 x 16K batch, "
                         "progressive streaming) after the timed region")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one 256 MiB device copy (counter calibration)")
    ap.add_argument("--progressive", action="store_true",
                    help="run the progressive plane-streaming harness (32 layers x 64K) instead")
    ap.add_argument("--stream-runs", type=int, default=3)
    ap.add_argument("--link-gbps", default="10,25,50",
                    help="emulated link rates for the progressive timeline (empty: none)")
    ap.add_argument("--no-verify", dest="verify", action="store_false",
                    help="skip the verify-pass measurements (speculative tokens over the planes)")
    ap.add_argument("--no-cuts", dest="cuts", action="store_false",
                    help="skip the measurement of the other code cuts and of the standalone dequantizers")
    ap.add_argument("--verify-only", action="store_true",
                    help="encode the buffer sets, then time the verify pass alone")
    ap.add_argument("--verify-tq", type=int, default=64,
                    help="speculative tokens of the main verify measurement")
    ap.add_argument("--verify-short-tq", type=int, default=5,
                    help="speculative tokens of the short verify measurement (0: skip it)")
    ap.add_argument("--verify-reps", type=int, default=4)
    ap.add_argument("--config-only", choices=("tiny", "qwen3_235b_128k", "batched64x16k",
                                              "progressive32x64k"),
                    help="run only that workload's leg and print its JSON (for profiling)")
    ap.add_argument("--summarize", nargs=4, metavar=("KIND", "DB_DIR", "OUT", "COMMAND"),
                    help="write a text summary of rocprofv3 output (KIND kt or pmc; for pmc "
                         "DB_DIR is '<FETCH_SIZE dir>,<WRITE_SIZE dir>') and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.config_only and args.gpus == 1 and world == 1:
        import torch
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        stream = torch.cuda.Stream()
        leg = {"tiny": lambda: tiny_leg(dev, stream), "qwen3_235b_128k": lambda: qwen3_leg(dev, stream),
               "batched64x16k": lambda: batched_leg(dev, stream),
               "progressive32x64k": lambda: progressive_leg(dev)}[args.config_only]
        res = leg()
        if args.copy_probe:
            a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
            torch.empty_like(a).copy_(a)
            torch.cuda.synchronize()
        print(json.dumps(res), flush=True)
        return
    if args.progressive and args.gpus == 1 and world == 1:
        progressive_main(args)
        return
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on exactly one GPU; --gpus %d (WORLD_SIZE=%d) is not "
              "supported (the library has no multi-GPU path)." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_serving_amd import lynx, synth

    w = synth.WORKLOADS[args.workload]
    if w.layers != 1 or w.batch != 1 or not w.q_heads:
        raise SystemExit("bench workload must be a single-request, single-layer decode workload "
                         "(the batched and multi-layer configurations are parity-test cases)")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    S = max(2, args.sets)
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    ab = algorithmic_bytes(w)

    log("bench: generating %d buffer sets of workload %s" % (S, w.name))
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    sets = []
    xk0 = xv0 = None
    for s in range(S):
        xk = synth.kv_pages(w, 0, 0, s)
        xv = synth.kv_pages(w, 0, 1, s)
        if s == 0:
            xk0, xv0 = xk, xv
        sets.append({
            "k": to_dev(xk), "v": to_dev(xv),
            "pk": lynx.alloc_planes(w.pages, w.kv_heads, lynx.ROLE_KEY, dev),
            "pv": lynx.alloc_planes(w.pages, w.kv_heads, lynx.ROLE_VALUE, dev),
        })
    qb = synth.queries(w)
    q = to_dev(qb)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = lynx.alloc_workspace(w.batch, w.kv_heads, w.q_heads, w.pages, dev)
    # A step is one pass of the hot path over one buffer set: encode K and V
    # (one launch), anchor-only decode, full decode.  The timed loop runs the steps in
    # rounds of S: one HIP graph encodes all S sets back to back, a second
    # runs the anchor decode of all S sets, a third the full decode.  Events
    # recorded on the launch stream between the three graphs give each
    # kernel's average time inside the timed region (the graph boundaries
    # are shared by S back-to-back launches).  Set j is decoded after
    # the other sets were encoded, so its planes are no longer cached.
    enc_calls = []
    anc_calls = []
    full_calls = []
    for j in range(S):
        e = sets[j]
        enc_calls.append(lambda e=e: lynx.quantize_kv_pages(e["k"], e["v"], out_k=e["pk"],
                                                            out_v=e["pv"]))
        anc_calls.append(lambda e=e: lynx.decode_attention(q, e["pk"], e["pv"], w.pages, full=False,
                                                           sm_scale=sm, out=out, workspace=ws))
        full_calls.append(lambda e=e: lynx.decode_attention(q, e["pk"], e["pv"], w.pages, full=True,
                                                            sm_scale=sm, out=out, workspace=ws))
    stream = torch.cuda.Stream()
    if args.verify_only:
        # only the verify pass (its kernels share names with the decode ones)
        for call in enc_calls:
            call()
        torch.cuda.synchronize()
        print(json.dumps({"workload": w.name,
                          "verify": verify_leg(args, w, sets, dev, sm, stream, args.verify_tq)}),
              flush=True)
        return
    for call in enc_calls + anc_calls + full_calls:  # eager pass
        call()
    torch.cuda.synchronize()

    def capture(calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for call in calls:
                call()
        return g

    # exactly K steps: full rounds of all S sets, then one round of the first
    # K mod S sets (graphs of their own)
    K = max(1, args.steps)
    full_rounds, rem = divmod(K, S)
    phases = [capture(enc_calls), capture(anc_calls), capture(full_calls)]
    tail_phases = ([capture(enc_calls[:rem]), capture(anc_calls[:rem]), capture(full_calls[:rem])]
                   if rem else None)
    torch.cuda.synchronize()
    plan = [phases] * full_rounds + ([tail_phases] if rem else [])

    def run_rounds(rounds, events=None):
        with torch.cuda.stream(stream):
            for r, graphs in enumerate(rounds):
                for p, g in enumerate(graphs):
                    if events is not None:
                        events[r][p].record(stream)
                    g.replay()
                if events is not None:
                    events[r][3].record(stream)

    run_rounds([phases] * max(1, -(-args.warmup // S)))
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(len(plan))]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    run_rounds(plan, evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = evs[0][0].elapsed_time(evs[-1][3]) / K
    phase_ms = [sum(evs[r][p].elapsed_time(evs[r][p + 1]) for r in range(len(plan))) for p in range(3)]
    per_call_ms = {"encode": phase_ms[0] / K, "decode_anchor": phase_ms[1] / K,
                   "decode_full": phase_ms[2] / K}

    verify = verify_leg(args, w, sets, dev, sm, stream, args.verify_tq) if args.verify else None
    verify_short = (verify_leg(args, w, sets, dev, sm, stream, args.verify_short_tq)
                    if args.verify and args.verify_short_tq > 0 else None)
    cuts = cuts_leg(args, w, sets, stream, q, out, ws, sm) if args.cuts else None
    dequant = dequant_leg(w, sets, stream) if args.cuts else None

    if args.copy_probe:
        a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    # counter runs (--copy-probe) leave the probe as the only large copy
    ceiling = None if args.copy_probe else copy_ceiling(dev, stream)

    enc_avg = per_call_ms["encode"]
    anc_avg = per_call_ms["decode_anchor"]
    full_avg = per_call_ms["decode_full"]
    gbps = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    step_bytes = ab["encode"] + ab["decode_full"] + ab["decode_anchor"]
    kernels = {
        "encode": {"us_per_launch": enc_avg * 1e3, "GBps": gbps(ab["encode"], enc_avg)},
        "decode_anchor": {"us_per_call": anc_avg * 1e3, "GBps": gbps(ab["decode_anchor"], anc_avg)},
        "decode_full": {"us_per_call": full_avg * 1e3, "GBps": gbps(ab["decode_full"], full_avg)},
    }
    for k in kernels.values():
        k["pct_of_hbm_peak"] = 100.0 * k["GBps"] / HBM_PEAK_GBPS
        if ceiling is not None:
            k["pct_of_copy_ceiling"] = 100.0 * k["GBps"] / ceiling["GBps"]

    result = {
        "metric": METRIC,
        "value": gbps(step_bytes, step_ms),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "input_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "tokens": w.tokens, "batch": w.batch,
                   "q_heads": w.q_heads, "buffer_sets": S},
        "pct_of_hbm_peak": 100.0 * gbps(step_bytes, step_ms) / HBM_PEAK_GBPS,
        "copy_ceiling": ceiling,
        "kernels": kernels,
        "tokens_per_s": {"encode_kv_tokens": w.tokens * w.batch / (enc_avg * 1e-3),
                         "decode_full_kv_tokens": w.tokens * w.batch / (full_avg * 1e-3),
                         "decode_anchor_kv_tokens": w.tokens * w.batch / (anc_avg * 1e-3)},
        "roofline": {"bound": "hbm", "kernel": "encode_kv_kernel",
                     "timing": "events on the launch stream around graphs of back-to-back launches, timed region",
                     "achieved": gbps(ab["encode"], enc_avg), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": gbps(ab["encode"], enc_avg) / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(), "algorithmic_bytes": ab["encode"]},
        "wall_s_timed": wall,
    }
    if verify is not None:
        result["verify"] = verify
    if verify_short is not None:
        result["verify_short"] = verify_short
    if cuts is not None:
        result["cuts"] = cuts
    if dequant is not None:
        result["dequant"] = dequant
    if args.configs:
        del sets, enc_calls, anc_calls, full_calls, phases, tail_phases, plan
        torch.cuda.empty_cache()
        configs = {}
        log("bench: tiny latencies")
        configs["tiny"] = tiny_leg(dev, stream)
        log("bench: 94-layer streaming encode")
        configs["qwen3_235b_128k"] = qwen3_leg(dev, stream)
        log("bench: 64 x 16K batched decode")
        configs["batched64x16k"] = batched_leg(dev, stream)
        log("bench: progressive streaming run")
        configs["progressive32x64k"] = progressive_leg(dev)
        result["configs"] = configs
        for key, leg in (("qwen3_235b_128k_encode", configs["qwen3_235b_128k"]),):
            kernels[key] = {"ms_per_pass": leg["ms_all_layers"], "GBps": leg["GBps"],
                            "pct_of_hbm_peak": leg["pct_of_hbm_peak"]}
        for name in ("decode_full", "decode_anchor", "encode"):
            b = configs["batched64x16k"][name]
            kernels["batched64x16k_" + name] = {"us_per_call": b.get("us_per_call", b.get("us_per_launch")),
                                                "GBps": b["GBps"], "pct_of_hbm_peak": b["pct_of_hbm_peak"]}
    if args.cpu:
        log("bench: CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, xk0, xv0, qb, sm)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
