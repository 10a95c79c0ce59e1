#!/usr/bin/env python3
"""Benchmark of the colibri quantized-matmul hot path on one MI355X.

A step is one decode MoE block (S=1) on fresh routing: 8 of 256 experts, each
gate/up 2048x6144 and down 6144x2048 in grouped int4 (fmt 4, gs 64, f32 scales
U[0.001,0.02]), hidden N(0,1) of 6144, softmax routing weights -- route,
dual gate/up + SiLU, down + weighted combine, all inside coli_moe_block.  The
routing changes every step (64 precomputed uniform draws), so the 170 MB the
block touches does not sit in the 256 MB last-level cache.

value = algorithmic HBM bytes per block / block time (GB/s), the K timed
blocks captured in one HIP graph and replayed once (one submission, as the
pages submit a layer's block in one command buffer); the same K blocks
launched one by one are reported beside it (extra.block_us_eager).  Per-kernel
durations come from one more pass of K blocks with HIP events the library
records on the launch stream around each kernel.  Side measurements ("extra")
cover the single fmt-4 GEMV, the 6144x6144 format sweep, the ceilings a
streaming read and a matrix-core loop reach on this part, the S=544 prefill
GEMM and MoE block, and the 75-layer decode stream.

Prints ONE JSON line.  N > 1 GPUs is not supported (one-GPU build).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fmt4 GEMV+MoE-block HBM GB/s (S=1) and prefill TFLOP/s (S=544), %roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

E, D, F, K, GS = 256, 6144, 2048, 8, 64


def qbytes(fmt, O, I, gs):
    rb = {1: I, 2: (I + 1) // 2, 4: (I + 1) // 2, 3: (I + 3) // 4}[fmt]
    ng = -(-I // gs) if fmt == 4 else 1
    return O * rb + O * ng * 4


def src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = ["bit_gemv_coli_amd/csrc/mgemv.hip", "bit_gemv_coli_amd/csrc/common.h"]


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_decode_moe_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != src_hash(KERNEL_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the side measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the S=544 prefill measurements (dense GEMM and MoE block); prints "
                         "their JSON (for profiling those kernels)")
    ap.add_argument("--gemv-only", action="store_true",
                    help="only the GEMV measurements (1024x2048 latency and ring, 6144x6144 format "
                         "sweep one and eight matrices per launch)")
    ap.add_argument("--layer-stream-only", action="store_true",
                    help="only the 75-layer decode stream (grouped and one launch per projection)")
    ap.add_argument("--layer-decode-only", action="store_true",
                    help="only the 75 whole decode layers (attention + expert half) and the "
                         "attention alone")
    ap.add_argument("--router-only", action="store_true",
                    help="only the router and top-K timings (S=1 and S=544); prints their JSON "
                         "(for profiling those kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy 5 times (reference for the "
                         "HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return

    import bit_gemv_coli_amd as coli
    import synthdata as sd

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.prefill_only:
        print(json.dumps(prefill_measurements(coli, sd, np, torch, log, make_timed(torch))), flush=True)
        return
    if args.gemv_only:
        print(json.dumps(gemv_measurements(coli, sd, np, torch, log)), flush=True)
        return
    if args.layer_stream_only:
        print(json.dumps(layer_stream(coli, sd, np, torch, log)), flush=True)
        return
    if args.layer_decode_only:
        out = full_layer_stream(coli, sd, np, torch, log)
        out.update(attention_prefill(coli, sd, np, torch, log))
        print(json.dumps(out), flush=True)
        return
    if args.router_only:
        print(json.dumps(router_measurements(coli, sd, np, torch, log, make_timed(torch))), flush=True)
        return

    # ---- inputs ----------------------------------------------------------
    log("drawing the 256-expert fmt-4 pool on the device")
    gq, gsc = sd.pool_on_device(100, 4, E, F, D, GS)
    uq, usc = sd.pool_on_device(101, 4, E, F, D, GS)
    dq, dsc = sd.pool_on_device(102, 4, E, D, F, GS)
    tg = coli.QTensor(4, gq, gsc, F, D, GS)
    tu = coli.QTensor(4, uq, usc, F, D, GS)
    td = coli.QTensor(4, dq, dsc, D, F, GS)
    for t in (tg, tu, td):  # upload-time repack for the matrix-core decode kernels
        t.pack()
    r = sd.rng(0)
    x = sd.gen_x(r, 1, D)
    NR = 64
    routes = [sd.gen_routing_uniform(r, 1, K, E) for _ in range(NR)]
    ids_d = torch.from_numpy(np.stack([a for a, _ in routes])).to(dev)      # [NR][1][K]
    w_d = torch.from_numpy(np.stack([b for _, b in routes])).to(dev)
    x_d = torch.from_numpy(x).to(dev)
    out = torch.empty((1, D), device=dev)
    wsb = coli.coli_moe_workspace_bytes(E, 1, K, F, D, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    expert_bytes = qbytes(4, F, D, GS) * 2 + qbytes(4, D, F, GS)
    block_bytes = K * expert_bytes + x.nbytes + out.numel() * 4 + K * 8
    gateup_bytes = K * 2 * qbytes(4, F, D, GS) + x.nbytes + K * F * 4

    def step(i, st=None):
        rc = coli.coli_moe_block(tg, tu, td, x_d, 1, ids_d[i % NR], w_d[i % NR], K, None, None,
                                 None, out, ws, wsb, stream if st is None else st)
        if rc != coli.COLI_OK:
            coli.check(rc, "coli_moe_block")

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed steps as one submission: the K blocks (each with its own
    # routing) captured in one HIP graph and replayed once -- every kernel of
    # every block runs; the host's launch calls are out of the timed region
    log(f"capturing {args.steps} steps in one graph")
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(0, side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cst = torch.cuda.current_stream()
        for i in range(args.steps):
            step(args.warmup + i, cst)
    graph.replay()  # untimed first replay
    torch.cuda.synchronize()

    log(f"timed {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    value = block_bytes / (ms * 1e-3) / 1e9
    del graph

    # the same steps launched one by one on the stream (eager), for reference
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / args.steps

    # the same steps again with HIP events recorded by the library around
    # every kernel launch (on the launch stream): per-kernel durations
    log(f"profiled {args.steps} steps")
    coli.coli_prof_reset()
    coli.coli_prof_enable(True)
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    coli.coli_prof_enable(False)
    kern = {}
    for tag in coli.coli_prof_tags():
        n, tot = coli.coli_prof_read(tag)
        if n > 0:
            kern[tag] = {"launches": n, "avg_us": tot / n * 1e3}
    log(f"block {ms * 1e3:.2f} us  {value:.1f} GB/s  kernels {kern}")

    dom = "moe_gateup_decode"
    dom_us = kern.get(dom, {}).get("avg_us")
    achieved = gateup_bytes / (dom_us * 1e-6) / 1e9 if dom_us else None
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS if achieved else None,
                "traffic": traffic_from_profiles(dom),
                "algorithmic_bytes_per_launch": gateup_bytes, "avg_launch_us": dom_us,
                # the whole block (both launches and the gap between them), for
                # reading beside the dominant kernel's fraction
                "block_GBps": value, "block_frac": value / HBM_PEAK_GBS}

    # ---- side measurements --------------------------------------------------
    extra = {"block_us": ms * 1e3, "block_us_eager": ms_eager * 1e3,
             "block_GBps_eager": block_bytes / (ms_eager * 1e-3) / 1e9, "kernels": kern,
             "wall_s_timed": wall}
    if not args.no_extra:
        # the same blocks in two submissions (begin: resident slots; end: the
        # late ones), half of the 8 slots late
        late = torch.from_numpy((np.arange(K) % 2).astype(np.int32).reshape(1, K)).to(dev)
        wsb2 = coli.coli_moe_block_two_phase_workspace_bytes(E, 1, K, F, D, 0)
        ws2 = torch.empty(wsb2, dtype=torch.uint8, device=dev)

        def step2(i):
            j = i % NR
            coli.check(coli.coli_moe_block_begin(tg, tu, td, x_d, 1, ids_d[j], w_d[j], K, late, None,
                                                 None, None, out, ws2, wsb2, stream), "begin")
            coli.check(coli.coli_moe_block_end(tg, tu, td, x_d, 1, w_d[j], K, 0, out, ws2, wsb2,
                                               stream), "end")
        us2 = make_timed(torch)(step2, args.steps)
        extra["two_phase_block_us"] = {"begin_plus_end": us2, "one_submission": ms * 1e3,
                                       "late_slots": K // 2}
        log(f"two-phase block (4 of 8 slots late): {us2:.2f} us against {ms * 1e3:.2f} us in one")
        extra["two_phase_overlapped_upload"] = two_phase_upload(
            coli, np, torch, tg, tu, td, x_d, ids_d[0], w_d[0], late, out, ws2, wsb2, stream, log)
        del ws2
        extra.update(side_measurements(coli, sd, np, torch, log))

    # ---- CPU oracle baseline -------------------------------------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(coli, sd, np, torch, gq, gsc, uq, usc, dq, dsc, x, routes,
                           block_bytes, args.cpu_seconds, log)
        if not args.no_extra:
            extra["oracle_timings"] = oracle_timings(sd, np, log)

    if not args.no_extra:
        extra["summary"] = summary(extra, value, roofline)

    res = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode MoE block S=1: 8 of 256 experts (uniform, fresh routing "
                               "each step), gate/up 2048x6144 + down 6144x2048, fmt4 gs64",
                   "E": E, "D": D, "F": F, "K": K, "gs": GS, "S": 1,
                   "bytes_per_step": block_bytes},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(res), flush=True)


def two_phase_upload(coli, np, torch, tg, tu, td, x_d, ids, w, late, out, ws2, wsb2, stream, log,
                     reps=10):
    """The two-phase block as the pages use it: the 4 late experts' packed
    weights (what the decode kernels read; 3 matrices each) arrive from
    pinned host memory.  Serial: the copies, then begin and end.  Overlapped:
    begin on the main stream while a second stream copies, end after an
    event.  Reports both, the copies alone, and what the overlap hides."""
    dev = x_d.device
    ids_h = ids.cpu().numpy().reshape(-1)
    late_e = sorted(set(int(ids_h[k]) for k in range(len(ids_h)) if k % 2 == 1))
    dev_sl = []
    for T in (tg, tu, td):
        d = T.desc
        for e in late_e:
            dev_sl.append(T.packed[e * d.pk_stride:(e + 1) * d.pk_stride])
    host = [torch.empty(t.shape, dtype=t.dtype, pin_memory=True) for t in dev_sl]
    for h_, d_ in zip(host, dev_sl):
        h_.copy_(d_)
    nbytes = sum(t.numel() for t in host)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    def copies(st):
        with torch.cuda.stream(st):
            for h_, d_ in zip(host, dev_sl):
                d_.copy_(h_, non_blocking=True)

    def begin():
        coli.check(coli.coli_moe_block_begin(tg, tu, td, x_d, 1, ids, w, K, late, None, None, None,
                                             out, ws2, wsb2, stream), "begin")

    def end():
        coli.check(coli.coli_moe_block_end(tg, tu, td, x_d, 1, w, K, 0, out, ws2, wsb2, stream),
                   "end")

    def serial():
        copies(stream)
        begin()
        end()

    def overlapped():
        side.wait_stream(stream)
        begin()
        copies(side)
        ev = torch.cuda.Event()
        ev.record(side)
        stream.wait_event(ev)
        end()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps * 1e6
    res = {"late_experts": len(late_e), "upload_bytes": nbytes,
           "copies_alone_us": timed(lambda: copies(stream)),
           "serial_us": timed(serial), "overlapped_us": timed(overlapped)}
    res["hidden_us"] = res["serial_us"] - res["overlapped_us"]
    log(f"two-phase with uploads ({nbytes / 1e6:.0f} MB from pinned host memory): serial "
        f"{res['serial_us']:.0f} us, overlapped {res['overlapped_us']:.0f} us, copies alone "
        f"{res['copies_alone_us']:.0f} us")
    return res


def summary(e, value, roofline):
    """One line per workload: the figure and its fraction of the bound that
    applies (HBM 8 TB/s for decode, max(flops/bf16 peak, bytes/HBM) for the
    prefill MoE block, bf16 peak for the dense prefill GEMM)."""
    out = {"decode_moe_block_S1": {"GBps": value, "frac_hbm": value / HBM_PEAK_GBS},
           "decode_moe_gateup_kernel": {"GBps": roofline.get("achieved"), "frac_hbm": roofline.get("frac")}}
    st = e.get("gemv_6144x6144_ring_stacked", {})
    for k in ("fmt4_g64_S1", "fmt4_g64_S4", "fmt4_g128_S1", "fmt2_S1", "fmt1_S1", "fmt3_S1"):
        if k in st:
            out[f"gemv_6144x6144_{k}_x8_per_launch"] = {"GBps": st[k]["GBps"], "frac_hbm": st[k]["frac_hbm"]}
    one = e.get("gemv_6144x6144_ring", {}).get("fmt4_g64_S1")
    if one:
        out["gemv_6144x6144_fmt4_g64_S1_one_per_launch"] = {"GBps": one["GBps"], "frac_hbm": one["frac_hbm"]}
    for k in ("layer_decode_75", "mla_decode_75"):
        if k in e:
            out[k] = {"us_per_layer": e[k]["us_per_layer"], "frac_hbm": e[k]["frac_hbm"]}
    ls = e.get("layer_stream_75")
    if ls:
        out["layer_stream_75"] = {"us_per_layer": ls["us_per_layer"], "frac_hbm": ls["frac_hbm"]}
    pm = e.get("prefill_moe_544_zipf1.1_g128")
    if pm:
        out["prefill_moe_544_zipf1.1"] = {"us": pm["us"], "TFLOPs": pm["TFLOPs"], "frac_roofline": pm["frac_roofline"]}
    pd = e.get("prefill_dense_544x6144x6144_g128")
    if pd:
        out["prefill_dense_544x6144x6144"] = {"TFLOPs": pd["TFLOPs"], "frac_bf16_peak": pd["frac_bf16_peak"]}
    ap = e.get("mla_prefill_544")
    if ap:
        out["mla_prefill_544"] = {"us_per_layer": ap["us_per_layer"], "TFLOPs": ap["TFLOPs"]}
    return out


def make_timed(torch):
    """timed(fn, n): 3 untimed calls fn(i), then the mean us of n calls, by
    events on the current stream."""
    st = torch.cuda.current_stream()

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a.record(st)
        for i in range(n):
            fn(i)
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3  # us
    return timed


def side_measurements(coli, sd, np, torch, log):
    """The GEMV measurements, the ceiling probes, the router, the S=544
    prefill and the 75-layer stream."""
    timed = make_timed(torch)
    out = gemv_measurements(coli, sd, np, torch, log)
    out.update(ceiling_probes(coli, torch, log))
    out.update(router_measurements(coli, sd, np, torch, log, timed))
    out.update(prefill_measurements(coli, sd, np, torch, log, timed))
    out.update(layer_stream(coli, sd, np, torch, log))
    out.update(full_layer_stream(coli, sd, np, torch, log))
    out.update(attention_prefill(coli, sd, np, torch, log))
    return out


def gemv_measurements(coli, sd, np, torch, log):
    """Single fmt-4 GEMV (1024x2048, latency and a >= 1 GiB ring) and the
    6144x6144 format sweep (ring of distinct copies >= 1 GiB so each launch
    streams from HBM), one and eight matrices per launch."""
    out = {}
    dev = "cuda"
    st = torch.cuda.current_stream()
    timed = make_timed(torch)

    # config 1: one matrix, back-to-back launches (cache-resident; latency)
    q, s = sd.pool_on_device(7, 4, 1, 1024, 2048, 64)
    T = coli.QTensor(4, q, s, 1024, 2048, 64)
    T.pack()
    x = torch.randn((1, 2048), device=dev)
    y = torch.empty((1, 1024), device=dev)
    us = timed(lambda i: coli.coli_qmatmul(T, x, y, 1, st), 200)
    out["gemv_1024x2048_g64_us"] = us
    log(f"gemv 1024x2048 g64: {us:.2f} us/call")
    del T, q, s
    # the same shape from a >= 1 GiB ring of distinct copies (HBM, not the
    # last-level cache): one matrix per launch, and stacks of 64 per launch
    mb1 = qbytes(4, 1024, 2048, 64)
    ncopy = -(-(1 << 30) // mb1) // 64 * 64 + 64
    q, s = sd.pool_on_device(8, 4, ncopy, 1024, 2048, 64)
    Ts = [coli.QTensor(4, q[c], s[c], 1024, 2048, 64, n=1) for c in range(ncopy)]
    for t in Ts:
        t.pack()
    us1 = timed(lambda i: coli.coli_qmatmul(Ts[i % ncopy], x, y, 1, st), 2 * ncopy)
    del Ts
    NST = 64
    Tst = [coli.QTensor(4, q[c * NST:(c + 1) * NST], s[c * NST:(c + 1) * NST], 1024, 2048, 64, n=NST)
           for c in range(ncopy // NST)]
    for t in Tst:
        t.pack()
    ys = torch.empty((NST, 1, 1024), device=dev)
    usn = timed(lambda i: coli.coli_qmatmul(Tst[i % len(Tst)], x, ys, 1, st), 4 * len(Tst))
    per = mb1 + 2048 * 4 + 1024 * 4
    out["gemv_1024x2048_g64_ring"] = {
        "copies": ncopy, "one_per_launch": {"us": us1, "GBps": per / (us1 * 1e-6) / 1e9},
        f"{NST}_per_launch": {"us_per_matrix": usn / NST, "GBps": NST * per / (usn * 1e-6) / 1e9,
                              "frac_hbm": NST * per / (usn * 1e-6) / 1e9 / HBM_PEAK_GBS}}
    log(f"gemv 1024x2048 g64 ring of {ncopy}: {us1:.2f} us per launch of one; "
        f"{usn / NST:.3f} us per matrix in launches of {NST} ({NST * per / (usn * 1e-6) / 1e9:.0f} GB/s)")
    del Tst, q, s
    torch.cuda.empty_cache()

    # what a trivial streaming read of one matrix-sized buffer reaches per
    # launch (same ring discipline): the per-launch ceiling at this size
    sink = torch.zeros(1, device=dev)
    mb21 = qbytes(4, 6144, 6144, 64)
    nring = max(2, -(-(1 << 30) // mb21))
    bufs = [torch.empty(mb21 // 16 * 16, dtype=torch.uint8, device=dev) for _ in range(nring)]
    us_probe = timed(lambda i: coli.check(coli.coli_probe_read(bufs[i % nring], sink, st), "probe"), 4 * nring)
    probe_gbs = bufs[0].numel() / (us_probe * 1e-6) / 1e9
    del bufs
    torch.cuda.empty_cache()
    out["stream_read_one_matrix"] = {"bytes": mb21, "us": us_probe, "GBps": probe_gbs}
    log(f"streaming read of one {mb21 / 1e6:.1f} MB matrix per launch: {us_probe:.2f} us ({probe_gbs:.0f} GB/s)")

    sweep, stack = {}, {}
    for fmt, gs in ((4, 64), (4, 128), (2, 0), (1, 0), (3, 0)):
        for S in (1, 4):
            mb = qbytes(fmt, 6144, 6144, gs)
            ncopy = max(2, -(-(1 << 30) // mb))
            q, s = sd.pool_on_device(11 + fmt, fmt, ncopy, 6144, 6144, gs)
            Ts = [coli.QTensor(fmt, q[c], s[c], 6144, 6144, gs, n=1) for c in range(ncopy)]
            for t in Ts:
                t.pack()
            x = torch.randn((S, 6144), device=dev)
            y = torch.empty((S, 6144), device=dev)
            us = timed(lambda i: coli.coli_qmatmul(Ts[i % ncopy], x, y, S, st), 4 * ncopy)
            gbs = (mb + S * 6144 * 8) / (us * 1e-6) / 1e9
            key = f"fmt{fmt}" + (f"_g{gs}" if fmt == 4 else "") + f"_S{S}"
            sweep[key] = {"us": us, "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                          "frac_stream_read_same_launch_size":
                              gbs / probe_gbs if abs(mb - mb21) < 0.2 * mb21 else None}
            log(f"sweep {key}: {us:.2f} us  {gbs:.0f} GB/s")
            # the same ring, NST distinct matrices per launch (a stack sharing
            # x, the pages' batched-expert form): the per-launch start-up is
            # paid once per NST matrices
            NST = 8
            nst = ncopy // NST
            Tst = [coli.QTensor(fmt, q[c * NST:(c + 1) * NST], s[c * NST:(c + 1) * NST], 6144,
                                6144, gs, n=NST) for c in range(nst)]
            for t in Tst:
                t.pack()
            ys = torch.empty((NST, S, 6144), device=dev)
            us = timed(lambda i: coli.coli_qmatmul(Tst[i % nst], x, ys, S, st), 4 * nst)
            gbs = NST * (mb + S * 6144 * 8) / (us * 1e-6) / 1e9
            stack[key] = {"matrices_per_launch": NST, "us_per_launch": us,
                          "us_per_matrix": us / NST, "GBps": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
            log(f"sweep {key} x{NST} per launch: {us / NST:.2f} us/matrix  {gbs:.0f} GB/s")
            del Ts, Tst, q, s
    out["gemv_6144x6144_ring"] = sweep
    out["gemv_6144x6144_ring_stacked"] = stack
    return out


def prefill_measurements(coli, sd, np, torch, log, timed):
    """S = 544 prefill: the dense 6144x6144 fmt-4 GEMM (compute-bound) and the
    256-expert MoE block with gs 128 on packed experts, routed by Zipf(1.1)
    popularity (HBM-bound: the union covers ~250 experts) and, as a labelled
    variant, Zipf(2.5) (union ~95, head experts with hundreds of rows)."""
    out = {}
    dev = "cuda"
    st = torch.cuda.current_stream()
    S = 544
    for gs in (128, 64):
        q, s = sd.pool_on_device(30 + gs, 4, 1, 6144, 6144, gs)
        T = coli.QTensor(4, q[0], s[0], 6144, 6144, gs, n=1)
        x = torch.randn((S, 6144), device=dev)
        y = torch.empty((S, 6144), device=dev)
        fl = 2.0 * S * 6144 * 6144
        # plain tensor, no workspace: the producer/consumer kernel
        us_pc = timed(lambda i: coli.coli_qmatmul(T, x, y, S, st), 20)
        # packed copy + workspace: inputs prepared once, K split over the
        # wavefronts (the launch pair the library uses for prefill rows)
        T.pack()
        wsb = coli.coli_qmatmul_workspace_bytes(T, S)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        us = timed(lambda i: coli.coli_qmatmul_ws(T, x, y, S, ws, wsb, st), 20)
        tf = fl / (us * 1e-6) / 1e12
        out[f"prefill_dense_544x6144x6144_g{gs}"] = {
            "us": us, "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            "kernels": "input prep + split-K GEMM (coli_qmatmul_ws, packed)",
            "producer_consumer_us": us_pc,
            "producer_consumer_frac_bf16_peak": fl / (us_pc * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
        log(f"prefill dense g{gs}: {us:.1f} us  {tf:.1f} TFLOP/s ({100 * tf / BF16_PEAK_TFLOPS:.1f}% of bf16 peak); "
            f"producer/consumer kernel {us_pc:.1f} us")
        del T, q, s, ws

    gs = 128
    gq, gsc = sd.pool_on_device(200, 4, E, F, D, gs)
    uq, usc = sd.pool_on_device(201, 4, E, F, D, gs)
    dq, dsc = sd.pool_on_device(202, 4, E, D, F, gs)
    tg = coli.QTensor(4, gq, gsc, F, D, gs)
    tu = coli.QTensor(4, uq, usc, F, D, gs)
    td = coli.QTensor(4, dq, dsc, D, F, gs)
    for t in (tg, tu, td):  # upload-time repack: the prefill kernels stream the packed blocks
        t.pack()
    wsb = coli.coli_moe_workspace_bytes(E, S, K, F, D, 0)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    outb = torch.empty((S, D), device=dev)
    for zs, key in ((1.1, "prefill_moe_544_zipf1.1_g128"), (2.5, "prefill_moe_544_zipf2.5_g128_variant")):
        r = sd.rng(4)
        xh = sd.gen_x(r, S, D)
        ids, w = sd.gen_routing_zipf(r, S, K, E, zs)
        xd = torch.from_numpy(xh).to(dev)
        idd = torch.from_numpy(ids).to(dev)
        wd = torch.from_numpy(w).to(dev)

        def blk(i):
            coli.check(coli.coli_moe_block(tg, tu, td, xd, S, idd, wd, K, None, None, None, outb,
                                           ws, wsb, st))
        us = timed(blk, 10)
        coli.coli_prof_reset()
        coli.coli_prof_enable(True)
        for i in range(5):
            blk(i)
        torch.cuda.synchronize()
        coli.coli_prof_enable(False)
        kern = {}
        for tag in coli.coli_prof_tags():
            n, tot = coli.coli_prof_read(tag)
            if n > 0 and not tag.startswith("probe") and tag != "pack":
                kern[tag] = tot / n * 1e3
        cnt = np.bincount(ids.ravel(), minlength=E)
        union = int((cnt > 0).sum())
        flops = 2.0 * S * K * 3 * F * D
        nbytes = union * (2 * qbytes(4, F, D, gs) + qbytes(4, D, F, gs)) + 2 * S * D * 4 + S * K * 8
        tf = flops / (us * 1e-6) / 1e12
        gbs = nbytes / (us * 1e-6) / 1e9
        ideal_us = max(flops / (BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)) * 1e6
        out[key] = {
            "us": us, "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS, "GBps": gbs,
            "frac_hbm": gbs / HBM_PEAK_GBS, "union_experts": union, "max_rows": int(cnt.max()),
            "experts_ge64_rows": int((cnt >= 64).sum()), "roofline_us": ideal_us,
            "frac_roofline": ideal_us / us, "kernels_us": kern}
        log(f"prefill MoE 544 zipf{zs}: {us:.1f} us  {tf:.1f} TFLOP/s  {gbs:.0f} GB/s  union {union}  "
            f"({100 * ideal_us / us:.1f}% of max(F/P, B/BW) = {ideal_us:.0f} us)  {kern}")
    del tg, tu, td, gq, gsc, uq, usc, dq, dsc, ws
    torch.cuda.empty_cache()
    return out


def router_measurements(coli, sd, np, torch, log, timed):
    """The router and exact top-K at the block's shape (E 256, D 6144, K 8)
    for one decode row and the S=544 prefill batch.  Device time per call
    from a graph of 20 calls replayed 10 times (a call from Python costs more
    than the kernels at S=1); the host-loop figure beside it."""
    dev = "cuda"
    r = sd.rng(9)
    R = torch.from_numpy((r.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)).to(dev)
    bias = torch.from_numpy((r.standard_normal(E) * 0.05).astype(np.float32)).to(dev)
    out = {}
    for S in (1, 544):
        x = torch.randn((S, D), device=dev)
        ids = torch.empty((S, K), dtype=torch.int32, device=dev)
        w = torch.empty((S, K), device=dev)
        wsb = coli.coli_moe_router_workspace_bytes(S, E)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def call(i=0):
            coli.check(coli.coli_moe_router(x, S, D, R, bias, E, K, 0.0, 1, 2.5, ids, w, ws, wsb,
                                            torch.cuda.current_stream()), "router")
        us_loop = timed(call, 50)
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            call()
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(20):
                call()
        us = timed(lambda i: g.replay(), 10) / 20
        del g
        nbytes = E * D * 4 + S * D * 4
        out[f"router_S{S}_E{E}_D{D}_K{K}"] = {"us": us, "us_host_loop": us_loop,
                                              "GBps": nbytes / (us * 1e-6) / 1e9}
        log(f"router S={S}: {us:.2f} us per call in a graph ({us_loop:.2f} us from a host loop; "
            f"{nbytes / (us * 1e-6) / 1e9:.0f} GB/s of router weights + inputs)")
    return out


def ceiling_probes(coli, torch, log):
    """What trivial kernels reach on this part: a streaming read of 4 GiB and a
    loop of independent bf16 32x32x16 matrix-core products."""
    st = torch.cuda.current_stream()
    sink = torch.zeros(1, device="cuda")

    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(st)
        for _ in range(n):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3  # s

    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    t = timed(lambda: coli.check(coli.coli_probe_read(buf, sink, st), "coli_probe_read"), 5)
    read_gbs = buf.numel() / t / 1e9
    del buf
    torch.cuda.empty_cache()
    wg, it = 2048, 1000
    t = timed(lambda: coli.check(coli.coli_probe_mfma(wg, it, sink, st), "coli_probe_mfma"), 3)
    mfma_tf = wg * it * coli.PROBE_MFMA_FLOPS_PER_WG_ITER / t / 1e12
    log(f"ceilings: streaming read {read_gbs:.0f} GB/s ({100 * read_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), "
        f"bf16 MFMA loop {mfma_tf:.0f} TFLOP/s ({100 * mfma_tf / BF16_PEAK_TFLOPS:.1f}% of 2.5 PFLOP/s)")
    # launch floor: an empty kernel back to back on the stream, and the same
    # launches replayed from a HIP graph (256 and 1024 workgroups)
    floor = {}
    for wg in (256, 1024):
        n = 2000
        t = timed(lambda: coli.check(coli.coli_probe_launch(wg, sink, st), "probe_launch"), n)
        floor[f"eager_{wg}wg_us"] = t * 1e6
        g = torch.cuda.CUDAGraph()
        gs_ = torch.cuda.Stream()
        with torch.cuda.stream(gs_):
            for _ in range(3):
                coli.check(coli.coli_probe_launch(wg, sink, gs_), "probe_launch")
            gs_.synchronize()
            g.capture_begin()
            for _ in range(100):
                coli.check(coli.coli_probe_launch(wg, sink, gs_), "probe_launch")
            g.capture_end()
        torch.cuda.synchronize()
        tg = timed(lambda: g.replay(), 20)
        floor[f"graph_{wg}wg_us"] = tg * 1e6 / 100
        del g
    log(f"launch floor (empty kernel): {floor}")
    return {"measured_ceilings": {"stream_read_GBps": read_gbs, "mfma_bf16_TFLOPs": mfma_tf,
                                  "stream_read_frac_spec": read_gbs / HBM_PEAK_GBS,
                                  "mfma_bf16_frac_spec": mfma_tf / BF16_PEAK_TFLOPS,
                                  "launch_floor_us": floor}}


def attention_prefill(coli, sd, np, torch, log, S=544, T_cap=1024, passes=5):
    """One MLA attention layer over a 544-token prompt (S = 544 rows from
    position 0, caches of 1024 rows): q_a, kv_a, q_b and o_proj on the bf16
    prefill GEMMs, the fp32 core on chunks of 4 rows; fmt 4 gs 64 at the
    layer's real dimensions.  FLOPs: the projections 2 S (qr D + (L + dr) D +
    H (dn + dr) qr + D H dv), the core (causal: row s has s + 1 keys) 2 H
    (dn L (S rows) + (L + dr) K + L K + L dv (S rows)) with K = the keys
    summed over the rows."""
    dev = "cuda"
    gs, H, dn, dr, dv, qr, Lat = 64, 64, 192, 64, 256, 1536, 512
    shapes = [(qr, D), (H * (dn + dr), qr), (Lat + dr, D), (H * (dn + dv), Lat), (D, H * dv)]
    P = [sd.pool_on_device(40000 + i, 4, 1, o, i_, gs) for i, (o, i_) in enumerate(shapes)]
    TP = [coli.QTensor(4, q[0], s_[0], o, i_, gs, n=1) for (q, s_), (o, i_) in zip(P, shapes)]
    for t in TP:  # (kv_b's packed copy serves the prefill value absorption)
        t.pack()
    qn = torch.rand(qr, device=dev) + 0.5
    kn = torch.rand(Lat, device=dev) + 0.5
    layer = coli.MlaLayer(*TP, qn, kn, H, dn, dr, dv, 1e-6, 10000.0)
    Lc = torch.zeros((T_cap, Lat), device=dev)
    Rc = torch.zeros((T_cap, dr), device=dev)
    x = torch.randn((S, D), device=dev)
    out = torch.empty((S, D), device=dev)
    wsb = coli.coli_mla_workspace_bytes(layer, S, T_cap)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def call(st):
        coli.check(coli.coli_mla_decode(layer, x, S, 0, Lc, Rc, T_cap, out, ws, wsb, st),
                   "coli_mla_decode")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = torch.cuda.current_stream()
    a.record(st)
    for _ in range(passes):
        graph.replay()
    b.record(st)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / passes * 1e3
    del graph
    keys = S * (S + 1) // 2
    proj = 2.0 * S * (qr * D + (Lat + dr) * D + H * (dn + dr) * qr + D * H * dv)
    core = 2.0 * H * (dn * Lat * S + (Lat + dr) * keys + Lat * keys + Lat * dv * S)
    # per-kernel split from one eager call with the library's events
    coli.coli_prof_reset()
    coli.coli_prof_enable(True)
    call(st)
    torch.cuda.synchronize()
    coli.coli_prof_enable(False)
    kern = {}
    for tag in coli.coli_prof_tags():
        n, tot = coli.coli_prof_read(tag)
        if n > 0:
            kern[tag] = {"launches": n, "total_us": tot * 1e3}
    log(f"MLA prefill attention S={S}: {us:.0f} us per layer, "
        f"{(proj + core) / us / 1e6:.1f} TFLOP/s ({proj / 1e9:.1f} GF projections, "
        f"{core / 1e9:.1f} GF core)")
    del TP, P, ws
    torch.cuda.empty_cache()
    return {"mla_prefill_544": {"us_per_layer": us, "ms_per_75_layers": us * 75 / 1e3,
                                "TFLOPs": (proj + core) / us / 1e6, "GF_projections": proj / 1e9,
                                "GF_core": core / 1e9, "kernels_eager": kern}}


def full_layer_stream(coli, sd, np, torch, log, layers=75, pool=20, passes=5, pos=544,
                      T_cap=1024):
    """75 whole decode layers (S = 1) back to back in one HIP graph, each one
    coli_layer_decode: in_ln RMSNorm, MLA attention at position 544 (64 heads
    of 192 + 64 / 256, latent 512 + 64, caches of 1024 rows holding 544
    earlier tokens; q_a 1536x6144, q_b 16384x1536, kv_a 576x6144, kv_b
    28672x512, o_proj 6144x16384), residual, post_ln RMSNorm, router with the
    exact top-8 over a resident pool of 20 experts, 8 routed + 1 shared
    expert (gate/up 2048x6144, down 6144x2048), residual -- all fmt 4 gs 64.
    Also the attention alone (75 coli_mla_decode calls in a graph) and, from
    one eager pass with the library's per-launch events, each kernel's
    average time."""
    dev = "cuda"
    gs, H, dn, dr, dv, qr, Lat = 64, 64, 192, 64, 256, 1536, 512
    log(f"full layer stream: drawing {layers} layers")
    shapes = [(qr, D), (H * (dn + dr), qr), (Lat + dr, D), (H * (dn + dv), Lat), (D, H * dv)]
    Ls = []
    for l in range(layers):
        P = [sd.pool_on_device(20000 + 10 * l + i, 4, 1, o, i_, gs) for i, (o, i_) in enumerate(shapes)]
        TP = [coli.QTensor(4, q[0], s_[0], o, i_, gs, n=1) for (q, s_), (o, i_) in zip(P, shapes)]
        for t in TP[:3] + TP[4:]:
            t.pack()
        qn = torch.rand(qr, device=dev) + 0.5
        kn = torch.rand(Lat, device=dev) + 0.5
        layer = coli.MlaLayer(*TP, qn, kn, H, dn, dr, dv, 1e-6, 10000.0)
        Lc = torch.zeros((T_cap, Lat), device=dev)
        Rc = torch.zeros((T_cap, dr), device=dev)
        Lc[:pos].normal_()
        Rc[:pos].normal_()
        mg = sd.pool_on_device(30000 + 4 * l, 4, pool + 1, F, D, gs)
        mu = sd.pool_on_device(30001 + 4 * l, 4, pool + 1, F, D, gs)
        md = sd.pool_on_device(30002 + 4 * l, 4, pool + 1, D, F, gs)
        tg = coli.QTensor(4, mg[0][:pool], mg[1][:pool], F, D, gs)
        tu = coli.QTensor(4, mu[0][:pool], mu[1][:pool], F, D, gs)
        td = coli.QTensor(4, md[0][:pool], md[1][:pool], D, F, gs)
        sg = coli.QTensor(4, mg[0][pool], mg[1][pool], F, D, gs, n=1)
        su = coli.QTensor(4, mu[0][pool], mu[1][pool], F, D, gs, n=1)
        sdn = coli.QTensor(4, md[0][pool], md[1][pool], D, F, gs, n=1)
        for t in (tg, tu, td, sg, su, sdn):
            t.pack()
        R = torch.randn((pool, D), device=dev) / D ** 0.5
        bias = torch.randn(pool, device=dev) * 0.05
        ln = (torch.rand(D, device=dev) + 0.5, torch.rand(D, device=dev) + 0.5)
        Ls.append((P, TP, layer, qn, kn, Lc, Rc, mg, mu, md, tg, tu, td, sg, su, sdn, R, bias, ln))
    x = torch.randn((1, D), device=dev)
    out = torch.empty((1, D), device=dev)
    a_out = torch.empty((1, D), device=dev)
    wsb = coli.coli_layer_decode_workspace_bytes(Ls[0][2], Ls[0][10], 1, K, T_cap, True)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    mwsb = coli.coli_mla_workspace_bytes(Ls[0][2], 1, T_cap)
    mws = torch.empty(mwsb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def layer_pass():
        st = torch.cuda.current_stream()
        for l in range(layers):
            (P, TP, layer, qn, kn, Lc, Rc, mg, mu, md, tg, tu, td, sg, su, sdn, R, bias,
             ln) = Ls[l]
            coli.check(coli.coli_layer_decode(layer, ln[0], tg, tu, td, ln[1], R, bias, K, 0.0, 1,
                                              2.5, sg, su, sdn, 1e-6, x, 1, pos, Lc, Rc, T_cap,
                                              out, ws, wsb, st), "coli_layer_decode")

    def attn_pass():
        st = torch.cuda.current_stream()
        for l in range(layers):
            layer, Lc, Rc = Ls[l][2], Ls[l][5], Ls[l][6]
            coli.check(coli.coli_mla_decode(layer, x, 1, pos, Lc, Rc, T_cap, a_out, mws, mwsb, st),
                       "coli_mla_decode")

    def timed_graph(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        a.record(st)
        for _ in range(passes):
            graph.replay()
        b.record(st)
        torch.cuda.synchronize()
        del graph
        return a.elapsed_time(b) / passes

    attn_w = sum(qbytes(4, o, i_, gs) for o, i_ in shapes)
    cache = (pos + 1) * (Lat + dr) * 4          # every key row read once
    attn_bytes = attn_w + cache + 2 * D * 4 + qr * 4 + Lat * 4
    moe_bytes = 9 * (2 * qbytes(4, F, D, gs) + qbytes(4, D, F, gs)) + pool * D * 4 + 3 * D * 4
    per_layer = attn_bytes + moe_bytes
    res = {}
    ms = timed_graph(layer_pass)
    gbs = layers * per_layer / (ms * 1e-3) / 1e9
    log(f"full decode layer x{layers}: {ms * 1e3 / layers:.1f} us/layer, {gbs:.0f} GB/s "
        f"({per_layer / 1e6:.1f} MB/layer)")
    res["layer_decode_75"] = {"us_per_layer": ms * 1e3 / layers, "GBps": gbs,
                              "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_layer": per_layer,
                              "pos": pos, "launches_per_layer": None}
    ms = timed_graph(attn_pass)
    gbs = layers * attn_bytes / (ms * 1e-3) / 1e9
    log(f"MLA decode attention x{layers}: {ms * 1e3 / layers:.1f} us/layer, {gbs:.0f} GB/s "
        f"({attn_bytes / 1e6:.1f} MB)")
    res["mla_decode_75"] = {"us_per_layer": ms * 1e3 / layers, "GBps": gbs,
                            "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_layer": attn_bytes,
                            "pos": pos}
    # per-kernel averages from one eager pass of whole layers
    n0 = coli.coli_stats()[2]
    coli.coli_prof_reset()
    coli.coli_prof_enable(True)
    layer_pass()
    torch.cuda.synchronize()
    coli.coli_prof_enable(False)
    res["layer_decode_75"]["launches_per_layer"] = (coli.coli_stats()[2] - n0) / layers
    kern = {}
    for tag in coli.coli_prof_tags():
        n, tot = coli.coli_prof_read(tag)
        if n > 0:
            kern[tag] = {"launches": n, "avg_us": tot / n * 1e3}
    res["layer_decode_75"]["kernels_eager"] = kern
    log(f"full layer kernels (eager, events per launch): {kern}")
    del Ls
    torch.cuda.empty_cache()
    return res


def layer_stream(coli, sd, np, torch, log, layers=75, pool=20, passes=10):
    """75 decode layers (S = 1) back to back in one HIP graph: per layer the
    q_a 1536x6144, q_b 16384x1536, kv_a 576x6144 and o_proj 6144x16384 GEMVs
    (each fed a fixed N(0,1) input of its length) and the MoE block with 8
    routed experts (drawn from a resident pool of 20 per layer) plus one
    shared expert, all fmt 4 gs 64 -- about 40 GB resident."""
    dev = "cuda"
    gs = 64
    log(f"layer stream: drawing {layers} layers")
    projs = [(1536, 6144), (16384, 1536), (576, 6144), (6144, 16384)]
    L = []
    for l in range(layers):
        P = [sd.pool_on_device(1000 + 10 * l + i, 4, 1, o, i_, gs) for i, (o, i_) in enumerate(projs)]
        TP = [coli.QTensor(4, q[0], s[0], o, i_, gs, n=1) for (q, s), (o, i_) in zip(P, projs)]
        for t in TP:
            t.pack()
        mg = sd.pool_on_device(5000 + 4 * l, 4, pool + 1, F, D, gs)
        mu = sd.pool_on_device(5001 + 4 * l, 4, pool + 1, F, D, gs)
        md = sd.pool_on_device(5002 + 4 * l, 4, pool + 1, D, F, gs)
        tg = coli.QTensor(4, mg[0][:pool], mg[1][:pool], F, D, gs)
        tu = coli.QTensor(4, mu[0][:pool], mu[1][:pool], F, D, gs)
        td = coli.QTensor(4, md[0][:pool], md[1][:pool], D, F, gs)
        sg = coli.QTensor(4, mg[0][pool], mg[1][pool], F, D, gs, n=1)
        su = coli.QTensor(4, mu[0][pool], mu[1][pool], F, D, gs, n=1)
        sdn = coli.QTensor(4, md[0][pool], md[1][pool], D, F, gs, n=1)
        for t in (tg, tu, td, sg, su, sdn):
            t.pack()
        L.append((P, TP, mg, mu, md, tg, tu, td, sg, su, sdn))
    r = sd.rng(75)
    routes = [sd.gen_routing_uniform(r, 1, K, pool) for _ in range(layers)]
    ids = torch.from_numpy(np.stack([a for a, _ in routes])).to(dev)
    wts = torch.from_numpy(np.stack([b for _, b in routes])).to(dev)
    xin = {i_: torch.randn((1, i_), device=dev) for _, i_ in projs}
    xin[D] = torch.randn((1, D), device=dev)
    outs = {o: torch.empty((1, o), device=dev) for o, _ in projs}
    mo = torch.empty((1, D), device=dev)
    wsb = coli.coli_moe_workspace_bytes(pool, 1, K, F, D, 1)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # the four projections take independent inputs here, so they go out as
    # one grouped submission; the second variant launches them one by one
    xs = [xin[i_] for _, i_ in projs]
    ys = [outs[o] for o, _ in projs]

    def one_pass(grouped):
        st = torch.cuda.current_stream()
        for l in range(layers):
            P, TP, mg, mu, md, tg, tu, td, sg, su, sdn = L[l]
            if grouped:
                coli.check(coli.coli_qmatmul_group(TP, xs, ys, 1, st))
            else:
                for T, (o, i_) in zip(TP, projs):
                    coli.check(coli.coli_qmatmul(T, xin[i_], outs[o], 1, st))
            coli.check(coli.coli_moe_block(tg, tu, td, xin[D], 1, ids[l], wts[l], K, sg, su, sdn,
                                           mo, ws, wsb, st))

    def timed_graph(grouped):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            one_pass(grouped)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_pass(grouped)
        graph.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        a.record(st)
        for _ in range(passes):
            graph.replay()
        b.record(st)
        torch.cuda.synchronize()
        del graph
        return a.elapsed_time(b) / passes

    attn = sum(qbytes(4, o, i_, gs) + (o + i_) * 4 for o, i_ in projs)
    moe = 9 * (2 * qbytes(4, F, D, gs) + qbytes(4, D, F, gs)) + 2 * D * 4
    per_layer = attn + moe
    resident = sum(sum(t.numel() * t.element_size() for t in (x[0], x[1]))
                   for l in L for x in (*l[0], l[2], l[3], l[4]))
    res = {}
    for grouped, key in ((True, "layer_stream_75"),
                         (False, "layer_stream_75_one_launch_per_projection")):
        n0 = coli.coli_stats()[2]
        one_pass(grouped)
        torch.cuda.synchronize()
        launches = (coli.coli_stats()[2] - n0) / layers
        ms = timed_graph(grouped)
        gbs = layers * per_layer / (ms * 1e-3) / 1e9
        log(f"{key}: {ms * 1e3:.0f} us/pass  {ms * 1e3 / layers:.1f} us/layer  {gbs:.0f} GB/s  "
            f"resident {resident / 1e9:.1f} GB")
        res[key] = {"us_per_pass": ms * 1e3, "us_per_layer": ms * 1e3 / layers, "GBps": gbs,
                    "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_layer": per_layer,
                    "resident_GB": resident / 1e9, "launches_per_layer": launches}
    del L
    torch.cuda.empty_cache()
    return res


def cpu_baseline(coli, sd, np, torch, gq, gsc, uq, usc, dq, dsc, x, routes, block_bytes,
                 seconds, log):
    """The oracle (plain f64 C, OpenMP over routed pairs) on decode blocks of
    the same workload, run until `seconds` of CPU time have been spent."""
    import oracle
    from oracle import QMat
    nthreads = len(os.sched_getaffinity(0))
    orc = oracle.get(nthreads=nthreads)
    done, spent = 0, 0.0
    for ids, w in routes:
        sel = torch.from_numpy(ids[0].astype(np.int64)).cuda()
        G = QMat(4, F, D, GS, gq[sel].cpu().numpy(), gsc[sel].cpu().numpy())
        U = QMat(4, F, D, GS, uq[sel].cpu().numpy(), usc[sel].cpu().numpy())
        Dn = QMat(4, D, F, GS, dq[sel].cpu().numpy(), dsc[sel].cpu().numpy())
        local = np.arange(K, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        orc.moe_block(G, U, Dn, x, local, w)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    gbs = done * block_bytes / spent / 1e9
    log(f"cpu oracle: {done} blocks in {spent:.1f} s -> {gbs:.3f} GB/s ({min(nthreads, K)} threads)")
    return {"value": gbs, "unit": "GB/s", "cores": min(nthreads, K), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{done} decode MoE blocks (S=1, 8 routed experts, full shapes), "
                      f"{spent:.1f} s of oracle time; OpenMP over the 8 routed pairs",
            "us_per_block": spent / done * 1e6}


def oracle_timings(sd, np, log):
    """The oracle on bounded samples of the other workloads, for context
    beside the GPU figures: the 6144x6144 fmt-4 g64 GEMV at S=1 (one and all
    host threads) and the S=544 Zipf(1.1) prefill MoE block on 4 of its
    tokens (each token's output depends only on its own row and routing),
    scaled to 544 tokens."""
    import oracle
    from oracle import QMat
    nthreads = len(os.sched_getaffinity(0))
    out = {"host_threads": nthreads, "cpu_model": _cpu_model()}
    r = sd.rng(3)
    x = sd.gen_x(r, 1, 6144)
    q, s = sd.gen_matrix(r, 4, 6144, 6144, 64)
    W = QMat(4, 6144, 6144, 64, q, s)
    for nt in (1, nthreads):
        orc = oracle.get(nthreads=nt)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 2.0:
            orc.qmatmul(W, x)
            n += 1
        us = (time.perf_counter() - t0) / n * 1e6
        out[f"gemv_6144x6144_g64_S1_threads{nt}_us"] = us
        log(f"oracle gemv 6144^2 g64 S=1, {nt} threads: {us:.0f} us")
    # prefill MoE: 4 tokens of the S=544 Zipf(1.1) draw, their experts only
    S, gs = 544, 128
    r = sd.rng(4)
    xh = sd.gen_x(r, S, D)
    ids, w = sd.gen_routing_zipf(r, S, K, E, 1.1)
    toks = np.arange(4)
    used = np.unique(ids[toks])
    remap = {int(e): i for i, e in enumerate(used)}
    rq = sd.rng(77)
    mats = [sd.gen_matrix(rq, 4, F, D, gs, n=len(used)), sd.gen_matrix(rq, 4, F, D, gs, n=len(used)),
            sd.gen_matrix(rq, 4, D, F, gs, n=len(used))]
    G = QMat(4, F, D, gs, *mats[0])
    U = QMat(4, F, D, gs, *mats[1])
    Dn = QMat(4, D, F, gs, *mats[2])
    local = np.vectorize(remap.get)(ids[toks]).astype(np.int32)
    orc = oracle.get(nthreads=nthreads)
    t0 = time.perf_counter()
    orc.moe_block(G, U, Dn, xh[toks], local, w[toks])
    sec = time.perf_counter() - t0
    out["prefill_moe_544_zipf1.1_4_tokens_s"] = sec
    out["prefill_moe_544_zipf1.1_scaled_to_544_tokens_s"] = sec * S / len(toks)
    log(f"oracle prefill MoE, 4 of 544 tokens ({nthreads} threads): {sec:.2f} s "
        f"-> ~{sec * S / len(toks):.0f} s for 544 tokens")
    return out


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name plus family /
    model / stepping (a virtual machine may shorten the name), and how many
    logical CPUs this process may use."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (t.strip() for t in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        pass
    name = info.get("model name", "unknown")
    fam = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    mhz = info.get("cpu MHz")
    extra = f"; {fam}" if fam else ""
    extra += f"; {mhz} MHz" if mhz else ""
    return (f"{name}{extra}; {len(os.sched_getaffinity(0))} logical CPUs usable of "
            f"{os.cpu_count()}")


if __name__ == "__main__":
    main()
