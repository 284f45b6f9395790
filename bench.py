#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one dsa_prefill call over the whole prefill workload (lightning indexer ->
top-k -> sparse MLA for every query row), inputs resident in HBM.  Prints ONE JSON line:
value = prefill tokens/s; `roofline` = the dominant kernel's algorithmic throughput against
MI355X's published peak, its average launch duration taken from HIP events in a per-kernel
pass that replays the fused call's chunks in the same launch configuration; `decode` = the
decode step (B sequences, one token each); `cpu_baseline` = the CPU oracle timed on a
bounded, uniformly sampled set of query rows of the same workload.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5000.0, "bf16": 2500.0}      # dense MFMA TFLOP/s, MI355X published
HBM_PEAK_GBS = 8000.0                       # GB/s
D_QK, D_V, D_I = 576, 512, 128
# HBM traffic per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by a
# plain copy of known size), keyed by workload; valid only for the kernel source it was taken on.
TRAFFIC_FILES = {"prefill-L131072-k2048": "profiles/prefill_L131072_k2048_hbm_traffic.txt"}
KERNEL_SOURCES = {"indexer": ["indexer.hip", "dsa_device.h"],
                  "topk": ["topk.hip", "dsa_device.h"],
                  "sparse_mla": ["sparse_mla.hip", "dsa_device.h"]}


def measured_traffic(workload, kernel, chunk_rows):
    """Counter-measured HBM bytes per launch (fetch + write) of `kernel` on `workload` at
    `chunk_rows` query rows per launch, or None when no such measurement exists or the kernel
    source has changed since it was taken."""
    import hashlib
    path = TRAFFIC_FILES.get(workload)
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_attention_05_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    with open(os.path.join(ROOT, path)) as fh:
        for line in fh:
            if not line.startswith("traffic "):
                continue
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if (kv.get("kernel") == kernel and kv.get("source") == digest
                    and kv.get("chunk_rows") == str(chunk_rows)):
                return int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-L131072-k2048")
    ap.add_argument("--decode-workload", default="decode-B64-L4096-131072-k2048")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-window", action="store_true",
                    help="skip timing sliding-window attention through the sparse MLA")
    ap.add_argument("--no-input-prep", action="store_true",
                    help="skip timing the fp8 quantisation of the indexer inputs")
    ap.add_argument("--varlen-workload", default="varlen-B16-L1024-32768-k2048,varlen-B128-L1024-k2048",
                    help="comma-separated packed-batch workloads")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip timing the packed multi-sequence prefill")
    ap.add_argument("--warmup-workload", default="prefill-L32768-k2048")
    ap.add_argument("--no-warmup-kl", action="store_true",
                    help="skip timing the indexer warm-up loss and gradient")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode only (for profiling runs; prints no prefill value)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the chip's MFMA and HBM-read peaks")
    ap.add_argument("--no-two-pass", action="store_true",
                    help="skip timing the prefill step with the two-pass selection")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other prefill configurations (dense fallback, 32K)")
    ap.add_argument("--configs", default="prefill-L2048-k2048-dense,prefill-L32768-k2048",
                    help="comma-separated further prefill workloads timed beside the main one")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy 5 times and exit (the known-size "
                         "reference for FETCH_SIZE / WRITE_SIZE counter scaling)")
    return ap.parse_args()


def prefill_units(L, T, q_pos0, k, t_lo, t_hi):
    """(visible pairs of rows that need scores, selected (row, index) pairs) over rows
    [t_lo, t_hi)."""
    pairs = sel = 0
    for t in range(t_lo, t_hi):
        n = min(L, q_pos0 + t + 1)
        if n > k:
            pairs += n
        sel += min(n, k)
    return pairs, sel


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_attention_05_amd as dsa
    from synth import WORKLOADS, make_decode, make_prefill

    dsa.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_launch": nbytes, "launches": 5}), flush=True)
        return
    cfg = WORKLOADS[args.workload]
    L, T, k, H_I, H = cfg.L, cfg.rows, cfg.k, cfg.H_I, cfg.H
    if args.no_prefill:
        decode = run_decode(args, WORKLOADS[args.decode_workload], dev)
        print(json.dumps({"decode": decode}), flush=True)
        return
    peaks = None if args.no_peaks else run_peaks(dev)
    log("generating", cfg.name)
    inp = make_prefill(cfg, device=dev)
    out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty((dsa.dsa_prefill_workspace_bytes(T, L, H_I, H, k),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step():
        dsa.dsa_prefill(inp["q8"], inp["qs"], inp["w"], inp["k8"], inp["ks"], inp["q"],
                        inp["kv"], k, cfg.q_pos0, cfg.score_scale, cfg.sm_scale, out=out,
                        lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done; timing %d steps" % args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tok_s = T / (ms / 1e3)
    log("prefill %.3f ms/step, %.0f tokens/s" % (ms, tok_s))

    # ---- the same step with the two-pass selection (every row's fp32 scores written by the
    # indexer and read back by top-k), for comparison with the candidate selection above
    two_pass = None
    if not args.no_two_pass:
        os.environ["DSA_PREFILL_UNFUSED"] = "1"
        try:
            step()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
        finally:
            del os.environ["DSA_PREFILL_UNFUSED"]
        ms2 = e0.elapsed_time(e1) / args.steps
        two_pass = dict(ms_per_step=round(ms2, 4), tokens_per_s=round(T / (ms2 / 1e3), 1),
                        steps=args.steps, candidate_selection_saves_ms=round(ms2 - ms, 3))
        log("prefill, two-pass selection: %.3f ms/step" % ms2)

    # ---- per-kernel pass: the fused call's chunks replayed through the single-kernel
    # entry points, HIP events around each launch on the same stream
    chunk = dsa.dsa_prefill_chunk_rows(T, L)
    sc = ws[: chunk * L * 4].view(torch.float32).view(chunk, L)
    idx = torch.empty((chunk, k), dtype=torch.int32, device=dev)
    t_sel = max(0, k - cfg.q_pos0)
    ktime = {"indexer": 0.0, "topk": 0.0, "sparse_mla": 0.0}
    kcount = {"indexer": 0, "topk": 0, "sparse_mla": 0}
    kunits = {"indexer": 0, "topk": 0, "sparse_mla": 0}
    events = []
    for r0 in range(0, T, chunk):
        rows = min(chunk, T - r0)
        s0 = max(r0, t_sel)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        evs[0].record(stream)
        if s0 < r0 + rows:
            sl = slice(s0, r0 + rows)
            dsa.dsa_index_scores(inp["q8"][sl], inp["qs"][sl], inp["w"][sl], inp["k8"],
                                 inp["ks"], cfg.q_pos0 + s0, cfg.score_scale,
                                 scores=sc[s0 - r0:rows], write_masked=False)
        evs[1].record(stream)
        dsa.dsa_topk(sc[:rows], L, cfg.q_pos0 + r0, k, idx=idx[:rows])
        evs[2].record(stream)
        dsa.dsa_sparse_mla(inp["q"][r0:r0 + rows], inp["kv"], idx[:rows], cfg.sm_scale,
                           out=out[r0:r0 + rows], lse=lse[r0:r0 + rows])
        evs[3].record(stream)
        pairs, sel = prefill_units(L, T, cfg.q_pos0, k, r0, r0 + rows)
        events.append((evs, s0 < r0 + rows, pairs, sel, rows))
    torch.cuda.synchronize()
    for evs, has_idx, pairs, sel, rows in events:
        if has_idx:
            ktime["indexer"] += evs[0].elapsed_time(evs[1])
            kcount["indexer"] += 1
            kunits["indexer"] += pairs
        ktime["topk"] += evs[1].elapsed_time(evs[2])
        kcount["topk"] += 1
        kunits["topk"] += pairs
        ktime["sparse_mla"] += evs[2].elapsed_time(evs[3])
        kcount["sparse_mla"] += 1
        kunits["sparse_mla"] += sel
    idx_flop = 2.0 * H_I * D_I                     # per visible pair
    mla_flop = 2.0 * H * (D_QK + D_V)              # per selected (row, index)
    kern = {}
    for name in ktime:
        if kcount[name] == 0:
            continue
        sec = ktime[name] / 1e3
        if name == "indexer":
            ach, unit, peak, bound = kunits[name] * idx_flop / sec / 1e12, "TFLOP/s", PEAK["fp8"], "mfma"
        elif name == "sparse_mla":
            ach, unit, peak, bound = kunits[name] * mla_flop / sec / 1e12, "TFLOP/s", PEAK["bf16"], "mfma"
        else:
            ach, unit, peak, bound = kunits[name] * 4.0 / sec / 1e9, "GB/s", HBM_PEAK_GBS, "hbm"
        kern[name] = dict(total_ms=round(ktime[name], 3), launches=kcount[name],
                          avg_launch_ms=round(ktime[name] / kcount[name], 4),
                          achieved=round(ach, 2), unit=unit, peak=peak,
                          frac=round(ach / peak, 4), bound=bound,
                          traffic=measured_traffic(cfg.name, name, chunk))
        mp = measured_peak_for(peaks, bound, name)
        if mp:
            kern[name]["measured_peak"] = mp
            kern[name]["frac_of_measured"] = round(ach / mp, 4)
        if name == "sparse_mla":
            # the selected rows it gathers (1152 B each) from L2 / the last-level cache / HBM
            kern[name]["gather_GBps"] = round(kunits[name] * D_QK * 2 / sec / 1e9, 1)
    dom = max(kern, key=lambda n: kern[n]["total_ms"])
    log("kernels:", json.dumps(kern))
    roofline = dict(bound=kern[dom]["bound"], achieved=kern[dom]["achieved"],
                    peak=kern[dom]["peak"], unit=kern[dom]["unit"], frac=kern[dom]["frac"],
                    traffic=kern[dom]["traffic"], kernel=dom, avg_launch_ms=kern[dom]["avg_launch_ms"])
    if "frac_of_measured" in kern[dom]:
        roofline["measured_peak"] = kern[dom]["measured_peak"]
        roofline["frac_of_measured"] = kern[dom]["frac_of_measured"]
    sum_pairs, sum_sel = prefill_units(L, T, cfg.q_pos0, k, 0, T)
    prefill_flops = sum_pairs * idx_flop + sum_sel * mla_flop
    del sc, idx

    # ---- the other prefill configurations (dense fallback, 32K), after the main one is freed
    main_inputs = (inp, out, lse, ws)

    # ---- decode
    decode = None if args.no_decode else run_decode(args, WORKLOADS[args.decode_workload], dev,
                                                    peaks, want_host=not args.no_cpu_baseline)
    dec_host = decode.pop("_host", None) if decode else None

    # ---- sliding-window attention through the same sparse MLA (an alternative index rule)
    window = None if args.no_window else run_window(args, cfg, inp, out, lse, chunk, dev)

    # ---- fp8 preparation of the same workload's indexer inputs (outside the step)
    prep = None if args.no_input_prep else run_input_prep(args, cfg, dev)

    # ---- packed multi-sequence prefill (fresh prefills and chunks against caches)
    varlen = None if args.no_varlen else [run_varlen(args, WORKLOADS[w], dev)
                                          for w in args.varlen_workload.split(",")]

    # ---- indexer warm-up: KL to the dense attention distribution and its gradient
    warm = None if args.no_warmup_kl else run_warmup_kl(args, WORKLOADS[args.warmup_workload], dev)

    # ---- CPU oracle baseline on sampled rows of the same prefill workload, and the whole
    # decode step of the decode workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, cfg, args.cpu_seconds)
        if dec_host is not None:
            cpu["decode"] = cpu_baseline_decode(dec_host)
        del dec_host
    del main_inputs, inp, out, lse, ws
    torch.cuda.empty_cache()
    configs = None if args.no_configs else [run_prefill_config(args, WORKLOADS[w], dev, peaks)
                                            for w in args.configs.split(",") if w]

    res = {
        "metric": "DSA prefill tokens/s at L=128K (k=2048); decode tokens/s; % MFMA/HBM peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 MLA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1), fp8 per-vector scales, 1% planted indexer keys)",
        "config": {"workload": cfg.name, "L": L, "query_rows": T, "k": k, "H_I": H_I, "H": H,
                   "batch": 1, "chunk_rows": chunk,
                   "algorithmic_tflop_per_step": round(prefill_flops / 1e12, 3)},
        "roofline": roofline,
        "measured_peaks": peaks,
        "kernels": kern,
        "prefill_two_pass": two_pass,
        "prefill_configs": configs,
        "decode": decode,
        "input_prep": prep,
        "window_attention": window,
        "varlen_prefill": varlen,
        "indexer_warmup": warm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def run_decode(args, dcfg, dev, peaks=None, want_host=False):
    """Time dsa_decode on one batch of the decode workload; returns its result object (with
    the inputs as host arrays under "_host" when want_host, for the CPU oracle's timing)."""
    import numpy as np
    import torch

    import sparse_attention_05_amd as dsa
    from synth import make_decode

    log("generating", dcfg.name)
    dinp = make_decode(dcfg, device=dev)
    B, N = dcfg.B, dinp["N"]
    dout = torch.empty((B, dcfg.H, D_V), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((B, dcfg.H), dtype=torch.float32, device=dev)
    dws = torch.empty((dsa.dsa_decode_workspace_bytes(B, dinp["max_len"], N, dcfg.H_I, dcfg.H,
                                                      dcfg.k),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def dstep():
        dsa.dsa_decode(dinp["seq_start"], dinp["max_len"], dinp["q8"], dinp["qs"], dinp["w"],
                       dinp["k8"], dinp["ks"], dinp["q"], dinp["kv"], dcfg.k, dcfg.score_scale,
                       dcfg.sm_scale, out=dout, lse=dlse, workspace=dws)

    for _ in range(args.warmup):
        dstep()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dsteps = max(args.steps, 20)
    d0.record(stream)
    for _ in range(dsteps):
        dstep()
    d1.record(stream)
    torch.cuda.synchronize()
    dms = d0.elapsed_time(d1) / dsteps
    lens = dinp["lens"].cpu().numpy()
    hbm = (lens.sum() * (D_I + 4) + np.minimum(lens, dcfg.k).sum() * D_QK * 2
           + B * dcfg.H_I * (D_I + 8) + B * dcfg.H * (D_QK * 2 + D_V * 2 + 4))
    gbs = hbm / (dms / 1e3) / 1e9
    log("decode %.4f ms/step, %.0f tokens/s, %.0f GB/s" % (dms, B / (dms / 1e3), gbs))
    # the cache append that precedes a decode step (new key quantised, latent row copied)
    g = torch.Generator(device=dev)
    g.manual_seed(17)
    k_new = torch.randn((B, D_I), generator=g, device=dev).to(torch.bfloat16)
    kv_new = torch.randn((B, D_QK), generator=g, device=dev).to(torch.bfloat16)

    def append():
        dsa.dsa_decode_append(dinp["seq_start"], k_new, kv_new, dinp["k8"], dinp["ks"], dinp["kv"])

    for _ in range(3):
        append()
    torch.cuda.synchronize()
    d0.record(stream)
    for _ in range(50):
        append()
    d1.record(stream)
    torch.cuda.synchronize()
    app_us = d0.elapsed_time(d1) / 50 * 1e3
    log("decode cache append %.2f us" % app_us)
    res = dict(workload=dcfg.name, ms_per_step=round(dms, 4),
               tokens_per_s=round(B / (dms / 1e3), 1), sequences=B, context_tokens=int(N),
               steps=dsteps, append_us=round(app_us, 2),
               roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS,
                             unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                             algorithmic_bytes=int(hbm)))
    mp = measured_peak_for(peaks, "hbm", "decode")
    if mp:
        res["roofline"]["measured_peak"] = mp
        res["roofline"]["frac_of_measured"] = round(gbs / mp, 4)
    if want_host:
        from synth import host_arrays
        res["_host"] = host_arrays(dinp)
    del dinp, dout, dlse, dws
    torch.cuda.empty_cache()
    return res


def measured_peak_for(peaks, bound, name):
    """The measured peak a kernel's roofline is also compared with (None when not measured)."""
    if not peaks:
        return None
    if bound == "hbm":
        return peaks["hbm_read_GBps"]
    return peaks["fp8_tflops"] if name == "indexer" else peaks["bf16_tflops"]


def run_peaks(dev):
    """The chip's measured peaks: dependency-free fp8 and bf16 MFMA streams on random
    operands (one and two waves per SIMD on all 256 CUs; the better of the two) and a plain
    16-byte read of an 8 GiB buffer (libdsa_peaks.so).  Each timed with HIP events on the
    launch stream, best of three."""
    import ctypes

    import torch

    from sparse_attention_05_amd import build as hip_build

    lib = ctypes.CDLL(hip_build.PEAKS_LIB)
    lib.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.dsa_peak_mfma.restype = lib.dsa_peak_read.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(2 * cus * 256, dtype=torch.float32, device=dev)

    def best(launch, reps=3):
        launch()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t)

    res = {}
    for kind, name, flop in ((0, "fp8_tflops", 2 * 16 * 16 * 128), (1, "bf16_tflops", 2 * 16 * 16 * 32)):
        iters = 4000 if kind == 0 else 8000
        rates = []
        for per_simd in (1, 2):
            blocks = cus * per_simd
            ms = best(lambda: lib.dsa_peak_mfma(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()), sp))
            rates.append(blocks * 4 * iters * 8 * flop / (ms / 1e3) / 1e12)
        res[name] = round(max(rates), 1)
    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ms = best(lambda: lib.dsa_peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes, cus * 16,
                                        ctypes.c_void_p(sink.data_ptr()), sp), reps=5)
    res["hbm_read_GBps"] = round(nbytes / (ms / 1e3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    res["method"] = ("dependency-free MFMA streams (8 independent accumulators per wave, random "
                     "finite operands, 1 and 2 waves per SIMD on every CU) and one 16-byte-load "
                     "read of an 8 GiB buffer; best of 3 / 5 runs")
    res["published"] = {"fp8_tflops": PEAK["fp8"], "bf16_tflops": PEAK["bf16"],
                        "hbm_GBps": HBM_PEAK_GBS}
    log("measured peaks:", json.dumps({k: v for k, v in res.items() if k not in ("method",)}))
    return res


def run_prefill_config(args, pcfg, dev, peaks):
    """One dsa_prefill call over a further prefill workload (every query row, inputs resident
    in HBM): ms, tokens/s, and the fraction of the time its algorithmic work takes at peak
    (indexer flops at the fp8 MFMA peak plus attention flops at the bf16 peak)."""
    import torch

    import sparse_attention_05_amd as dsa
    from synth import make_prefill

    log("generating", pcfg.name)
    inp = make_prefill(pcfg, device=dev)
    L, T, k, H_I, H = pcfg.L, pcfg.rows, pcfg.k, pcfg.H_I, pcfg.H
    out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty((max(1, dsa.dsa_prefill_workspace_bytes(T, L, H_I, H, k)),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        dsa.dsa_prefill(inp["q8"], inp["qs"], inp["w"], inp["k8"], inp["ks"], inp["q"],
                        inp["kv"], k, pcfg.q_pos0, pcfg.score_scale, pcfg.sm_scale, out=out,
                        lse=lse, workspace=ws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    reps = 10 if L <= 4096 else 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs, sel = prefill_units(L, T, pcfg.q_pos0, k, 0, T)
    f_idx, f_mla = pairs * 2.0 * H_I * D_I, sel * 2.0 * H * (D_QK + D_V)
    ideal = (f_idx / (PEAK["fp8"] * 1e12) + f_mla / (PEAK["bf16"] * 1e12)) * 1e3
    res = dict(workload=pcfg.name, L=L, query_rows=T, k=k, H_I=H_I, H=H, ms=round(ms, 4),
               tokens_per_s=round(T / (ms / 1e3), 1),
               algorithmic_tflop=round((f_idx + f_mla) / 1e12, 4),
               ms_at_peak=round(ideal, 4), frac_of_peak=round(ideal / ms, 4))
    if peaks:
        ideal_m = (f_idx / (peaks["fp8_tflops"] * 1e12) + f_mla / (peaks["bf16_tflops"] * 1e12)) * 1e3
        res["frac_of_measured_peak"] = round(ideal_m / ms, 4)
    log("prefill %s: %.3f ms, %.0f tokens/s, %.3f of peak" % (pcfg.name, ms, T / (ms / 1e3),
                                                             ideal / ms))
    del inp, out, lse, ws
    torch.cuda.empty_cache()
    return res


def run_window(args, cfg, inp, out, lse, chunk, dev, W=2048):
    """Time sliding-window attention (window W = k) over the workload's query rows: per chunk
    of `chunk` rows, the window index lists (dsa_window_indices) and dsa_sparse_mla on them.
    The same flops per selected row as the DSA path; the gathered rows are contiguous."""
    import torch

    import sparse_attention_05_amd as dsa

    L, T, H = cfg.L, cfg.rows, cfg.H
    idx = torch.empty((chunk, W), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        for r0 in range(0, T, chunk):
            r1 = min(T, r0 + chunk)
            ic = idx[:r1 - r0]
            dsa.dsa_window_indices(r1 - r0, L, cfg.q_pos0 + r0, W, idx=ic)
            dsa.dsa_sparse_mla(inp["q"][r0:r1], inp["kv"], ic, cfg.sm_scale, out=out[r0:r1],
                               lse=lse[r0:r1])

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 2
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    sel = sum(min(cfg.q_pos0 + t + 1, W) for t in range(T))
    tflops = sel * 2.0 * H * (D_QK + D_V) / (ms / 1e3) / 1e12
    log("window attention W=%d: %.2f ms, %.0f TFLOP/s" % (W, ms, tflops))
    return dict(workload="%s, window %d" % (cfg.name, W), ms=round(ms, 3),
                tokens_per_s=round(T / (ms / 1e3), 1), selected_rows=int(sel),
                roofline=dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK["bf16"],
                              unit="TFLOP/s", frac=round(tflops / PEAK["bf16"], 4)))


def run_varlen(args, vcfg, dev):
    """Time dsa_prefill_varlen on a packed batch of sequences (host cu_seqlens): every query
    row of every sequence through indexer -> top-k -> sparse MLA, as in the main step."""
    import torch

    import sparse_attention_05_amd as dsa
    from synth import make_varlen_cfg

    log("generating", vcfg.name)
    d = make_varlen_cfg(vcfg, device=dev)
    Tq, H = d["Tq"], vcfg.H
    out = torch.empty((Tq, H, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    ws = torch.empty((max(1, dsa.dsa_prefill_varlen_workspace_bytes(d["cu_q"], d["cu_k"],
                                                                    vcfg.H_I, H, vcfg.k)),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        dsa.dsa_prefill_varlen(d["cu_q"], d["cu_k"], d["q8"], d["qs"], d["w"], d["k8"],
                               d["ks"], d["q"], d["kv"], vcfg.k, vcfg.score_scale,
                               vcfg.sm_scale, out=out, lse=lse, workspace=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs = sel = 0
    for T, L in zip(d["lens_q"], d["lens_k"]):
        p, s_ = prefill_units(L, T, L - T, vcfg.k, 0, T)
        pairs += p
        sel += s_
    f_idx = pairs * 2.0 * vcfg.H_I * D_I                 # fp8 MFMA
    f_mla = sel * 2.0 * H * (D_QK + D_V)                  # bf16 MFMA
    flops = f_idx + f_mla
    # the call's work at peak: indexer flops at the fp8 peak, attention flops at the bf16
    # peak, the top-k's 4-byte score reads at HBM peak
    ideal_ms = (f_idx / (PEAK["fp8"] * 1e12) + f_mla / (PEAK["bf16"] * 1e12)
                + pairs * 4.0 / (HBM_PEAK_GBS * 1e9)) * 1e3
    log("varlen prefill %s: %d query rows over %d cached tokens, %.2f ms, %.0f tokens/s"
        % (vcfg.name, Tq, d["Lk"], ms, Tq / (ms / 1e3)))
    res = dict(workload=vcfg.name, sequences=vcfg.B, query_rows=Tq, key_rows=d["Lk"],
               lens_q=d["lens_q"], lens_k=d["lens_k"], ms=round(ms, 3),
               tokens_per_s=round(Tq / (ms / 1e3), 1),
               algorithmic_tflop=round(flops / 1e12, 3),
               effective_tflop_s=round(flops / (ms / 1e3) / 1e12, 1),
               ms_at_peak=round(ideal_ms, 3), frac_of_peak=round(ideal_ms / ms, 4))
    del d, out, lse, ws
    torch.cuda.empty_cache()
    return res


def run_warmup_kl(args, wcfg, dev):
    """Time dsa_indexer_warmup (teacher lse and distribution, indexer scores, per-row KL and
    G, the dq/dw and dk contractions) over every query row of the workload; the two teacher
    passes are also timed per chunk through their own entry points (HIP events on the same
    stream) for the roofline of the dominant kernel."""
    import torch

    import sparse_attention_05_amd as dsa
    from synth import make_prefill

    log("generating", wcfg.name, "for the warm-up step")
    d = make_prefill(wcfg, device=dev)
    T, L, H_I, H = wcfg.rows, wcfg.L, wcfg.H_I, wcfg.H
    out = dict(kl=torch.empty((T,), dtype=torch.float32, device=dev),
               dq=torch.empty((T, H_I, 128), dtype=torch.float32, device=dev),
               dw=torch.empty((T, H_I), dtype=torch.float32, device=dev),
               dk=torch.empty((L, 128), dtype=torch.float32, device=dev),
               lse_teacher=torch.empty((T, H), dtype=torch.float32, device=dev),
               lse_index=torch.empty((T,), dtype=torch.float32, device=dev))
    ws = torch.empty((dsa.dsa_indexer_warmup_workspace_bytes(T, L, H_I, H),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def run():
        dsa.dsa_indexer_warmup(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["q"], d["kv"],
                               wcfg.q_pos0, wcfg.score_scale, wcfg.sm_scale, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps

    # teacher passes per chunk (the call's own chunking), events around each launch
    chunk = dsa.dsa_prefill_chunk_rows(T, L)
    P = ws[: chunk * L * 4].view(torch.float32).view(chunk, L)
    evs = []
    for r0 in range(0, T, chunk):
        rows = min(chunk, T - r0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        dsa.dsa_attention_lse(d["q"][r0:r0 + rows], d["kv"], wcfg.q_pos0 + r0, wcfg.sm_scale,
                              lse=out["lse_teacher"][r0:r0 + rows])
        ev[1].record(stream)
        dsa.dsa_attention_distribution(d["q"][r0:r0 + rows], d["kv"],
                                       out["lse_teacher"][r0:r0 + rows], wcfg.q_pos0 + r0,
                                       wcfg.sm_scale, P=P[:rows])
        ev[2].record(stream)
        evs.append(ev)
    torch.cuda.synchronize()
    t_lse = sum(e[0].elapsed_time(e[1]) for e in evs)
    t_dist = sum(e[1].elapsed_time(e[2]) for e in evs)
    pairs = sum(min(L, wcfg.q_pos0 + t + 1) for t in range(T))
    f_teacher = pairs * 2.0 * H * D_QK                 # one pass over the dense logits
    f_index = pairs * 2.0 * H_I * D_I                  # indexer scores (fp8)
    f_back = 2 * (pairs * 2.0 * H_I * D_I) * 2         # dq and dk: fp8 recompute + bf16 contraction
    flops = 2 * f_teacher + f_index + f_back
    ach = f_teacher / (t_dist / 1e3) / 1e12
    log("indexer warm-up %s: %.2f ms (teacher lse %.2f ms, distribution %.2f ms), %.0f tokens/s"
        % (wcfg.name, ms, t_lse, t_dist, T / (ms / 1e3)))
    res = dict(workload="%s, indexer warm-up (KL to the dense distribution + gradient)" % wcfg.name,
               ms=round(ms, 3), tokens_per_s=round(T / (ms / 1e3), 1),
               teacher_lse_ms=round(t_lse, 3), teacher_dist_ms=round(t_dist, 3),
               chunk_rows=chunk, launches_per_pass=len(evs),
               algorithmic_tflop=round(flops / 1e12, 3),
               effective_tflop_s=round(flops / (ms / 1e3) / 1e12, 1),
               roofline=dict(kernel="teacher distribution", bound="mfma", achieved=round(ach, 2),
                             peak=PEAK["bf16"], unit="TFLOP/s", frac=round(ach / PEAK["bf16"], 4),
                             avg_launch_ms=round(t_dist / len(evs), 4)))
    del d, out, ws, P
    torch.cuda.empty_cache()
    return res


def run_input_prep(args, cfg, dev):
    """Time dsa_quantize_fp8 on the workload's indexer inputs (T x H_I query vectors and L key
    vectors, bf16, in one call): HBM-bound, 256 B read + 132 B written per vector."""
    import torch

    import sparse_attention_05_amd as dsa

    n = cfg.L * cfg.H_I + cfg.L
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    x = torch.randn((n, D_I), generator=g, device=dev).to(torch.bfloat16)
    q8 = torch.empty((n, D_I), dtype=torch.uint8, device=dev)
    sc = torch.empty((n,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dsa.dsa_quantize_fp8(x, q8, sc)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        dsa.dsa_quantize_fp8(x, q8, sc)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = n * (D_I * 2 + D_I + 4)
    gbs = nbytes / (ms / 1e3) / 1e9
    log("input prep: %d vectors in %.3f ms, %.0f GB/s" % (n, ms, gbs))
    del x, q8, sc
    return dict(workload="fp8 quantisation of %s indexer inputs (bf16)" % cfg.name, vectors=n,
                ms=round(ms, 4), vectors_per_s=round(n / (ms / 1e3), 1),
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(gbs / HBM_PEAK_GBS, 4), algorithmic_bytes=int(nbytes)))


def host_info():
    """The host the oracle ran on: the CPUs this process may use, OMP_NUM_THREADS, the model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(affinity_cpus=len(os.sched_getaffinity(0)),
                omp_num_threads=os.environ.get("OMP_NUM_THREADS"), cpu_model=model)


def cpu_baseline(inp, cfg, seconds):
    """The oracle, as it is, on uniformly sampled query rows of the workload (indexer scores,
    top-k and sparse MLA of each row), all sampled rows in one call per step so that its
    OpenMP loop over rows uses every thread it has.  Rows are drawn uniformly over the
    workload, so rows/s is an unbiased estimate of the oracle's tokens/s on all of it."""
    import numpy as np
    import torch

    import oracle

    k8 = inp["k8"].cpu().numpy()
    ks = inp["ks"].cpu().numpy()
    kv = inp["kv"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    q8, qs, w = inp["q8"].cpu().numpy(), inp["qs"].cpu().numpy(), inp["w"].cpu().numpy()
    rng = np.random.default_rng(cfg.seed)

    def run(rows):
        rows = np.sort(np.asarray(rows, np.int64))
        dev_rows = torch.as_tensor(rows, device=inp["q"].device)
        q = inp["q"][dev_rows].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        sc = oracle.index_scores(q8, qs, w, k8, ks, cfg.q_pos0, cfg.score_scale, rows=rows)
        idx = oracle.topk(sc, cfg.q_pos0 + rows + 1, cfg.k)
        oracle.sparse_mla(q, kv, idx, cfg.sm_scale)
        return time.perf_counter() - t0

    threads = oracle.num_threads()
    probe = rng.integers(0, cfg.rows, max(8, threads))
    tp = run(probe)
    n = int(min(1024, max(len(probe), seconds / max(tp / len(probe), 1e-6))))
    rows = rng.integers(0, cfg.rows, n)
    log("cpu oracle: %d sampled rows (probe %.2f s for %d)" % (n, tp, len(probe)))
    sec = run(rows)
    res = dict(value=round(n / sec, 3), unit="tokens/s", cores=threads, kind="oracle",
               seconds=round(sec, 2),
               sample="%d query rows drawn uniformly from the %d rows of %s (indexer scores + "
                      "top-k + sparse MLA per row, rows spread over %d host threads)"
                      % (n, cfg.rows, cfg.name, threads))
    res.update(host_info())
    return res


def cpu_baseline_decode(h):
    """The oracle on the whole decode step of the decode workload (every sequence: indexer
    scores over its cache, top-k, sparse MLA), sequences spread over the host threads."""
    from concurrent.futures import ThreadPoolExecutor
    import ctypes

    import numpy as np

    import oracle

    st = np.asarray(h["seq_start"], np.int64)
    B, k = h["B"], h["k"]
    threads = oracle.num_threads()

    def one(b):
        try:
            ctypes.CDLL("libgomp.so.1").omp_set_num_threads(1)
        except OSError:
            pass
        a, e = int(st[b]), int(st[b + 1])
        sc = oracle.index_scores(h["q8"][b:b + 1], h["qs"][b:b + 1], h["w"][b:b + 1],
                                 h["k8"][a:e], h["ks"][a:e], e - a - 1, h["score_scale"])
        idx = oracle.topk(sc, [e - a], k)
        oracle.sparse_mla(h["q"][b:b + 1], h["kv"][a:e], idx, h["sm_scale"])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(B)))
    sec = time.perf_counter() - t0
    log("cpu oracle decode: %d sequences in %.2f s" % (B, sec))
    res = dict(value=round(B / sec, 3), unit="tokens/s", cores=threads, kind="oracle",
               seconds=round(sec, 2),
               sample="the whole decode step: %d sequences, %d cached tokens" % (B, int(st[-1])))
    res.update(host_info())
    return res


if __name__ == "__main__":
    main()
