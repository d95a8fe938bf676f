"""Benchmark: exact attention prefill TFLOP/s and KV-cache decode GB/s on one MI355X.

One JSON line is printed.  ``value`` is the prefill throughput of the headline
workload: attn_fwd on B=2, H=8, S=2048, D=64, fp16 (N(0,1) inputs, scale
1/8), one non-causal and one causal call per step; algorithmic work
2*(Dqk+Dv) flop per unmasked (query, key) pair.  The same line carries the
decode throughput (KV bytes read per second) of the single-token GQA decode
workload, every other workload's timing, the roofline entry of the dominant
kernel and the fp64 CPU oracle's throughput on a bounded sample.

Inputs are resident in HBM before the timed region.  GPU time comes from HIP
events recorded on the stream the library launches on (torch's current
stream), around back-to-back calls.  Decode and chunked-prefill calls cycle
through 4 input/cache replicas so each call reads HBM rather than the 256 MB
Infinity Cache.
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

PEAK_TFLOPS = 2516.6     # dense fp16/bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0    # HBM3E
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 MFMA (twice the fp16 rate)
# FP8-input attention runs Q K^T in fp8 and P V in bf16 (half of the flops each)
PEAK_FP8_BLEND = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_TFLOPS)
METRIC = "attn prefill TFLOP/s + decode KV GB/s at 1 GPU, as % of MI355X peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of extra workloads to time: decode, chunked, window, bwd, varlen, fp8, asym, empty "
                         "(default: all; 'none' times the headline only)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize", default="",
                    help="print a text summary of a rocprofv3 CSV output directory and exit")
    return ap.parse_args()


def time_loop(calls, steps, warmup, torch):
    """Average seconds per call over `steps` back-to-back calls (cycling through `calls`)."""
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        calls[i % n]()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def summarize(d):
    """Text summary of rocprofv3 CSV output: kernel durations and per-dispatch counters."""
    import csv
    import glob
    from collections import defaultdict
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print("# kernel statistics (%s)" % os.path.relpath(path, d))
        print("%-100s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
        for r in csv.DictReader(open(path)):
            print("%-100s %6s %12.2f %12.2f %12.2f" % (r["Name"][:100], r["Calls"],
                  float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        print("# counters per dispatch, averaged (%s)" % os.path.relpath(path, d))
        agg = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, cs in agg.items():
            print(k[:120])
            for cn, v in sorted(cs.items()):
                print("    %-32s %16.6g   (dispatches: %d)" % (cn, sum(v) / len(v), len(v)))


def sources_sha256(paths):
    """One digest over the given source files (the kernel file and the headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(p.encode())
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def traffic_entry(kernel_key):
    """Measured HBM bytes per launch for a kernel, if its sources are unchanged since measured."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec:
        return None
    srcs = rec.get("sources", [])
    if not srcs or not all(os.path.exists(os.path.join(ROOT, p)) for p in srcs):
        return None
    if sources_sha256(srcs) != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_qk_amd as E     # raises if libattn.so is missing
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    dev = "cuda"
    K, Wm = args.steps, args.warmup
    only = set(x for x in args.only.split(",") if x)
    results = {}

    def want(name):
        return not only or name in only   # "none" matches no workload

    # ---------------- headline: attn_fwd B=2 H=8 S=2048 D=64 fp16, non-causal + causal
    hl = {}
    for causal in (False, True):
        c = W.fwd_d64(causal)
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        out = torch.empty_like(q)
        call = E.prepare_fwd(q, k, v, out, causal, c.softmax_scale)
        t = time_loop([call], K, Wm, torch)
        fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, causal)
        hl[causal] = (t, fl)
        results["fwd_b2h8s2048d64" + ("_causal" if causal else "")] = {
            "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
            "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS}
    step_s = hl[False][0] + hl[True][0]
    step_flops = hl[False][1] + hl[True][1]
    value = step_flops / step_s / 1e12

    # ---------------- decode: GQA 32/8, D=128, bf16, RoPE rd=128, cache 8192 (4 replicas)
    decode = None
    if want("decode"):
        c = W.decode_gqa()
        lens = W.seqlens_list(c.cache_seqlens, 8)
        calls = []
        cs = c.cache_seqlens.to(dev)
        cos, sin = c.rotary_cos.to(dev), c.rotary_sin.to(dev)
        q, kn, vn = c.q.to(dev), c.k_new.to(dev), c.v_new.to(dev)
        for r in range(4):
            kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
            out = torch.empty((8, 1, 32, 128), dtype=q.dtype, device=dev)
            calls.append(E.prepare_kvcache(q, kc, vc, kn, vn, out, rotary_cos=cos, rotary_sin=sin,
                                           cache_seqlens=cs, causal=True,
                                           softmax_scale=c.softmax_scale, rotary_interleaved=False))
        del c
        t = time_loop(calls, K, Wm, torch)
        kv_bytes = sum(L + 1 for L in lens) * 8 * (128 + 128) * 2
        other = (8 * 32 * 128 * 2) * 2 + (8 * 8 * 128 * 2) * 4
        decode = {"workload": "attn_fwd_kvcache decode B=8 Hq=32 Hkv=8 D=128 bf16 cap=8192 "
                              "RoPE rd=128 non-interleaved, seqlens seed 0",
                  "us": t * 1e6, "kv_bytes": kv_bytes, "gbs": kv_bytes / t / 1e9,
                  "gbs_all_bytes": (kv_bytes + other) / t / 1e9,
                  "pct_hbm_peak": 100 * kv_bytes / t / 1e9 / PEAK_HBM_GBS}
        results["decode_gqa"] = decode
        del calls
        torch.cuda.empty_cache()

    # ---------------- chunked prefill: B=4 H=16 D=128 bf16, 512 new tokens, RoPE rd=64 interleaved
    if want("chunked"):
        c = W.chunked_prefill()
        lens = W.seqlens_list(c.cache_seqlens, 4)
        cs = c.cache_seqlens.to(dev)
        cos, sin = c.rotary_cos.to(dev), c.rotary_sin.to(dev)
        calls = []
        for r in range(4):
            q, kn, vn = c.q.to(dev), c.k_new.to(dev), c.v_new.to(dev)
            kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
            out = torch.empty_like(q)
            calls.append(E.prepare_kvcache(q, kc, vc, kn, vn, out, rotary_cos=cos, rotary_sin=sin,
                                           cache_seqlens=cs, causal=True,
                                           softmax_scale=c.softmax_scale, rotary_interleaved=True))
        del c
        t = time_loop(calls, K, Wm, torch)
        fl = 2.0 * 256 * 16 * W.kvcache_pairs(lens, 512, 512, True)
        byt = sum(lens) * 16 * 256 * 2 + 3 * 4 * 512 * 16 * 256 * 2
        results["chunked_prefill"] = {"us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                                      "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS,
                                      "gbs": byt / t / 1e9, "pct_hbm_peak": 100 * byt / t / 1e9 / PEAK_HBM_GBS}
        del calls
        torch.cuda.empty_cache()

    # ---------------- local window: the headline shape with window_size=(256, 256), causal
    if want("window"):
        c = W.fwd_d64(True)
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        out = torch.empty_like(q)
        call = E.prepare_fwd(q, k, v, out, True, c.softmax_scale, window_size=(256, 256))
        t = time_loop([call], K, Wm, torch)
        fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, True, window=(256, 256))
        results["fwd_b2h8s2048d64_causal_window256"] = {
            "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
            "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS}
        del call, q, k, v, out, c

    # ---------------- gradients on the headline shape (dq, dk, dv from dO), non-causal and causal
    if want("bwd"):
        for causal in (False, True):
            c = W.fwd_d64(causal)
            q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
            g = torch.Generator().manual_seed(1)
            dout = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
            out, lse = E.attn_fwd(q, k, v, causal=causal, softmax_scale=c.softmax_scale, return_lse=True)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            call = E.prepare_bwd(dout, q, k, v, out, lse, dq, dk, dv, causal, c.softmax_scale)
            t = time_loop([call], K, Wm, torch)
            fl = W.bwd_flops(2, 2048, 2048, 8, 64, 64, causal)
            results["bwd_b2h8s2048d64" + ("_causal" if causal else "")] = {
                "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS}
            del call, q, k, v, out, lse, dout, dq, dk, dv, c

    # ---------------- packed sequences: the headline token budget (2 x 2048) as 7 seeded lengths
    if want("varlen"):
        lens = W.packed_lengths(4096, 7, seed=0)
        c = W.random_varlen(lens, lens, 8, 8, 64, 64, "fp16", True, seed=0)
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        cq, ck = c.cu_seqlens_q.to(dev), c.cu_seqlens_k.to(dev)
        out = torch.empty_like(q)
        call = E.prepare_varlen(q, k, v, out, cq, ck, c.max_seqlen_q, True, 0.125)
        t = time_loop([call], K, Wm, torch)
        fl = sum(W.fwd_flops(1, n, n, 8, 64, 64, True) for n in lens)
        results["varlen_7seq_4096tok_h8d64_causal"] = {
            "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
            "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS, "lengths": lens}
        del call, q, k, v, out, c

    # ---------------- FP8 (e4m3) inputs on the headline shape, non-causal and causal
    if want("fp8"):
        for causal in (False, True):
            c = W.fwd_fp8_d64(causal)
            q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
            out = torch.empty((2, 2048, 8, 64), dtype=torch.bfloat16, device=dev)
            call = E.prepare_fp8(q, k, v, out, causal, None)
            t = time_loop([call], K, Wm, torch)
            fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, causal)
            results["fwd_fp8_b2h8s2048d64" + ("_causal" if causal else "")] = {
                "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                "pct_blended_peak": 100 * fl / t / 1e12 / PEAK_FP8_BLEND,
                "peak_note": "QK^T on fp8 MFMA, PV on bf16 MFMA: blended peak %.0f TFLOP/s" % PEAK_FP8_BLEND}
            del call, q, k, v, out, c

    # ---------------- asymmetric head dims: B=2 H=16 S=4096 Dqk=192 Dv=128 bf16 causal
    if want("asym"):
        c = W.fwd_asym()
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        out = torch.empty((2, 4096, 16, 128), dtype=q.dtype, device=dev)
        call = E.prepare_fwd(q, k, v, out, True, c.softmax_scale)
        t = time_loop([call], max(5, K // 5), max(2, Wm // 5), torch)
        fl = W.fwd_flops(2, 4096, 4096, 16, 192, 128, True)
        results["fwd_asym_b2h16s4096"] = {"us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                                          "pct_mfma_peak": 100 * fl / t / 1e12 / PEAK_TFLOPS}
        del call, q, k, v, out, c

    # ---------------- empty-cache kvcache (latency only)
    if want("empty"):
        c = W.kvcache_empty()
        q = c.q.to(dev)
        kc, vc = c.k_cache.to(dev), c.v_cache.to(dev)
        out = torch.empty((4, 2, 16, 16), dtype=q.dtype, device=dev)
        call = E.prepare_kvcache(q, kc, vc, q, q, out, cache_seqlens=0)
        t = time_loop([call], K, Wm, torch)
        results["kvcache_empty"] = {"us": t * 1e6}

    # ---------------- plain copy (calibrates the HBM byte counters)
    if args.copy_mib:
        src = torch.empty(args.copy_mib * 2**20 // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        t = time_loop([lambda: dst.copy_(src)], K, Wm, torch)
        results["copy_%dmib" % args.copy_mib] = {"us": t * 1e6, "gbs_read_plus_write":
                                                 2 * args.copy_mib * 2**20 / t / 1e9}
        del src, dst

    # ---------------- roofline entry: the non-causal headline kernel
    t_nc, fl_nc = hl[False]
    roofline = {"kernel": "tile_attn_kernel<F16,64,64,non-causal>", "bound": "mfma",
                "achieved": fl_nc / t_nc / 1e12, "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": fl_nc / t_nc / 1e12 / PEAK_TFLOPS,
                "traffic": traffic_entry("tile_attn_fwd_b2h8s2048d64"),
                "avg_launch_us": t_nc * 1e6,
                "algorithmic": "2*(64+64) flop x 2*8*2048*2048 (query,key) pairs = %.4g GFLOP per launch"
                               % (fl_nc / 1e9)}

    # ---------------- CPU oracle on the headline workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "attn_fwd B=2 H=8 S=2048 D=64 fp16 N(0,1) scale 1/8, "
                               "one non-causal + one causal call per step",
                   "global_batch": 2, "seq_len": 2048, "heads": 8, "head_dim": 64,
                   "parallelism": "single-gpu"},
        "pct_mfma_peak": 100 * value / PEAK_TFLOPS,
        "decode": decode,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": results,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline():
    """The fp64 oracle, as it stands, on the headline step (both masks), repeated to ~10 s."""
    import workloads as W
    from oracle import attention_ref, to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count() or 1
    cases = [W.fwd_d64(False), W.fwd_d64(True)]
    arrs = [(to_f64(c.q), to_f64(c.k), to_f64(c.v), c.causal, c.softmax_scale) for c in cases]
    flops = sum(W.fwd_flops(2, 2048, 2048, 8, 64, 64, c.causal) for c in cases)
    reps, t_tot = 0, 0.0
    while reps < 8 and t_tot < 10.0:
        t0 = time.perf_counter()
        for q, k, v, causal, sc in arrs:
            attention_ref(q, k, v, causal=causal, softmax_scale=sc)
        t_tot += time.perf_counter() - t0
        reps += 1
    return {"value": flops * reps / t_tot / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "full headline step (non-causal + causal attn_fwd, B=2 H=8 S=2048 D=64) "
                      "x%d, fp64 numpy, %.1f s" % (reps, t_tot)}


if __name__ == "__main__":
    main()
