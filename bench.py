"""Benchmark: exact attention prefill TFLOP/s and KV-cache decode GB/s on one MI355X.

One JSON line is printed.  ``value`` is the prefill throughput of the largest
configuration that fits one GPU: causal attn_fwd on B=2, H=16, S=4096,
head_dim_qk=192, head_dim_v=128, bf16, N(0,1) inputs, scale 1/sqrt(192)
(flash-attention PR #1604's head sizes); algorithmic work is 2*(Dqk+Dv) flop
per unmasked (query, key) pair, 171.84 GFLOP per call.  A step is one such
call.  The same line carries every other configuration ("configs": the
empty-cache kvcache call, attn_fwd B=2 H=8 S=2048 D=64 fp16 non-causal and
causal, the GQA single-token decode, the chunked prefill) with its own
roofline entry, the extra rows (local window, packed sequences, backward,
FP8 inputs), the peaks re-derived from rocminfo, and the fp64 CPU oracle's
timing together with each configuration's error against it.

GPU time comes from HIP events recorded on the stream the library launches
on (torch's current stream), around back-to-back calls, with inputs already
resident in HBM.  Each timed loop is preceded by 50 ms of the same calls,
untimed (the engine clock ramps up over the first ~10 ms of load), and then
by the requested warmup calls.  After the timed loop of a configuration the
same number of calls runs again, each between its own pair of events, for
the shortest single call ("us_min_per_call"; the mean is "us").  A call
timed alone includes its dispatch latency, which back-to-back calls hide, so
for calls of a few tens of microseconds the minimum can exceed the mean.  The headline, decode and chunked-prefill calls cycle through
input replicas (2, 4 and 4) whose total exceeds the 256 MB Infinity Cache, so
each call reads HBM rather than that cache; the workload-2 calls are timed on one
input (their headline figure) and again over 16 replicas ("us_16_replicas").
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn prefill TFLOP/s + decode KV GB/s at 1 GPU, as % of MI355X peak"
# Published MI355X figures, used when rocminfo is not available.
PUB_CUS, PUB_MHZ = 256, 2400
FLOP_PER_CLK_CU_BF16 = 4096   # v_mfma_f32_32x32x16_bf16: 32768 flop per 32 cycles per SIMD, 4 SIMDs per CU
PEAK_HBM_GBS = 8000.0         # HBM3E, 8 stacks (rocminfo lists no memory bandwidth)

TILE_SRCS = ["exact_attention_qk_amd/csrc/tile_attn.hip", "exact_attention_qk_amd/csrc/device_common.hpp",
             "exact_attention_qk_amd/csrc/attn_args.hpp", "exact_attention_qk_amd/csrc/launchers.hpp"]
DECODE_SRCS = ["exact_attention_qk_amd/csrc/decode_attn.hip", "exact_attention_qk_amd/csrc/device_common.hpp",
               "exact_attention_qk_amd/csrc/attn_args.hpp", "exact_attention_qk_amd/csrc/launchers.hpp"]
# dominant kernel of each configuration: a pattern of its rocprofv3 name, and its sources
DOMINANT = {
    "C5_fwd_asym_b2h16s4096_causal": (r"tile_attn_kernel<attn::BF16, 192, 128, true, false,", TILE_SRCS),
    "C2_fwd_b2h8s2048d64": (r"tile_attn_kernel<attn::F16, 64, 64, false, false,", TILE_SRCS),
    "C2_fwd_b2h8s2048d64_causal": (r"tile_attn_kernel<attn::F16, 64, 64, true, false,", TILE_SRCS),
    "C3_decode_gqa": (r"decode_attn_kernel<attn::BF16, 128, 128, true,", DECODE_SRCS),
    "C4_chunked_prefill": (r"tile_attn_kernel<attn::BF16, 128, 128, true, false,", TILE_SRCS),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of configurations / rows to time besides the headline: "
                         "c1, c2, c3, c4, window, bwd, varlen, fp8 (default: all; 'none': the headline only)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (calibrates the HBM byte counters)")
    ap.add_argument("--summarize", default="",
                    help="print a text summary of a rocprofv3 CSV output directory and exit")
    ap.add_argument("--record-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_MIB"),
                    help="write profiles/traffic.json from a FETCH_SIZE and a WRITE_SIZE rocprofv3 run "
                         "of this script (both with --copy-mib COPY_MIB) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- peaks

def peaks():
    """Compute units and peak engine clock of the gfx950 agent from rocminfo; the dense
    bf16/fp16 MFMA peak follows from the per-CU rate of the instruction set."""
    cus, mhz, src = PUB_CUS, PUB_MHZ, "published (rocminfo unavailable)"
    try:
        txt = subprocess.run(["rocminfo"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True,
                             timeout=60).stdout
        for agent in txt.split("*******")[1:]:
            if "gfx950" not in agent:
                continue
            cu = re.search(r"Compute Unit:\s+(\d+)", agent)
            mc = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
            if cu and mc:
                cus, mhz, src = int(cu.group(1)), int(mc.group(1)), "rocminfo (gfx950 agent)"
                break
    except Exception:
        pass
    mfma = cus * FLOP_PER_CLK_CU_BF16 * mhz * 1e6 / 1e12
    return {"compute_units": cus, "max_clock_mhz": mhz, "source": src,
            "mfma_bf16_tflops": mfma, "mfma_fp8_tflops": 2 * mfma,
            "hbm_gbs": PEAK_HBM_GBS, "hbm_source": "published HBM3E figure"}


# ---------------------------------------------------------------- timing

CLOCK_WARMUP_S = 0.05   # untimed calls before each timed loop: the engine clock ramps up over ~10 ms of load


def time_loop(calls, steps, warmup, torch):
    """Average seconds per call over `steps` back-to-back calls (cycling through `calls`),
    from HIP events on the stream the calls enqueue on.  Before the `warmup` calls, the
    same calls run untimed for CLOCK_WARMUP_S so that the device is at its working clock."""
    n = len(calls)
    t0, i = time.perf_counter(), 0
    while True:
        calls[i % n]()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= CLOCK_WARMUP_S:
                break
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


def min_per_call(calls, steps, torch):
    """Shortest single call (seconds) over `steps` calls cycling through `calls`, each
    bracketed by its own pair of HIP events on the current stream (run right after a
    time_loop of the same calls, so the device is warm)."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(st)
        calls[i % len(calls)]()
        e1.record(st)
    torch.cuda.synchronize()
    return min(e0.elapsed_time(e1) for e0, e1 in evs) / 1e3


def mfma_entry(name, fl, t, pk, kernel):
    a = fl / t / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": a, "peak": pk["mfma_bf16_tflops"], "unit": "TFLOP/s",
            "frac": a / pk["mfma_bf16_tflops"], "traffic": traffic_entry(name), "avg_launch_us": t * 1e6}


# ---------------------------------------------------------------- rocprofv3 helpers

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
            print(k[:140])
            for cn, v in sorted(cs.items()):
                print("    %-32s %16.6g   (dispatches: %d)" % (cn, sum(v) / len(v), len(v)))


def _counter_means(d, counter):
    import csv
    import glob
    from collections import defaultdict
    acc = defaultdict(list)
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def sources_sha256(paths):
    """One digest over the given source files (a kernel file and the headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(p.encode())
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def record_traffic(fetch_dir, write_dir, copy_mib):
    """HBM bytes per launch of each configuration's dominant kernel: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what they read for an elementwise pass
    over copy_mib MiB (which reads and writes exactly that many bytes)."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cp = [k for k in fetch if "neg_kernel" in k]
    assert len(cp) == 1, "no calibration pass in the FETCH_SIZE run (run it with --copy-mib)"
    moved_kib = int(copy_mib) * 1024.0
    fs, ws = moved_kib / fetch[cp[0]], moved_kib / write[cp[0]]
    out = {"_calibration": {"copy_mib": int(copy_mib), "fetch_scale": fs, "write_scale": ws}}
    for name, (pat, srcs) in DOMINANT.items():
        ks = sorted({k for k in fetch if re.search(pat, k)})
        if len(ks) != 1 or ks[0] not in write:
            continue
        k = ks[0]
        out[name] = {"kernel": k, "sources": srcs, "sources_sha256": sources_sha256(srcs),
                     "fetch_kib_per_dispatch": fetch[k], "write_kib_per_dispatch": write[k],
                     "hbm_bytes_per_launch": 1024.0 * (fetch[k] * fs + write[k] * ws)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out, indent=1))


def traffic_entry(name):
    """Measured HBM bytes per launch of a configuration's dominant kernel, if its
    sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(name)
    if not rec:
        return None
    srcs = rec.get("sources", [])
    if not srcs or not all(os.path.exists(os.path.join(ROOT, p)) for p in srcs):
        return None
    if sources_sha256(srcs) != rec["sources_sha256"]:
        return None
    return rec["hbm_bytes_per_launch"]


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
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
    pk = peaks()
    configs, rows, outputs = {}, {}, {}

    def want(name):
        return not only or name in only   # "none" matches nothing

    # ---------------- C1: empty-cache kvcache (latency only)
    if want("c1"):
        c1 = W.kvcache_empty()
        q = c1.q.to(dev)
        kc, vc = c1.k_cache.to(dev), c1.v_cache.to(dev)
        out = torch.empty((4, 2, 16, 16), dtype=q.dtype, device=dev)
        call = E.prepare_kvcache(q, kc, vc, q, q, out, cache_seqlens=0)
        t = time_loop([call], K, Wm, torch)
        configs["C1_kvcache_empty"] = {"us": t * 1e6, "us_min_per_call": min_per_call([call], K, torch) * 1e6,
                                       "bound": "latency"}
        outputs["C1_kvcache_empty"] = out.cpu()

    # ---------------- C2: attn_fwd B=2 H=8 S=2048 D=64 fp16, non-causal and causal
    if want("c2"):
        for causal in (False, True):
            c2 = W.fwd_d64(causal)
            q, k, v = c2.q.to(dev), c2.k.to(dev), c2.v.to(dev)
            out = torch.empty_like(q)
            call = E.prepare_fwd(q, k, v, out, causal, c2.softmax_scale)
            t = time_loop([call], K, Wm, torch)
            t_min = min_per_call([call], K, torch)
            # the same call over 16 input replicas (16 x 16.8 MB > the 256 MB Infinity
            # Cache): each call then reads q, k, v from HBM
            reps = []
            for r in range(16):
                qr, kr, vr = c2.q.to(dev), c2.k.to(dev), c2.v.to(dev)
                reps.append(E.prepare_fwd(qr, kr, vr, torch.empty_like(qr), causal, c2.softmax_scale))
            t_rot = time_loop(reps, K, Wm, torch)
            del reps, qr, kr, vr
            fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, causal)
            nm = "C2_fwd_b2h8s2048d64" + ("_causal" if causal else "")
            configs[nm] = {"us": t * 1e6, "us_min_per_call": t_min * 1e6, "us_16_replicas": t_rot * 1e6,
                           "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                           "pct_mfma_peak": 100 * fl / t / 1e12 / pk["mfma_bf16_tflops"],
                           "roofline": mfma_entry(nm, fl, t, pk, "tile_attn_kernel<F16,64,64,%s>"
                                                  % ("causal" if causal else "non-causal"))}
            outputs[nm] = out.cpu()
            del call, q, k, v, out

    # ---------------- C3: decode, GQA 32/8, D=128, bf16, RoPE rd=128, cache 8192 (4 replicas)
    if want("c3"):
        c3 = W.decode_gqa()
        lens = W.seqlens_list(c3.cache_seqlens, 8)
        cs = c3.cache_seqlens.to(dev)
        cos, sin = c3.rotary_cos.to(dev), c3.rotary_sin.to(dev)
        q, kn, vn = c3.q.to(dev), c3.k_new.to(dev), c3.v_new.to(dev)
        calls, calls_nc, outs = [], [], []
        for r in range(4):
            kc, vc = c3.k_cache.to(dev), c3.v_cache.to(dev)
            out = torch.empty((8, 1, 32, 128), dtype=q.dtype, device=dev)
            for causal, lst in ((True, calls), (False, calls_nc)):
                lst.append(E.prepare_kvcache(q, kc, vc, kn, vn, out, rotary_cos=cos, rotary_sin=sin,
                                             cache_seqlens=cs, causal=causal,
                                             softmax_scale=c3.softmax_scale, rotary_interleaved=False))
            outs.append(out)
        # the same call with causal off (one query token: the same keys are visible), then the
        # headline decode figure with causal on, which leaves outs[0] with its output
        t_nc = time_loop(calls_nc, K, Wm, torch)
        t = time_loop(calls, K, Wm, torch)
        t_min = min_per_call(calls, K, torch)
        del calls_nc
        kv_bytes = sum(L + 1 for L in lens) * 8 * (128 + 128) * 2
        other = (8 * 32 * 128 * 2) * 2 + (8 * 8 * 128 * 2) * 4
        a = kv_bytes / t / 1e9
        configs["C3_decode_gqa"] = {
            "us": t * 1e6, "us_min_per_call": t_min * 1e6, "us_noncausal": t_nc * 1e6, "kv_bytes": kv_bytes,
            "gbs": a,
            "gbs_all_bytes": (kv_bytes + other) / t / 1e9,
            "pct_hbm_peak": 100 * a / pk["hbm_gbs"], "seqlens": lens,
            "roofline": {"kernel": "decode_attn_kernel<BF16,128,128> + split_merge_kernel (whole call)",
                         "bound": "hbm", "achieved": a, "peak": pk["hbm_gbs"], "unit": "GB/s",
                         "frac": a / pk["hbm_gbs"], "traffic": traffic_entry("C3_decode_gqa"),
                         "avg_launch_us": t * 1e6}}
        outputs["C3_decode_gqa"] = outs[0].cpu()
        del calls, outs, kc, vc
        torch.cuda.empty_cache()

    # ---------------- C4: chunked prefill B=4 H=16 D=128 bf16, 512 new tokens, RoPE rd=64 interleaved
    if want("c4"):
        c4 = W.chunked_prefill()
        lens = W.seqlens_list(c4.cache_seqlens, 4)
        cs = c4.cache_seqlens.to(dev)
        cos, sin = c4.rotary_cos.to(dev), c4.rotary_sin.to(dev)
        calls, outs = [], []
        for r in range(4):
            q, kn, vn = c4.q.to(dev), c4.k_new.to(dev), c4.v_new.to(dev)
            kc, vc = c4.k_cache.to(dev), c4.v_cache.to(dev)
            out = torch.empty_like(q)
            calls.append(E.prepare_kvcache(q, kc, vc, kn, vn, out, rotary_cos=cos, rotary_sin=sin,
                                           cache_seqlens=cs, causal=True,
                                           softmax_scale=c4.softmax_scale, rotary_interleaved=True))
            outs.append(out)
        t = time_loop(calls, K, Wm, torch)
        t_min = min_per_call(calls, K, torch)
        fl = 2.0 * 256 * 16 * W.kvcache_pairs(lens, 512, 512, True)
        byt = sum(lens) * 16 * 256 * 2 + 3 * 4 * 512 * 16 * 256 * 2
        a = fl / t / 1e12
        configs["C4_chunked_prefill"] = {
            "us": t * 1e6, "us_min_per_call": t_min * 1e6, "gflop": fl / 1e9, "tflops": a,
            "pct_mfma_peak": 100 * a / pk["mfma_bf16_tflops"], "bytes": byt, "gbs": byt / t / 1e9, "pct_hbm_peak": 100 * byt / t / 1e9 / pk["hbm_gbs"],
            "seqlens": lens,
            "roofline": {"kernel": "rope append + tile_attn_kernel<BF16,128,128,causal> (whole call)",
                         "bound": "mfma", "achieved": a, "peak": pk["mfma_bf16_tflops"], "unit": "TFLOP/s",
                         "frac": a / pk["mfma_bf16_tflops"], "traffic": traffic_entry("C4_chunked_prefill"),
                         "avg_launch_us": t * 1e6, "hbm_frac": byt / t / 1e9 / pk["hbm_gbs"]}}
        outputs["C4_chunked_prefill"] = outs[0].cpu()
        del calls, outs, q, kn, vn, kc, vc
        torch.cuda.empty_cache()

    # ---------------- extra rows
    if want("window"):
        c = W.fwd_d64(True)
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        out = torch.empty_like(q)
        call = E.prepare_fwd(q, k, v, out, True, c.softmax_scale, window_size=(256, 256))
        t = time_loop([call], K, Wm, torch)
        fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, True, window=(256, 256))
        rows["fwd_b2h8s2048d64_causal_window256"] = {
            "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
            "pct_mfma_peak": 100 * fl / t / 1e12 / pk["mfma_bf16_tflops"]}
        del call, q, k, v, out, c

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
            rows["bwd_b2h8s2048d64" + ("_causal" if causal else "")] = {
                "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                "pct_mfma_peak": 100 * fl / t / 1e12 / pk["mfma_bf16_tflops"]}
            del call, q, k, v, out, lse, dout, dq, dk, dv, c

    if want("varlen"):
        lens = W.packed_lengths(4096, 7, seed=0)
        c = W.random_varlen(lens, lens, 8, 8, 64, 64, "fp16", True, seed=0)
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        cq, ck = c.cu_seqlens_q.to(dev), c.cu_seqlens_k.to(dev)
        out = torch.empty_like(q)
        call = E.prepare_varlen(q, k, v, out, cq, ck, c.max_seqlen_q, True, 0.125)
        t = time_loop([call], K, Wm, torch)
        fl = sum(W.fwd_flops(1, n, n, 8, 64, 64, True) for n in lens)
        rows["varlen_7seq_4096tok_h8d64_causal"] = {
            "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
            "pct_mfma_peak": 100 * fl / t / 1e12 / pk["mfma_bf16_tflops"], "lengths": lens}
        del call, q, k, v, out, c

    if want("fp8"):
        blend = 1.0 / (0.5 / pk["mfma_fp8_tflops"] + 0.5 / pk["mfma_bf16_tflops"])
        for causal in (False, True):
            c = W.fwd_fp8_d64(causal)
            q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
            out = torch.empty((2, 2048, 8, 64), dtype=torch.bfloat16, device=dev)
            call = E.prepare_fp8(q, k, v, out, causal, None)
            t = time_loop([call], K, Wm, torch)
            fl = W.fwd_flops(2, 2048, 2048, 8, 64, 64, causal)
            rows["fwd_fp8_b2h8s2048d64" + ("_causal" if causal else "")] = {
                "us": t * 1e6, "gflop": fl / 1e9, "tflops": fl / t / 1e12,
                "pct_blended_peak": 100 * fl / t / 1e12 / blend,
                "peak_note": "Q K^T on fp8 MFMA, P V on bf16 MFMA: blended peak %.0f TFLOP/s" % blend}
            del call, q, k, v, out, c

    # ---------------- C5 (headline): causal B=2 H=16 S=4096 Dqk=192 Dv=128 bf16, 2 replicas.
    # Timed after the other configurations, so that the device runs at its
    # working clocks (the first milliseconds of a process run slower).
    c = W.fwd_asym()
    calls, outs = [], []
    for r in range(2):
        q, k, v = c.q.to(dev), c.k.to(dev), c.v.to(dev)
        out = torch.empty((2, 4096, 16, 128), dtype=q.dtype, device=dev)
        calls.append(E.prepare_fwd(q, k, v, out, True, c.softmax_scale))
        outs.append(out)
    t5_one = time_loop(calls[:1], K, Wm, torch)
    t5 = time_loop(calls, K, Wm, torch)
    t5_min = min_per_call(calls, K, torch)
    fl5 = W.fwd_flops(2, 4096, 4096, 16, 192, 128, True)
    name5 = "C5_fwd_asym_b2h16s4096_causal"
    configs[name5] = {"us": t5 * 1e6, "us_min_per_call": t5_min * 1e6, "us_same_inputs": t5_one * 1e6,
                      "gflop": fl5 / 1e9,
                      "tflops": fl5 / t5 / 1e12, "pct_mfma_peak": 100 * fl5 / t5 / 1e12 / pk["mfma_bf16_tflops"],
                      "roofline": mfma_entry(name5, fl5, t5, pk, "tile_attn_kernel<BF16,192,128,causal>")}
    outputs[name5] = outs[0].cpu()
    del calls, outs, q, k, v, out
    torch.cuda.empty_cache()

    if args.copy_mib:
        # an elementwise pass (torch.neg) that reads and writes exactly copy_mib MiB, under a
        # kernel name of its own (input uploads use the runtime's copy kernel)
        src = torch.zeros(args.copy_mib * 2**20 // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        t = time_loop([lambda: torch.neg(src, out=dst)], K, Wm, torch)
        rows["copy_%dmib" % args.copy_mib] = {"us": t * 1e6,
                                              "gbs_read_plus_write": 2 * args.copy_mib * 2**20 / t / 1e9}
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(outputs)

    h = configs[name5]
    line = {
        "metric": METRIC, "value": h["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": t5 * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "attn_fwd causal B=2 H=16 S=4096 head_dim_qk=192 head_dim_v=128 bf16, "
                               "q/k/v N(0,1) seed 0, scale 1/sqrt(192); one call per step, 2 input replicas",
                   "global_batch": 2, "seq_len": 4096, "heads": 16, "head_dim_qk": 192, "head_dim_v": 128,
                   "parallelism": "single-gpu"},
        "pct_mfma_peak": h["pct_mfma_peak"],
        "clock_warmup_s": CLOCK_WARMUP_S,
        "roofline": dict(h["roofline"], algorithmic="2*(192+128) flop x 2*16*4096*4097/2 unmasked (query,key) "
                                                    "pairs = %.5g GFLOP per launch" % (fl5 / 1e9)),
        "decode": configs.get("C3_decode_gqa"),
        "peaks": pk,
        "cpu_baseline": cpu,
        "configs": configs,
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------- CPU oracle leg

def _ulp(ref, dtype):
    """Spacing of the target format at each reference value (normal range; subnormals
    share the smallest normal's spacing)."""
    import numpy as np
    mant, emin = (10, -14) if dtype == "fp16" else (7, -126)
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - mant)


def _errors(got, ref, dtype):
    import numpy as np
    from oracle import to_f64
    g = to_f64(got.float())
    d = np.abs(g - ref)
    u = d / _ulp(ref, dtype)
    return {"max_abs_err": float(d.max()), "max_ulp_err": float(u.max()),
            "p999_ulp_err": float(np.quantile(u, 0.999)), "frac_within_1ulp": float((u <= 1.0).mean()),
            "elements": int(d.size)}


def cpu_baseline(outputs):
    """The fp64 oracle, as it stands, timed on this host on every configuration the
    run timed (each once, whole), and compared with the GPU output of that run."""
    import numpy as np
    import torch
    import workloads as W
    from oracle import attention_ref, kvcache_ref, to_f64
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:
        cores = os.cpu_count() or 1
    per = {}

    def fwd(name, case, fl):
        qf, kf, vf = to_f64(case.q), to_f64(case.k), to_f64(case.v)
        t0 = time.perf_counter()
        ref, _ = attention_ref(qf, kf, vf, causal=case.causal, softmax_scale=case.softmax_scale)
        dt = time.perf_counter() - t0
        per[name] = dict(_errors(outputs[name], ref, case.dtype), oracle_s=dt, oracle_tflops=fl / dt / 1e12)

    def kv(name, case, work_key, work):
        B = case.q.shape[0]
        lens = W.seqlens_list(case.cache_seqlens, B)
        f = to_f64
        args = (f(case.q), f(case.k_cache), f(case.v_cache), f(case.k_new), f(case.v_new),
                lens if isinstance(case.cache_seqlens, torch.Tensor) else case.cache_seqlens)
        kw = dict(dtype=case.dtype, rotary_interleaved=case.rotary_interleaved, causal=case.causal,
                  softmax_scale=case.softmax_scale,
                  rotary_cos=None if case.rotary_cos is None else f(case.rotary_cos),
                  rotary_sin=None if case.rotary_sin is None else f(case.rotary_sin))
        t0 = time.perf_counter()
        ref = kvcache_ref(*args, **kw)[0]
        dt = time.perf_counter() - t0
        e = dict(_errors(outputs[name], ref, case.dtype), oracle_s=dt)
        if work_key:
            e[work_key] = work / dt
        per[name] = e

    name5 = "C5_fwd_asym_b2h16s4096_causal"
    fl5 = W.fwd_flops(2, 4096, 4096, 16, 192, 128, True)
    fwd(name5, W.fwd_asym(), fl5)
    for causal in (False, True):
        nm = "C2_fwd_b2h8s2048d64" + ("_causal" if causal else "")
        if nm in outputs:
            fwd(nm, W.fwd_d64(causal), W.fwd_flops(2, 2048, 2048, 8, 64, 64, causal))
    if "C1_kvcache_empty" in outputs:
        c1 = W.kvcache_empty()
        kv("C1_kvcache_empty", c1, None, 0)
    if "C3_decode_gqa" in outputs:
        c3 = W.decode_gqa()
        lens = W.seqlens_list(c3.cache_seqlens, 8)
        kv("C3_decode_gqa", c3, "oracle_kv_gbs", sum(L + 1 for L in lens) * 8 * 256 * 2 / 1e9)
    if "C4_chunked_prefill" in outputs:
        c4 = W.chunked_prefill()
        lens = W.seqlens_list(c4.cache_seqlens, 4)
        kv("C4_chunked_prefill", c4, "oracle_tflops", 2.0 * 256 * 16 * W.kvcache_pairs(lens, 512, 512, True) / 1e12)
    h = per[name5]
    return {"value": fl5 / h["oracle_s"] / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "the whole headline call (causal B=2 H=16 S=4096 Dqk=192 Dv=128), once, fp64 numpy, "
                      "%.1f s; every other configuration once in per_config" % h["oracle_s"],
            "per_config": per}


if __name__ == "__main__":
    main()
