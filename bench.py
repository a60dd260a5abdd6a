#!/usr/bin/env python3
"""Benchmark of the fused softmax / LayerNorm row-reduction hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
    attn_softmax_fw -> attn_softmax_bw -> layernorm_fw -> layernorm_bw
on the GPT-2 training shapes (B=32, T=256, C=256, H=8, fp16 storage, fp32 compute):
softmax over [32, 8, 256, 256] causal scores and LayerNorm over [8192, 256] activations.
``--workload w5`` runs the large encoder-layer shapes instead (softmax [64,16,512,512] with
key padding, LayerNorm [32768,1024]).

The metric is achieved HBM bandwidth: the algorithmic bytes of one step (every tensor read
or written once, dense) divided by the measured step time. Inputs are resident in HBM before
the timed region; the steps rotate over enough copies of every buffer (>= 1 GiB in total) that
the 256 MB Infinity Cache cannot serve a step from the previous pass over the same buffers.

Printed on stdout: ONE JSON line. Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of ~8 TB/s peak) for softmax & LayerNorm fw+bw, fp16"
PEAK_HBM_GBPS = 8000.0
MIN_FOOTPRINT = 1 << 30


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", choices=("w2", "w5"), default="w2")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-ops", action="store_true", help="skip the per-op diagnostic timings")
    return p.parse_args()


def source_digest() -> str:
    """sha256 over the HIP sources: a traffic figure is only reported for the kernels it was
    measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "layernorm_reduction_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only; multi-GPU runs (--gpus N > 1) are not "
              "supported. Rows shard across GPUs with no communication except one 2*C-float "
              "all-reduce of the LayerNorm parameter gradients.", file=sys.stderr)
        sys.exit(2)

    import torch

    import layernorm_reduction_amd as lnr
    from layernorm_reduction_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lnr.load()

    # ---------------------------------------------------------------- workload
    if args.workload == "w2":
        [sc], [lc] = W.workload2()
        wl_name = "GPT-2 training shapes B=32 T=256 C=256 H=8: causal softmax [32,8,256,256] + LayerNorm [8192,256]"
    else:
        sc = W.workload5_softmax(torch.float16)
        lc = W.workload5_layernorm(1024, torch.float16)
        wl_name = "encoder layer: padded softmax [64,16,512,512] + LayerNorm [32768,1024]"
    s = W.dtype_size(sc.dtype)
    b_sfw = W.softmax_fw_bytes(sc.B, sc.H, sc.Tq, sc.Tk, s, has_mask=sc.mask is not None)
    b_sbw = W.softmax_bw_bytes(sc.B, sc.H, sc.Tq, sc.Tk, s)
    b_lfw = W.layernorm_fw_bytes(lc.N, lc.C, s)
    b_lbw = W.layernorm_bw_bytes(lc.N, lc.C, s)
    step_bytes = b_sfw + b_sbw + b_lfw + b_lbw

    per_set = 4 * sc.x.numel() * s + 4 * lc.x.numel() * s
    n_sets = max(2, math.ceil(MIN_FOOTPRINT / per_set))
    log(f"workload {args.workload}: {wl_name}; {step_bytes / 1e6:.1f} MB/step; {n_sets} input sets "
        f"({n_sets * per_set / 2 ** 30:.2f} GiB)")

    sets = []
    ws_bytes = lnr.layernorm_bw_workspace_bytes(lc.N, lc.C, lnr.LNR_F16 if lc.dtype == torch.float16 else lnr.LNR_F32)
    for i in range(n_sets):
        t = {
            "sx": sc.x.to(dev), "sdy": sc.dy.to(dev), "sy": torch.empty_like(sc.x, device=dev),
            "sdx": torch.empty_like(sc.x, device=dev),
            "smask": None if sc.mask is None else sc.mask.to(dev),
            "lx": lc.x.to(dev), "ldy": lc.dy.to(dev), "lg": lc.gamma.to(dev), "lb": lc.beta.to(dev),
            "ly": torch.empty_like(lc.x, device=dev), "ldx": torch.empty_like(lc.x, device=dev),
            "mean": torch.empty(lc.N, dtype=torch.float32, device=dev),
            "rstd": torch.empty(lc.N, dtype=torch.float32, device=dev),
            "dg": torch.empty(lc.C, dtype=lc.dtype, device=dev),
            "db": torch.empty(lc.C, dtype=lc.dtype, device=dev),
            "ws": torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev),
        }
        t["calls"] = (
            lnr.bind_attn_softmax_fw(t["sx"], t["smask"], sc.causal, t["sy"]),
            lnr.bind_attn_softmax_bw(t["sdy"], t["sy"], t["sdx"]),
            lnr.bind_layernorm_fw(t["lx"], t["lg"], t["lb"], lc.eps, t["ly"], t["mean"], t["rstd"]),
            lnr.bind_layernorm_bw(t["ldy"], t["lx"], t["lg"], t["mean"], t["rstd"], t["ldx"], t["dg"],
                                  t["db"], t["ws"]),
        )
        sets.append(t)
    torch.cuda.synchronize()

    def step(i):
        for c in sets[i % n_sets]["calls"]:
            c()

    # ---------------------------------------------------------------- warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # The dominant kernel (softmax backward: 3 tensor passes of the quadratic score tensor)
    # is bracketed by HIP events on the stream it runs on, inside the timed steps.
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        sfw, sbw, lfw, lbw = sets[i % n_sets]["calls"]
        sfw()
        evs[i][0].record()
        sbw()
        evs[i][1].record()
        lfw()
        lbw()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    value = step_bytes * K / elapsed / 1e9
    sbw_ms = [a.elapsed_time(b) for a, b in evs]
    sbw_avg_us = statistics.mean(sbw_ms) * 1e3
    sbw_gbps = b_sbw / (sbw_avg_us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us -> {value:.0f} GB/s ({value / PEAK_HBM_GBPS:.1%} of 8 TB/s); "
        f"softmax_bw {sbw_avg_us:.1f} us -> {sbw_gbps:.0f} GB/s")

    # ---------------------------------------------------------------- diagnostics (untimed)
    ops = {}
    if not args.no_ops:
        names = ("attn_softmax_fw", "attn_softmax_bw", "layernorm_fw", "layernorm_bw")
        nbytes = (b_sfw, b_sbw, b_lfw, b_lbw)
        reps = max(20, min(K, 200))
        for k, (name, nb) in enumerate(zip(names, nbytes)):
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i in range(reps):
                c = sets[i % n_sets]["calls"][k]
                pairs[i][0].record()
                c()
                pairs[i][1].record()
            torch.cuda.synchronize()
            us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
            med = us[len(us) // 2]
            ops[name] = {"bytes": nb, "median_us": round(med, 2), "min_us": round(us[0], 2),
                         "GBps": round(nb / (med * 1e-6) / 1e9, 1),
                         "frac_of_peak": round(nb / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        # streaming copy ceiling: 16-byte loads/stores over 1 GiB
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            lnr.copy_bytes(dst, src)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a, b in pairs:
            a.record()
            lnr.copy_bytes(dst, src)
            b.record()
        torch.cuda.synchronize()
        cus = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)[5]
        ops["copy_1GiB"] = {"bytes": 2 * n, "median_us": round(cus, 1),
                            "GBps": round(2 * n / (cus * 1e-6) / 1e9, 1)}
        del src, dst
        for k, v in ops.items():
            log(f"  {k:16s} {v['median_us']:9.1f} us  {v['GBps']:8.1f} GB/s")

    # ---------------------------------------------------------------- roofline
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_softmax_bw_{args.workload}.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tr = json.load(fh)
        if tr.get("source_sha256") == source_digest():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "kernel": "softmax_bw_vec (attn_softmax_bw)", "achieved": round(sbw_gbps, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(sbw_gbps / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "avg_us": round(sbw_avg_us, 2), "bytes_per_launch": b_sbw}

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the oracle on the host cores")
        if args.workload == "w2":
            xs, dys, ms = sc.x, sc.dy, sc.mask
            xl, dyl = lc.x, lc.dy
            frac = 1.0
            sample = "one whole step: softmax fw+bw [32,8,256,256] and LayerNorm fw+bw [8192,256]"
        else:
            bsub = 8
            xs, dys, ms = sc.x[:bsub], sc.dy[:bsub], None if sc.mask is None else sc.mask[:bsub]
            xl, dyl = lc.x[: lc.N // 8], lc.dy[: lc.N // 8]
            frac = bsub / sc.B
            sample = "1/8 of a step: softmax fw+bw [8,16,512,512] and LayerNorm fw+bw [4096,1024]"
        g64 = lc.gamma
        b64 = lc.beta
        times = []
        t_start = time.perf_counter()
        while True:
            c0 = time.perf_counter()
            y = oracle.softmax_fw(xs, ms, sc.causal)
            oracle.softmax_bw(y, dys)
            del y
            oracle.layernorm_fw(xl, g64, b64, lc.eps)
            oracle.layernorm_bw(xl, dyl, g64, lc.eps)
            times.append(time.perf_counter() - c0)
            if len(times) >= 3 or time.perf_counter() - t_start > 20.0:
                break
        tmed = statistics.median(times)
        cpu = {"value": round(step_bytes * frac / tmed / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
               "kind": "oracle", "sample": sample, "seconds_per_sample": round(tmed, 3),
               "repeats": len(times), "note": "fp64 correctness oracle, not a tuned CPU kernel"}
        log(f"oracle: {tmed:.2f} s per sample on {cpu['cores']} threads -> {cpu['value']} GB/s")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "config": {"workload": wl_name, "storage": "fp16", "compute": "fp32",
                   "softmax": [sc.B, sc.H, sc.Tq, sc.Tk], "causal": sc.causal,
                   "key_padding": sc.mask is not None, "layernorm": [lc.N, lc.C],
                   "bytes_per_step": step_bytes, "input_sets": n_sets, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": ops,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
