#!/usr/bin/env python3
"""Benchmark of the fused softmax / LayerNorm row-reduction hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the large
encoder-layer training shapes (LightSeq's max_seq_len 512, fp16 storage, fp32 compute):
    attn_softmax_fw -> attn_softmax_bw   on [64, 16, 512, 512] scores with key padding,
    layernorm_fw -> layernorm_bw         on [32768, 1024] activations,
    layernorm_fw -> layernorm_bw         on [32768, 4096] activations.
The same shapes are repeated in fp32 storage (reported under "fp32_repeat", not part of the
step). ``--workload w2`` runs the GPT-2 training shapes instead (B=32, T=256, C=256, H=8:
causal softmax over [32, 8, 256, 256] and LayerNorm over [8192, 256]).

The metric is achieved HBM bandwidth: the algorithmic bytes of one step (every tensor read
or written once, dense) divided by the measured step time. Inputs are resident in HBM before
the timed region; the steps rotate over enough copies of every buffer (>= 1 GiB in total) that
the 256 MB Infinity Cache cannot serve a step from the previous pass over the same buffers.
The GPU idles for seconds while the host builds those inputs; before the warm-up steps the
step runs untimed for PREWARM_S seconds so that the timed steps start at steady clocks
(reported under "prewarm"; the warm-up and timed step counts are exactly the ones asked for).

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
PREWARM_S = 0.25


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--workload", choices=("w2", "w5"), default="w5")
    p.add_argument("--sample-every", type=int, default=8, metavar="S",
                   help="time the dominant kernel's own duration on every S-th timed step (each "
                        "timed launch goes through hipExtLaunchKernel with two events, which "
                        "costs a few microseconds of step time; sampling keeps that out of the "
                        "throughput)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-ops", action="store_true", help="skip the per-op diagnostic timings")
    p.add_argument("--table", action="store_true",
                   help="time every op at every workload shape (row-length sweep, hidden-size sweep, "
                        "encoder layer fp16/fp32); one JSON line per case")
    p.add_argument("--warm-cache", action="store_true",
                   help="with --table: reuse one input set per case (tensors may be served from the "
                        "Infinity Cache); reported as warm-cache figures, not against the target")
    p.add_argument("--match", default="", metavar="TEXT",
                   help="with --table: only the cases whose name contains TEXT")
    p.add_argument("--cpu-table", action="store_true",
                   help="CPU only: time the oracle's fw+bw on the tiny, GPT-2 and hidden-size-sweep "
                        "shapes with all host threads and with one thread; one JSON line per case")
    p.add_argument("--skip-traffic", action="store_true",
                   help="run the dense and the read-skipping softmax kernels on three masked "
                        "workloads (plus the 1 GiB calibration copy) for counter collection; one "
                        "JSON line per case with the analytic bytes of both")
    p.add_argument("--summarize-skip-traffic", metavar="DIR",
                   help="CPU only: read pmc_fetch_skip/ and pmc_write_skip/ under DIR and the "
                        "--skip-traffic output DIR/skip_traffic.jsonl; write "
                        "profiles/softmax_skip_traffic.md")
    p.add_argument("--summarize-table-trace", metavar="DIR",
                   help="CPU only: read DIR/prof_table/table_kernel_trace.csv and the table's JSON lines "
                        "DIR/table_prof.jsonl; write profiles/table_kernel_trace.md (rocprofv3 kernel "
                        "durations and achieved GB/s per case)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="CPU only: read the rocprofv3 outputs under DIR (prof_<w>/, pmc_fetch_<w>/, "
                        "pmc_write_<w>/) and write the summaries under profiles/")
    return p.parse_args()


TRACE_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
             "-d $OUT/prof_{w} -o {w} -- python3 $REPO/bench.py{args}")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc {ctr} -f csv "
           "-d $OUT/pmc_{kind}_{w} -o {w} -- python3 $REPO/bench.py{args}")
DOMINANT = "softmax_bw_vec"
COPY = "copy16"
# Work-items of the 1 GiB calibration copy (`lnr_copy` moves one 16-byte vector per thread);
# the same kernel also times the same-size ceilings, so counters keep only this launch.
CALIB_GRID = (1 << 30) // 16
SKIP_PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc {ctr} -f csv "
                "-d $OUT/pmc_{kind}_skip -o skip -- python3 $REPO/bench.py --skip-traffic")


def skip_traffic_cases():
    """(name, B, H, T, dtype, causal, padded): the GPT-2 causal scores, a row-length-sweep shape
    with causal and padding masks, and the padded encoder shape."""
    import torch
    return [("w2 [32,8,256,256] causal", 32, 8, 256, torch.float16, True, False),
            ("w3 [16,8,1024,1024] causal padded", 16, 8, 1024, torch.float16, True, True),
            ("w5 [64,16,512,512] padded", 64, 16, 512, torch.float16, False, True)]


def run_skip_traffic():
    """Dense and skipping softmax kernels, 3 launches each per case, after the 1 GiB streaming
    copy that calibrates the counters. Padded masks keep the first 3/4 of the keys."""
    import torch
    import layernorm_reduction_amd as lnr
    from layernorm_reduction_amd import workloads as W

    dev = torch.device("cuda:0")
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        lnr.copy_bytes(b, a)
    torch.cuda.synchronize()
    del a, b
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    for name, B, H, T, dt, causal, padded in skip_traffic_cases():
        x = torch.randn(B, H, T, T, device=dev, dtype=dt, generator=g)
        dy = torch.randn_like(x)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        m = None
        if padded:
            m = torch.zeros(B, T, device=dev, dtype=dt)
            m[:, T * 3 // 4:] = float("-inf")
        for _ in range(3):
            lnr.attn_softmax_fw(x, m, causal, out=y)
            lnr.attn_softmax_bw(dy, y, dinp=dx)
            lnr.attn_softmax_fw_skip(x, m, causal, out=y)
            lnr.attn_softmax_bw_skip(dy, y, m, causal, dinp=dx)
        torch.cuda.synchronize()
        s = W.dtype_size(dt)
        sf, sb = W.softmax_skip_bytes(m.cpu() if m is not None else None, causal, B, H, T, T, s)
        print(json.dumps({"case": name, "grid_rows": B * H * T,
                          "dense_fw_bytes": W.softmax_fw_bytes(B, H, T, T, s, has_mask=padded),
                          "dense_bw_bytes": W.softmax_bw_bytes(B, H, T, T, s),
                          "skip_fw_bytes": sf, "skip_bw_bytes": sb}), flush=True)
        log(f"skip traffic: {name} done")
        del x, dy, y, dx, m
        torch.cuda.empty_cache()


def summarize_skip_traffic(root_dir: str):
    """profiles/softmax_skip_traffic.md: FETCH_SIZE / WRITE_SIZE per dispatch of the dense and
    skipping softmax kernels (scaled by the 1 GiB copy), beside the analytic bytes."""
    import csv
    import collections

    calib_grid = str(CALIB_GRID)

    def per_kernel(kind):
        path = os.path.join(root_dir, f"pmc_{kind}_skip", "skip_counter_collection.csv")
        by = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if COPY in r["Kernel_Name"] and r["Grid_Size"] != calib_grid:
                continue
            by[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
        return {k: statistics.mean(v) for k, v in by.items()}

    fetch, write = per_kernel("fetch"), per_kernel("write")
    pick = lambda d, key: next(v for k, v in d.items() if key in k)
    f_scale = float(1 << 30) / pick(fetch, COPY)
    w_scale = float(1 << 30) / pick(write, COPY)
    cases = [json.loads(l) for l in open(os.path.join(root_dir, "skip_traffic.jsonl")) if l.startswith("{")]
    rows = ["# HBM traffic of the read-skipping softmax kernels\n",
            "Commands (each counter in a run of its own; the analytic bytes come from the same "
            "program's output; $REPO = the repository root, $OUT = the directory the profiler "
            "writes to):\n", "```",
            SKIP_PMC_CMD.format(ctr="FETCH_SIZE", kind="fetch"),
            SKIP_PMC_CMD.format(ctr="WRITE_SIZE", kind="write"), "```\n",
            f"Scale: the 1 GiB streaming copy reads {pick(fetch, COPY) / 2**20:.1f} MiB by FETCH_SIZE "
            f"and writes {pick(write, COPY) / 2**20:.1f} MiB by WRITE_SIZE; fetch counts are multiplied "
            f"by {f_scale:.4f}, write counts by {w_scale:.4f}. Padded masks keep the first 3/4 of the "
            f"keys. Each case runs its own (G, IT) instantiation, so each kernel name is one case.\n",
            "| kernel | fetch MB (scaled) | write MB (scaled) | total MB |", "|---|---|---|---|"]
    for k in fetch:
        if "softmax" in k and k in write:
            fb, wb = fetch[k] * f_scale, write[k] * w_scale
            rows.append(f"| `{k[:90]}` | {fb / 1e6:.3f} | {wb / 1e6:.3f} | {(fb + wb) / 1e6:.3f} |")
    rows += ["", "Analytic bytes per launch (dense: every element read and written once; skipping: "
             "the runs holding an open key read, every element written, the mask once):\n",
             "| case | dense fw MB | skip fw MB | dense bw MB | skip bw MB |", "|---|---|---|---|---|"]
    for c in cases:
        rows.append(f"| {c['case']} | {c['dense_fw_bytes'] / 1e6:.3f} | {c['skip_fw_bytes'] / 1e6:.3f} | "
                    f"{c['dense_bw_bytes'] / 1e6:.3f} | {c['skip_bw_bytes'] / 1e6:.3f} |")
    with open(os.path.join(ROOT, "profiles", "softmax_skip_traffic.md"), "w") as fh:
        fh.write("\n".join(rows) + "\n")


TABLE_TRACE_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace -f csv -d $OUT/prof_table "
                   "-o table -- python3 $REPO/bench.py --table > $OUT/table_prof.jsonl")


def summarize_table_trace(root_dir: str):
    """profiles/table_kernel_trace.md: each table case's kernels as rocprofv3 timed them.

    The dispatches are taken in order. The table's warm-up copies come first; after that every
    case ends with its same-size ceiling launches (the copy and read-two-write-one helpers), so
    the dispatches between two such blocks are one case, matched to the table's JSON lines in
    order. Within a case each kernel's median duration over all its dispatches is taken (the
    table also runs each operation once per input set while it prepares the calls); an
    operation's time is its kernel's, plus its column-sum or finish kernel where it has one."""
    import csv

    trace = os.path.join(root_dir, "prof_table", "table_kernel_trace.csv")
    rows = sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"]))
    recs = [json.loads(l) for l in open(os.path.join(root_dir, "table_prof.jsonl")) if l.startswith("{")]
    helper = lambda n: COPY in n or "xor16" in n
    blocks, cur, i = [], [], 0
    while i < len(rows) and helper(rows[i]["Kernel_Name"]):
        i += 1                                    # warm-up copies
    for r in rows[i:]:
        n = r["Kernel_Name"]
        if helper(n):
            if cur:
                blocks.append(cur)
                cur = []
            continue
        if "lnr" not in n:
            continue                              # not this library's (torch's input generation)
        cur.append((n, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    if cur:
        blocks.append(cur)
    if len(blocks) != len(recs):
        raise SystemExit(f"{len(blocks)} traced cases against {len(recs)} table records")
    lines = ["# rocprofv3 kernel durations of every table case\n",
             "Command ($REPO = the repository root, $OUT = the directory the profiler writes to):\n",
             "```", TABLE_TRACE_CMD, "```\n",
             "Median kernel durations under the tracer (no launch gaps), and the achieved GB/s of the "
             "algorithmic bytes over them. For the read-skipping rows the bytes are those the kernels "
             "move, and the dense kernels' durations on the same inputs are listed beside them.\n",
             "| case | fw µs | bw µs | fw GB/s | bw GB/s | fw+bw GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for rec, blk in zip(recs, blocks):
        durs, order = {}, []
        for n, d in blk:
            if n not in durs:
                durs[n] = []
                order.append(n)
            durs[n].append(d)
        med = {n: statistics.median(v) for n, v in durs.items()}
        # second kernels of two-kernel operations belong with their first kernel
        fin = sum(med[n] for n in order if "finish" in n)
        col = sum(med[n] for n in order if "colsum" in n)
        prim = [n for n in order if "finish" not in n and "colsum" not in n]
        if any("skip" in n for n in prim):
            pick = lambda key: next(n for n in prim if key in n)
            tf, tb = med[pick("fw_skip")], med[pick("bw_skip")]
            extra = f" (dense {med[pick('softmax_fw_vec')]:.1f} / {med[pick('softmax_bw_vec')]:.1f} µs)"
        else:
            fw_n = next(n for n in prim if "fw" in n)
            bw_n = next(n for n in prim if "bw" in n)
            tf, tb = med[fw_n] + fin, med[bw_n] + col
            extra = ""
        bf, bb = rec["bytes_fw"], rec["bytes_bw"]
        gf, gb, gfb = bf / tf * 1e-3, bb / tb * 1e-3, (bf + bb) / (tf + tb) * 1e-3
        lines.append(f"| {rec['case']}{extra} | {tf:.1f} | {tb:.1f} | {gf:.0f} | {gb:.0f} | {gfb:.0f} | "
                     f"{gfb / PEAK_HBM_GBPS:.0%} |")
    with open(os.path.join(ROOT, "profiles", "table_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


def summarize_profiles(root_dir: str, workload: str):
    """Write profiles/<workload>_kernel_trace.md from the kernel-trace statistics and, when the
    two counter runs are present, profiles/<workload>_traffic.md plus the machine-readable
    profiles/traffic_softmax_bw_<workload>.json that the benchmark reports as roofline.traffic
    (only while the HIP sources still hash to the value recorded there)."""
    import csv
    import collections

    args = (" --workload w2" if workload == "w2" else "") + " --steps 20 --warmup 5 --no-cpu-baseline"
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    stats = os.path.join(root_dir, f"prof_{workload}", f"{workload}_kernel_stats.csv")
    lines = [f"# Kernel trace: {workload} benchmark\n",
             "Command ($REPO = the repository root, $OUT = the directory the profiler writes to):\n",
             "```", TRACE_CMD.format(w=workload, args=args), "```\n"]
    def roofline_of(path):
        if os.path.exists(path):
            for line in open(path):
                if line.startswith("{") and '"roofline"' in line:
                    return json.loads(line)["roofline"]
        return None

    live = roofline_of(os.path.join(root_dir, f"bench_{workload}.json"))
    under = roofline_of(os.path.join(root_dir, f"prof_{workload}.log"))
    if live:
        lines.append(f"The same command run without the profiler (same sources): `{DOMINANT}` averages "
                     f"{live['avg_us']} us over {live.get('launches', '?')} timed launches (HIP events "
                     f"recorded by the kernel itself), {live['achieved']} GB/s, {live['frac']:.1%} of "
                     f"8 TB/s.\n")
    if under:
        lines.append(f"Under the profiler the bench's own events read {under['avg_us']} us: the tracer adds "
                     f"work to every dispatch between the recorded start and the kernel, so the table "
                     f"below, not that figure, is the profiled duration.\n")
    lines += ["| kernel | calls | average us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats)):
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    with open(os.path.join(out_dir, f"{workload}_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    calib_grid = str(CALIB_GRID)

    def per_kernel(kind):
        path = os.path.join(root_dir, f"pmc_{kind}_{workload}", f"{workload}_counter_collection.csv")
        if not os.path.exists(path):
            return None
        by = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if COPY in name:  # the same kernel also measures same-size ceilings: keep 1 GiB only
                if r["Grid_Size"] != calib_grid:
                    continue
            by[name].append(float(r["Counter_Value"]) * 1024.0)  # KiB -> bytes
        return {k: statistics.mean(v) for k, v in by.items()}

    fetch, write = per_kernel("fetch"), per_kernel("write")
    if not fetch or not write:
        return
    pick = lambda d, key: next(v for k, v in d.items() if key in k)
    copy_bytes = float(1 << 30)
    f_scale = copy_bytes / pick(fetch, COPY)
    w_scale = copy_bytes / pick(write, COPY)
    rows = ["# HBM traffic per dispatch: {w} benchmark\n".format(w=workload),
            "Commands (each counter in a run of its own; $REPO = the repository root, $OUT = the "
            "directory the profiler writes to):\n", "```",
            PMC_CMD.format(ctr="FETCH_SIZE", kind="fetch", w=workload, args=args),
            PMC_CMD.format(ctr="WRITE_SIZE", kind="write", w=workload, args=args), "```\n",
            f"Scale: the 16-byte streaming copy of 1 GiB (`copy16`) reads {pick(fetch, COPY) / 2**20:.1f} MiB "
            f"by FETCH_SIZE and writes {pick(write, COPY) / 2**20:.1f} MiB by WRITE_SIZE, so fetch counts are "
            f"multiplied by {f_scale:.4f} and write counts by {w_scale:.4f}.\n",
            "| kernel | fetch MB (scaled) | write MB (scaled) | total MB |", "|---|---|---|---|"]
    for k in fetch:
        if k in write:
            fb, wb = fetch[k] * f_scale, write[k] * w_scale
            rows.append(f"| `{k[:90]}` | {fb / 1e6:.3f} | {wb / 1e6:.3f} | {(fb + wb) / 1e6:.3f} |")
    # the step's softmax backward is the fp16 instantiation (the fp32 repeat has its own)
    dom_f, dom_w = pick(fetch, DOMINANT + "IDF16_") * f_scale, pick(write, DOMINANT + "IDF16_") * w_scale
    with open(os.path.join(out_dir, f"{workload}_traffic.md"), "w") as fh:
        fh.write("\n".join(rows) + "\n")
    with open(os.path.join(out_dir, f"traffic_softmax_bw_{workload}.json"), "w") as fh:
        json.dump({"kernel": DOMINANT, "workload": workload, "source_sha256": source_digest(),
                   "fetch_bytes": round(dom_f), "write_bytes": round(dom_w),
                   "bytes_per_launch": round(dom_f + dom_w), "fetch_scale": f_scale,
                   "write_scale": w_scale}, fh, indent=1)
        fh.write("\n")


class HipEvents:
    """Timing events created through the HIP runtime (hipEvent_t handles as plain ints), so
    the library's lnr_time_next_launch hook can record them at a kernel's own start/end.

    They are created with hipEventDisableSystemFence: recording one then skips the
    system-scope cache writeback and invalidation that a default event performs, which would
    slow the kernel it brackets. The events only give timestamps, read after a device-wide
    synchronize."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.ct.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(h.value)
        return out

    def record(self, ev, stream):
        """Record `ev` on `stream` (a hipStream_t as an int; 0 is the default stream)."""
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventSynchronize(b) != 0 or self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def source_digest() -> str:
    """sha256 over the sources the dominant kernel (softmax backward) is built from: a traffic
    figure is only reported for the kernel code it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "layernorm_reduction_amd", "csrc")
    for f in ("lnr_common.h", "lnr_prims.h", "lnr_softmax.hip"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def table_cases():
    """(name, kind, shape, dtype, extra) for every op shape of the five workloads."""
    import torch
    from layernorm_reduction_amd import workloads as W
    cases = []
    for Tk in W.SOFTMAX_TK_SWEEP:
        for causal in (True, False):
            B = W.workload3_batch(Tk)
            cases.append((f"w3 softmax [{B},8,{Tk},{Tk}] {'causal' if causal else 'full'} padded fp16",
                          "softmax", (B, 8, Tk, Tk), torch.float16, {"causal": causal, "mask": True}))
    cases.append(("w2 softmax [32,8,256,256] causal fp16", "softmax", (32, 8, 256, 256), torch.float16,
                  {"causal": True, "mask": False}))
    for dt in (torch.float16, torch.float32):
        tag = "fp16" if dt == torch.float16 else "fp32"
        cases.append((f"w5 softmax [64,16,512,512] padded {tag}", "softmax", (64, 16, 512, 512), dt,
                      {"causal": False, "mask": True}))
    cases.append(("w2 layernorm [8192,256] fp16", "layernorm", (8192, 256), torch.float16, {}))
    for C in W.LAYERNORM_C_SWEEP:
        cases.append((f"w4 layernorm [16384,{C}] fp16", "layernorm", (16384, C), torch.float16, {}))
    for dt in (torch.float16, torch.float32):
        tag = "fp16" if dt == torch.float16 else "fp32"
        for C in (1024, 4096):
            cases.append((f"w5 layernorm [32768,{C}] {tag}", "layernorm", (32768, C), dt, {}))
    # RMSNorm (the FastTransformer page's Pre-RMSNorm): its own model shape, then wider rows.
    cases.append(("rmsnorm [8192,256] fp16", "rmsnorm", (8192, 256), torch.float16, {}))
    for C in (1024, 4096, 8192):
        cases.append((f"rmsnorm [16384,{C}] fp16", "rmsnorm", (16384, C), torch.float16, {}))
    for dt in (torch.float16, torch.float32):
        tag = "fp16" if dt == torch.float16 else "fp32"
        for C in (1024, 4096):
            cases.append((f"rmsnorm [32768,{C}] {tag}", "rmsnorm", (32768, C), dt, {}))
    # Softmax cross-entropy over a vocabulary: the GPT-2 batch of tokens, two vocabularies,
    # and a 64-row decoding batch (its backward splits rows over workgroups).
    for V in W.XENT_VOCABS:
        cases.append((f"xent [8192,{V}] fp16", "xent", (8192, V), torch.float16, {}))
    cases.append(("xent [8192,32000] fp32", "xent", (8192, 32000), torch.float32, {}))
    cases.append(("xent [64,32000] fp16 (decoding batch)", "xent", (64, 32000), torch.float16, {}))
    # Bias + dropout + residual feeding LayerNorm: post-LN (s has one consumer) and pre-LN (s
    # is the residual stream, so a second gradient reaches it) at the model shape, then wider.
    for extra in (False, True):
        cases.append((f"bdr-ln [8192,256] fp16 {'pre-LN' if extra else 'post-LN'}", "bdr", (8192, 256),
                      torch.float16, {"extra": extra}))
    for C in (1024, 4096):
        cases.append((f"bdr-ln [16384,{C}] fp16 post-LN", "bdr", (16384, C), torch.float16,
                      {"extra": False}))
    cases.append(("bdr-ln [32768,1024] fp32 post-LN", "bdr", (32768, 1024), torch.float32,
                  {"extra": False}))
    # Mask-aware read skipping: the same softmax, reading only runs with an unmasked key.
    cases.append(("skip w2 softmax [32,8,256,256] causal fp16", "softmax_skip", (32, 8, 256, 256),
                  torch.float16, {"causal": True, "mask": False}))
    for Tk in (256, 512, 1024, 2048):
        B = W.workload3_batch(Tk)
        for causal in (True, False):
            cases.append((f"skip w3 softmax [{B},8,{Tk},{Tk}] {'causal' if causal else 'full'} padded fp16",
                          "softmax_skip", (B, 8, Tk, Tk), torch.float16, {"causal": causal, "mask": True}))
    for dt in (torch.float16, torch.float32):
        tag = "fp16" if dt == torch.float16 else "fp32"
        cases.append((f"skip w5 softmax [64,16,512,512] padded {tag}", "softmax_skip", (64, 16, 512, 512),
                      dt, {"causal": False, "mask": True}))
    return cases


def run_table(match: str = "", warm: bool = False):
    """Back-to-back launches of each op over rotating buffers (>= 1 GiB footprint): average
    per launch from one event pair around a batch (the median of five batches), plus the
    kernel's own min / median / p90
    duration from events the kernel records (first kernel only for layernorm_bw).

    Beside each op, the same-size streaming ceiling: the library's 16-byte non-temporal copy
    (read one tensor, write one: the forward pattern) and read-two-write-one (lnr_xor2: the
    backward pattern) over tensors of the op's own size, timed the same way. Small tensors
    cannot reach the large-transfer bandwidth (launch ramp and drain), so
    fwbw_frac_of_ceiling = (t_copy + t_xor2) / (t_fw + t_bw) says how close an op comes to
    what any streaming kernel achieves at its size.

    warm: one input set reused by every launch, so tensors that fit the 256 MB Infinity Cache
    may be served from it. Those records say "cache": "warm" and are never the target's
    figures; by default the launches rotate over >= 1 GiB of input sets, which no cache holds."""
    import torch
    import layernorm_reduction_amd as lnr
    from layernorm_reduction_amd import workloads as W

    dev = torch.device("cuda:0")
    hev = HipEvents()
    hook = lnr.load().lnr_time_next_launch
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    reps = 30

    rounds = 5  # each back-to-back figure is the median of this many batches of `reps`

    def b2b_median(calls):
        for c in calls[:3]:
            c()
        torch.cuda.synchronize()
        per = []
        for _ in range(rounds):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                calls[i % len(calls)]()
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / reps)
        return statistics.median(per)

    def timed(calls):
        b2b = b2b_median(calls)
        ka, kb = hev.create(reps), hev.create(reps)
        for i in range(reps):
            hook(ka[i], kb[i])
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        k = sorted(hev.elapsed_ms(x, y) * 1e3 for x, y in zip(ka, kb))
        hev.destroy(ka + kb)
        return b2b, {"min": round(k[0], 2), "median": round(k[len(k) // 2], 2),
                     "p90": round(k[int(0.9 * (len(k) - 1))], 2)}

    def sets_for(set_bytes):
        return 1 if warm else max(2, math.ceil(MIN_FOOTPRINT / set_bytes))

    def ceiling(nbytes):
        """(copy us, read-two-write-one us) over rotating nbytes tensors, back to back."""
        nb = (nbytes + 15) // 16 * 16
        n = sets_for(3 * nb)
        bufs = [[torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(3)] for _ in range(n)]
        cp = [(lambda b=b: lnr.copy_bytes(b[2], b[0])) for b in bufs]
        xr = [(lambda b=b: lnr.xor_bytes(b[2], b[0], b[1])) for b in bufs]
        out = [b2b_median(calls) for calls in (cp, xr)]
        del bufs
        torch.cuda.empty_cache()
        return out

    # Warm-up: about 0.2 s of 1 GiB streaming copies, so the first cases do not run while the
    # device is still ramping up (the same case measured 5-15% slower at the start of a run).
    wa = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    wb = torch.empty_like(wa)
    for _ in range(600):
        lnr.copy_bytes(wb, wa)
    torch.cuda.synchronize()
    del wa, wb
    torch.cuda.empty_cache()

    for name, kind, shape, dt, extra in table_cases():
        if match not in name:
            continue
        s = W.dtype_size(dt)
        dense = None
        if kind in ("softmax", "softmax_skip"):
            B, H, T, _ = shape
            per = B * H * T * T * s
            n = sets_for(4 * per)
            fw, bw, dfw, dbw = [], [], [], []
            keep = []
            for _ in range(n):
                x = torch.randn(shape, device=dev, dtype=dt, generator=g)
                dy = torch.randn(shape, device=dev, dtype=dt, generator=g)
                y, dx = torch.empty_like(x), torch.empty_like(x)
                m = None
                if extra["mask"]:
                    m = torch.zeros(B, T, device=dev, dtype=dt)
                    m[:, T * 3 // 4:] = float("-inf")
                dfw.append(lnr.bind_attn_softmax_fw(x, m, extra["causal"], y))
                dbw.append(lnr.bind_attn_softmax_bw(dy, y, dx))
                if kind == "softmax_skip":
                    fw.append(lnr.bind_attn_softmax_fw_skip(x, m, extra["causal"], y))
                    bw.append(lnr.bind_attn_softmax_bw_skip(dy, y, m, extra["causal"], dx))
                keep += [x, dy, y, dx, m]
            bf = W.softmax_fw_bytes(B, H, T, T, s, has_mask=extra["mask"])
            bb = W.softmax_bw_bytes(B, H, T, T, s)
            if kind == "softmax":
                fw, bw = dfw, dbw
            else:
                # HBM figures use the bytes the skipping kernels move; the dense figures are
                # kept apart as dense-equivalent rates.
                dense = (dfw, dbw, bf, bb)
                bf, bb = W.softmax_skip_bytes(keep[4].cpu() if extra["mask"] else None,
                                              extra["causal"], B, H, T, T, s)
            rows, tensor = B * H * T, per
        elif kind == "layernorm":
            N, C = shape
            per = N * C * s
            n = sets_for(4 * per)
            fw, bw = [], []
            keep = []
            wsb = lnr.layernorm_bw_workspace_bytes(N, C, lnr.LNR_F16 if dt == torch.float16 else lnr.LNR_F32)
            for _ in range(n):
                x = torch.randn(shape, device=dev, dtype=dt, generator=g)
                dy = torch.randn(shape, device=dev, dtype=dt, generator=g)
                gm = torch.rand(C, device=dev, dtype=dt, generator=g) + 0.5
                bt = torch.randn(C, device=dev, dtype=dt, generator=g)
                y, dx = torch.empty_like(x), torch.empty_like(x)
                mean = torch.empty(N, device=dev, dtype=torch.float32)
                rstd = torch.empty(N, device=dev, dtype=torch.float32)
                dg, db = torch.empty(C, device=dev, dtype=dt), torch.empty(C, device=dev, dtype=dt)
                ws = torch.empty(max(wsb, 1), device=dev, dtype=torch.uint8)
                fw.append(lnr.bind_layernorm_fw(x, gm, bt, W.LN_EPS, y, mean, rstd))
                bw.append(lnr.bind_layernorm_bw(dy, x, gm, mean, rstd, dx, dg, db, ws))
                keep += [x, dy, gm, bt, y, dx, mean, rstd, dg, db, ws]
            bf = W.layernorm_fw_bytes(N, C, s)
            bb = W.layernorm_bw_bytes(N, C, s)
            rows, tensor = N, per
        elif kind == "xent":
            N, V = shape
            per = N * V * s
            n = sets_for(2 * per)
            fw, bw = [], []
            keep = []
            wsb = lnr.cross_entropy_fw_workspace_bytes(N, V, lnr.LNR_F16 if dt == torch.float16 else lnr.LNR_F32)
            for _ in range(n):
                z = torch.randn(shape, device=dev, dtype=dt, generator=g)
                t = torch.randint(0, V, (N,), device=dev, generator=g, dtype=torch.int64)
                loss = torch.empty(N, device=dev, dtype=torch.float32)
                lse = torch.empty(N, device=dev, dtype=torch.float32)
                dl = torch.ones(N, device=dev, dtype=torch.float32)
                dz = torch.empty_like(z)
                ws = torch.empty(wsb, device=dev, dtype=torch.uint8) if wsb > 0 else None
                fw.append(lnr.bind_cross_entropy_fw(z, t, -100, loss, lse, ws))
                bw.append(lnr.bind_cross_entropy_bw(z, t, lse, dl, 1.0, -100, dz))
                keep += [z, t, loss, lse, dl, dz, ws]
            bf = W.xent_fw_bytes(N, V, s)
            bb = W.xent_bw_bytes(N, V, s)
            rows, tensor = N, per
        elif kind == "rmsnorm":
            N, C = shape
            per = N * C * s
            n = sets_for(4 * per)
            fw, bw = [], []
            keep = []
            wsb = lnr.rmsnorm_bw_workspace_bytes(N, C, lnr.LNR_F16 if dt == torch.float16 else lnr.LNR_F32)
            for _ in range(n):
                x = torch.randn(shape, device=dev, dtype=dt, generator=g)
                dy = torch.randn(shape, device=dev, dtype=dt, generator=g)
                gm = torch.rand(C, device=dev, dtype=dt, generator=g) + 0.5
                y, dx = torch.empty_like(x), torch.empty_like(x)
                rstd = torch.empty(N, device=dev, dtype=torch.float32)
                dg = torch.empty(C, device=dev, dtype=dt)
                ws = torch.empty(max(wsb, 1), device=dev, dtype=torch.uint8)
                fw.append(lnr.bind_rmsnorm_fw(x, gm, W.RMS_EPS, y, rstd))
                bw.append(lnr.bind_rmsnorm_bw(dy, x, gm, rstd, dx, dg, ws))
                keep += [x, dy, gm, y, dx, rstd, dg, ws]
            bf = W.rmsnorm_fw_bytes(N, C, s)
            bb = W.rmsnorm_bw_bytes(N, C, s)
            rows, tensor = N, per
        elif kind == "bdr":
            N, C = shape
            per = N * C * s
            n = sets_for(8 * per)
            fw, bw = [], []
            keep = []
            wsb = lnr.bdr_layernorm_bw_workspace_bytes(N, C, lnr.LNR_F16 if dt == torch.float16 else lnr.LNR_F32)
            for _ in range(n):
                x = torch.randn(shape, device=dev, dtype=dt, generator=g)
                r = torch.randn(shape, device=dev, dtype=dt, generator=g)
                dy = torch.randn(shape, device=dev, dtype=dt, generator=g)
                de = torch.randn(shape, device=dev, dtype=dt, generator=g) if extra["extra"] else None
                mk = torch.randint(0, 256, (N, (C + 7) // 8), device=dev, generator=g,
                                   dtype=torch.int32).to(torch.uint8)
                bi = torch.randn(C, device=dev, dtype=dt, generator=g)
                gm = torch.rand(C, device=dev, dtype=dt, generator=g) + 0.5
                bt = torch.randn(C, device=dev, dtype=dt, generator=g)
                so, y, dr, dx = (torch.empty_like(x) for _ in range(4))
                mean = torch.empty(N, device=dev, dtype=torch.float32)
                rstd = torch.empty(N, device=dev, dtype=torch.float32)
                dg, db, dbi = (torch.empty(C, device=dev, dtype=dt) for _ in range(3))
                ws = torch.empty(max(wsb, 1), device=dev, dtype=torch.uint8)
                fw.append(lnr.bind_bdr_layernorm_fw(x, r, bi, mk, W.BDR_P, gm, bt, W.LN_EPS, so, y,
                                                    mean, rstd))
                bw.append(lnr.bind_bdr_layernorm_bw(dy, so, mk, W.BDR_P, gm, mean, rstd, de, dr, dx,
                                                    dg, db, dbi, ws))
                keep += [x, r, dy, de, mk, bi, gm, bt, so, y, dr, dx, mean, rstd, dg, db, dbi, ws]
            bf = W.bdr_fw_bytes(N, C, s)
            bb = W.bdr_bw_bytes(N, C, s, extra["extra"])
            rows, tensor = N, per
        torch.cuda.synchronize()
        f_b2b, f_k = timed(fw)
        b_b2b, b_k = timed(bw)
        skip_rec = None
        if dense is not None:
            dfw, dbw, dbf, dbb = dense
            df_b2b, _ = timed(dfw)
            db_b2b, _ = timed(dbw)
            skip_rec = {"dense_fw_us": round(df_b2b, 2), "dense_bw_us": round(db_b2b, 2),
                        "dense_equivalent_GBps": round((dbf + dbb) / (f_b2b + b_b2b) * 1e-3, 1),
                        "dense_bytes_fw": dbf, "dense_bytes_bw": dbb,
                        "speedup_fwbw_vs_dense": round((df_b2b + db_b2b) / (f_b2b + b_b2b), 3)}
            del dfw, dbw, dense
        del keep, fw, bw
        torch.cuda.empty_cache()
        c_copy, c_x2 = ceiling(tensor)
        # Same-size patterns: fw reads one tensor and writes one, bw reads two and writes one;
        # the cross-entropy forward only reads (no helper matches it) and its backward reads
        # one tensor and writes one.
        if kind == "xent":
            c_fw, c_bw = None, c_copy
        elif kind == "softmax_skip":
            c_fw, c_bw = None, None       # a dense-size ceiling does not bound a skipping kernel
        elif kind == "bdr":
            # fw reads two tensors and writes two, bw reads two or three and writes two: the
            # read-two-write-one time scaled by the tensor count (same size, same bandwidth)
            c_fw, c_bw = c_x2 * 4 / 3, c_x2 * (5 if extra["extra"] else 4) / 3
        else:
            c_fw, c_bw = c_copy, c_x2
        rec = {"case": name + (" (warm cache)" if warm else ""), "cache": "warm" if warm else "rotated",
               "fw_us": round(f_b2b, 2), "bw_us": round(b_b2b, 2),
               "fw_kernel_us": f_k, "bw_first_kernel_us": b_k,
               "fw_GBps": round(bf / f_b2b * 1e-3, 1), "bw_GBps": round(bb / b_b2b * 1e-3, 1),
               "fwbw_GBps": round((bf + bb) / (f_b2b + b_b2b) * 1e-3, 1),
               "fwbw_frac_of_peak": round((bf + bb) / (f_b2b + b_b2b) * 1e-3 / PEAK_HBM_GBPS, 4),
               "fw_rows_per_s": round(rows / (f_b2b * 1e-6)), "bw_rows_per_s": round(rows / (b_b2b * 1e-6)),
               "ceiling_copy_us": round(c_copy, 2), "ceiling_read2write1_us": round(c_x2, 2),
               "fwbw_frac_of_ceiling": (round((c_fw + c_bw) / (f_b2b + b_b2b), 4)
                                        if c_fw is not None else None),
               "bw_frac_of_ceiling": round(c_bw / b_b2b, 4) if c_bw is not None else None,
               "bytes_fw": bf, "bytes_bw": bb, "input_sets": n}
        if skip_rec is not None:
            rec.update(skip_rec)
        print(json.dumps(rec), flush=True)
        log(f"{name:48s} fw {f_b2b:8.1f} us {rec['fw_GBps']:7.0f} GB/s | bw {b_b2b:8.1f} us "
            f"{rec['bw_GBps']:7.0f} GB/s | fw+bw {rec['fwbw_GBps']:7.0f} GB/s "
            f"({rec['fwbw_frac_of_peak']:.0%} of 8 TB/s; same-size ceiling: "
            + (f"fw+bw {rec['fwbw_frac_of_ceiling']:.0%}" if rec['fwbw_frac_of_ceiling'] is not None
               else (f"bw {rec['bw_frac_of_ceiling']:.0%}" if rec['bw_frac_of_ceiling'] is not None
                     else "n/a")) + ")")
        if skip_rec is not None:
            log(f"{'':48s} dense fw {skip_rec['dense_fw_us']:8.1f} us | bw {skip_rec['dense_bw_us']:8.1f} us"
                f" | skip fw+bw {skip_rec['speedup_fwbw_vs_dense']:.2f}x faster, dense-equivalent "
                f"{skip_rec['dense_equivalent_GBps']:7.0f} GB/s")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_table():
    """The oracle (fp64 correctness reference, not a tuned CPU kernel) on the tiny, GPT-2 and
    hidden-size-sweep shapes: wall-clock median of 3 runs of fw + bw, with every host thread
    the process may use and with one, as rows/s and algorithmic GB/s (same byte formulas as
    the GPU lines, at the storage dtype)."""
    import oracle
    from layernorm_reduction_amd import workloads as W

    affinity = len(os.sched_getaffinity(0))
    model = cpu_model()
    cases = []
    [s1], [l1] = W.workload1()
    [s2], [l2] = W.workload2()
    cases += [("w1", s1), ("w1", l1), ("w2", s2), ("w2", l2)]
    cases += [("w4", W.workload4_case(C)) for C in W.LAYERNORM_C_SWEEP]
    for tag, case in cases:
        st = W.dtype_size(case.dtype)
        if hasattr(case, "Tk"):
            what = f"softmax [{case.B},{case.H},{case.Tq},{case.Tk}]"
            rows = case.B * case.H * case.Tq
            nbytes = (W.softmax_fw_bytes(case.B, case.H, case.Tq, case.Tk, st, has_mask=case.mask is not None)
                      + W.softmax_bw_bytes(case.B, case.H, case.Tq, case.Tk, st))

            def run(c=case):
                y = oracle.softmax_fw(c.x, c.mask, c.causal)
                oracle.softmax_bw(y, c.dy)
        else:
            what = f"layernorm [{case.N},{case.C}]"
            rows = case.N
            nbytes = W.layernorm_fw_bytes(case.N, case.C, st) + W.layernorm_bw_bytes(case.N, case.C, st)

            def run(c=case):
                oracle.layernorm_fw(c.x, c.gamma, c.beta, c.eps)
                oracle.layernorm_bw(c.x, c.dy, c.gamma, c.eps)
        for nthreads in (affinity, 1):
            oracle.set_threads(nthreads)
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                run()
                times.append(time.perf_counter() - t0)
            t = statistics.median(times)
            rec = {"case": f"{tag} {what} fw+bw", "threads": oracle.threads(), "seconds": round(t, 4),
                   "rows_per_s": round(rows / t), "GBps": round(nbytes / t / 1e9, 3),
                   "cpu_model": model, "kind": "oracle",
                   "note": "fp64 correctness oracle, not a tuned CPU kernel"}
            print(json.dumps(rec), flush=True)
            log(f"{rec['case']:44s} {nthreads:3d} threads {t * 1e3:10.1f} ms  {rec['GBps']:8.3f} GB/s")
    oracle.set_threads(affinity)


def main():
    args = parse()
    if args.table:
        run_table(args.match, warm=args.warm_cache)
        return
    if args.cpu_table:
        run_cpu_table()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.summarize_table_trace:
        summarize_table_trace(args.summarize_table_trace)
        return
    if args.skip_traffic:
        run_skip_traffic()
        return
    if args.summarize_skip_traffic:
        summarize_skip_traffic(args.summarize_skip_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; multi-GPU runs (--gpus N > 1) are not "
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
    wl_name, parts = workload_parts(args.workload)
    calls_meta = []       # (op label, algorithmic bytes) in step order
    per_set = 0
    for kind, c in parts:
        s = W.dtype_size(c.dtype)
        if kind == "softmax":
            tag = f"[{c.B},{c.H},{c.Tq},{c.Tk}]"
            calls_meta += [(f"attn_softmax_fw {tag}", W.softmax_fw_bytes(c.B, c.H, c.Tq, c.Tk, s, has_mask=c.mask is not None)),
                           (f"attn_softmax_bw {tag}", W.softmax_bw_bytes(c.B, c.H, c.Tq, c.Tk, s))]
        else:
            tag = f"[{c.N},{c.C}]"
            calls_meta += [(f"layernorm_fw {tag}", W.layernorm_fw_bytes(c.N, c.C, s)),
                           (f"layernorm_bw {tag}", W.layernorm_bw_bytes(c.N, c.C, s))]
        per_set += 4 * c.x.numel() * s
    step_bytes = sum(nb for _, nb in calls_meta)
    dom = 1                                   # the softmax backward: three passes over the scores
    b_sbw = calls_meta[dom][1]
    n_sets = max(2, math.ceil(MIN_FOOTPRINT / per_set))
    log(f"workload {args.workload}: {wl_name}; {step_bytes / 1e6:.1f} MB/step; {n_sets} input sets "
        f"({n_sets * per_set / 2 ** 30:.2f} GiB)")

    sets = [bind_parts(lnr, parts, dev) for _ in range(n_sets)]
    torch.cuda.synchronize()

    def step(i):
        for c in sets[i % n_sets]["calls"]:
            c()

    # ---------------------------------------------------------------- clock ramp (untimed)
    # The GPU sat idle while the host built the inputs. A few warm-up steps do not bring it
    # back to its steady clocks: after 5 of them, 20 timed steps ran 3% slower than after 2000.
    # Untimed steps for PREWARM_S seconds of device time (the host waits every 32 steps, so
    # the clock measures the device, not the launch queue); the warm-up steps follow.
    n_pre, t_pre = 0, time.perf_counter()
    while time.perf_counter() - t_pre < PREWARM_S:
        step(n_pre)
        n_pre += 1
        if n_pre % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    prewarm = {"steps": n_pre, "seconds": round(time.perf_counter() - t_pre, 3)}

    # ---------------------------------------------------------------- warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # The dominant kernel (softmax backward: three passes over the quadratic score tensor) is
    # timed inside the timed steps with HIP events that the kernel itself records at its start
    # and end (lnr_time_next_launch), on the stream it runs on: on every step of a short run
    # (fewer than 160 steps), else on every S-th step.
    K = args.steps
    every = 1 if K < 160 else max(1, args.sample_every)
    n_samp = (K + every - 1) // every
    hev = HipEvents()
    ev_a, ev_b = hev.create(n_samp), hev.create(n_samp)
    hook = lnr.load().lnr_time_next_launch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for j, c in enumerate(sets[i % n_sets]["calls"]):
            if j == dom and i % every == 0:
                hook(ev_a[i // every], ev_b[i // every])
            c()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / K
    value = step_bytes * K / elapsed / 1e9
    sbw_us = sorted(hev.elapsed_ms(a, b) * 1e3 for a, b in zip(ev_a, ev_b))
    hev.destroy(ev_a + ev_b)
    sbw_avg_us = statistics.mean(sbw_us)
    sbw_gbps = b_sbw / (sbw_avg_us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us -> {value:.0f} GB/s ({value / PEAK_HBM_GBPS:.1%} of 8 TB/s); "
        f"softmax_bw kernel {sbw_avg_us:.1f} us over {len(sbw_us)} launches -> {sbw_gbps:.0f} GB/s")

    # ---------------------------------------------------------------- diagnostics (untimed)
    ops, parts_out, fp32 = {}, {}, None
    if not args.no_ops:
        reps = max(20, min(K, 200))
        stream = torch.cuda.current_stream().cuda_stream
        for k, (name, nb) in enumerate(calls_meta):
            ops[name] = time_op(hev, hook, stream, [st["calls"][k] for st in sets], nb, reps)
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
        ops["copy_1GiB"] = {"bytes": 2 * n, "call_median_us": round(cus, 1),
                            "GBps": round(2 * n / (cus * 1e-6) / 1e9, 1)}
        del src, dst
        torch.cuda.empty_cache()
        # Same-size streaming ceilings, back to back over rotating buffers like the step: a
        # copy of one op tensor (the forward pattern) and read-two-write-one (the backward).
        for (kind, c), k in zip(parts, range(0, len(calls_meta), 2)):
            nb = c.x.numel() * W.dtype_size(c.dtype)
            for name, pattern in ((calls_meta[k][0], "copy"), (calls_meta[k + 1][0], "read2write1")):
                ops[name]["same_size_ceiling"] = {"pattern": pattern, "tensor_bytes": nb,
                                                  "b2b_us": round(same_size_ceiling(lnr, dev, nb, pattern, reps), 2)}
        parts_out = fwbw_summary(parts, calls_meta, ops)
        for k, v in ops.items():
            log(f"  {k:32s} call {v['call_median_us']:9.1f} us  {v['GBps']:8.1f} GB/s"
                + (f"  | kernel {v['kernel_median_us']:8.1f} us" if "kernel_median_us" in v else ""))
        for k, v in parts_out.items():
            log(f"  fw+bw {k:40s} {v['GBps']:8.1f} GB/s ({v['frac_of_peak']:.1%} of 8 TB/s)")
        if args.workload == "w5":
            # The same encoder-layer shapes repeated in fp32 storage (both dtypes against the
            # roofline); each op back to back over rotating input sets, not part of the step.
            del sets
            torch.cuda.empty_cache()
            fp32 = run_fp32_repeat(lnr, W, dev, hev, hook, stream, reps)

    # ---------------------------------------------------------------- roofline
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_softmax_bw_{args.workload}.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tr = json.load(fh)
        if tr.get("source_sha256") == source_digest():
            traffic = tr.get("bytes_per_launch")
    pct = lambda q: sbw_us[min(len(sbw_us) - 1, int(q * len(sbw_us)))]
    roofline = {"bound": "hbm", "kernel": "softmax_bw_vec (attn_softmax_bw)", "achieved": round(sbw_gbps, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(sbw_gbps / PEAK_HBM_GBPS, 4),
                "traffic": traffic, "avg_us": round(sbw_avg_us, 3), "median_us": round(pct(0.5), 3),
                "min_us": round(sbw_us[0], 3), "p90_us": round(pct(0.9), 3), "launches": len(sbw_us),
                "sampled": f"every {every} of {K} timed steps" if every > 1 else f"every one of {K} timed steps",
                "bytes_per_launch": b_sbw}

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, parts, step_bytes)

    first = parts[0][1]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm": prewarm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "config": {"workload": wl_name, "storage": "fp16", "compute": "fp32",
                   "softmax": [first.B, first.H, first.Tq, first.Tk], "causal": first.causal,
                   "key_padding": first.mask is not None,
                   "layernorm": [[c.N, c.C] for kind, c in parts if kind == "layernorm"],
                   "bytes_per_step": step_bytes, "input_sets": n_sets, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ops": ops,
        "fwbw": parts_out,
        "fp32_repeat": fp32,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


def workload_parts(name):
    """(description, [(kind, case), ...]) of a bench workload: the ops of one step in order."""
    import torch
    from layernorm_reduction_amd import workloads as W
    if name == "w5":
        return ("encoder layer, max_seq_len 512: padded softmax [64,16,512,512] + LayerNorm "
                "[32768,1024] + LayerNorm [32768,4096], fp16 storage",
                [("softmax", W.workload5_softmax(torch.float16)),
                 ("layernorm", W.workload5_layernorm(1024, torch.float16)),
                 ("layernorm", W.workload5_layernorm(4096, torch.float16))])
    [sc], [lc] = W.workload2()
    return ("GPT-2 training shapes B=32 T=256 C=256 H=8: causal softmax [32,8,256,256] + "
            "LayerNorm [8192,256], fp16 storage", [("softmax", sc), ("layernorm", lc)])


def bind_parts(lnr, parts, dev):
    """One input set on the device: every buffer of every op, and the bound calls (fw, bw per
    op, in step order)."""
    import torch
    t = {"calls": [], "keep": []}
    for kind, c in parts:
        if kind == "softmax":
            x, dy = c.x.to(dev), c.dy.to(dev)
            y, dx = torch.empty_like(x), torch.empty_like(x)
            m = None if c.mask is None else c.mask.to(dev)
            t["calls"] += [lnr.bind_attn_softmax_fw(x, m, c.causal, y), lnr.bind_attn_softmax_bw(dy, y, dx)]
            t["keep"] += [x, dy, y, dx, m]
        else:
            code = lnr.LNR_F16 if c.dtype == torch.float16 else lnr.LNR_F32
            x, dy, g, b = c.x.to(dev), c.dy.to(dev), c.gamma.to(dev), c.beta.to(dev)
            y, dx = torch.empty_like(x), torch.empty_like(x)
            mean = torch.empty(c.N, dtype=torch.float32, device=dev)
            rstd = torch.empty(c.N, dtype=torch.float32, device=dev)
            dg, db = torch.empty(c.C, dtype=c.dtype, device=dev), torch.empty(c.C, dtype=c.dtype, device=dev)
            ws = torch.empty(max(lnr.layernorm_bw_workspace_bytes(c.N, c.C, code), 1), dtype=torch.uint8,
                             device=dev)
            t["calls"] += [lnr.bind_layernorm_fw(x, g, b, c.eps, y, mean, rstd),
                           lnr.bind_layernorm_bw(dy, x, g, mean, rstd, dx, dg, db, ws)]
            t["keep"] += [x, dy, g, b, y, dx, mean, rstd, dg, db, ws]
    return t


def time_op(hev, hook, stream, calls, nb, reps):
    """One op over rotating input sets, in two passes so that neither set of events perturbs
    the other: the first kernel's own duration through the hook, then the whole call
    bracketed by events on its stream (includes the launch latency of each of its kernels)."""
    import torch
    n = len(calls)
    ka, kb = hev.create(reps), hev.create(reps)
    for i in range(reps):
        hook(ka[i], kb[i])
        calls[i % n]()
    torch.cuda.synchronize()
    kus = sorted(hev.elapsed_ms(a, b) * 1e3 for a, b in zip(ka, kb))
    ca, cb = hev.create(reps), hev.create(reps)
    for i in range(reps):
        hev.record(ca[i], stream)
        calls[i % n]()
        hev.record(cb[i], stream)
    torch.cuda.synchronize()
    us = sorted(hev.elapsed_ms(a, b) * 1e3 for a, b in zip(ca, cb))
    hev.destroy(ka + kb + ca + cb)
    med, kmed = us[len(us) // 2], kus[len(kus) // 2]
    return {"bytes": nb, "call_median_us": round(med, 2), "call_min_us": round(us[0], 2),
            "call_p90_us": round(us[int(0.9 * len(us))], 2), "kernel_median_us": round(kmed, 2),
            "GBps": round(nb / (med * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nb / (med * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "kernel_GBps": round(nb / (kmed * 1e-6) / 1e9, 1)}


def same_size_ceiling(lnr, dev, nb, pattern, reps):
    """Back-to-back time of the copy (forward pattern) or read-two-write-one (backward) helper
    over tensors of nb bytes, rotating buffers like the step."""
    import torch
    nbuf = max(2, math.ceil(MIN_FOOTPRINT / (3 * nb)))
    bufs = [[torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(3)] for _ in range(nbuf)]
    go = ((lambda b: lnr.copy_bytes(b[2], b[0])) if pattern == "copy"
          else (lambda b: lnr.xor_bytes(b[2], b[0], b[1])))
    for i in range(3):
        go(bufs[i % nbuf])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        go(bufs[i % nbuf])
    b.record()
    torch.cuda.synchronize()
    cu = a.elapsed_time(b) * 1e3 / reps
    del bufs
    torch.cuda.empty_cache()
    return cu


def fwbw_summary(parts, calls_meta, ops):
    """fw+bw GB/s per op of the step from the call medians: (fw bytes + bw bytes) / (t_fw + t_bw)."""
    out = {}
    for (kind, c), k in zip(parts, range(0, len(calls_meta), 2)):
        fw, bw = ops[calls_meta[k][0]], ops[calls_meta[k + 1][0]]
        nb = fw["bytes"] + bw["bytes"]
        us = fw["call_median_us"] + bw["call_median_us"]
        label = calls_meta[k][0].split(" ", 1)[1]
        name = f"{'softmax' if kind == 'softmax' else 'layernorm'} {label} {'fp16' if c.dtype.itemsize == 2 else 'fp32'}"
        out[name] = {"bytes": nb, "us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    return out


def run_fp32_repeat(lnr, W, dev, hev, hook, stream, reps):
    """The encoder-layer shapes in fp32 storage: each op's call and kernel medians over two
    rotating input sets, and fw+bw GB/s per op."""
    import torch
    parts = [("softmax", W.workload5_softmax(torch.float32)),
             ("layernorm", W.workload5_layernorm(1024, torch.float32)),
             ("layernorm", W.workload5_layernorm(4096, torch.float32))]
    ops, calls_meta = {}, []
    for kind, c in parts:
        s = W.dtype_size(c.dtype)
        sets = [bind_parts(lnr, [(kind, c)], dev) for _ in range(2)]
        torch.cuda.synchronize()
        if kind == "softmax":
            tag = f"[{c.B},{c.H},{c.Tq},{c.Tk}]"
            meta = [(f"attn_softmax_fw {tag}", W.softmax_fw_bytes(c.B, c.H, c.Tq, c.Tk, s, has_mask=True)),
                    (f"attn_softmax_bw {tag}", W.softmax_bw_bytes(c.B, c.H, c.Tq, c.Tk, s))]
        else:
            tag = f"[{c.N},{c.C}]"
            meta = [(f"layernorm_fw {tag}", W.layernorm_fw_bytes(c.N, c.C, s)),
                    (f"layernorm_bw {tag}", W.layernorm_bw_bytes(c.N, c.C, s))]
        for k, (name, nb) in enumerate(meta):
            for i in range(3):
                sets[i % 2]["calls"][k]()
            ops[name] = time_op(hev, hook, stream, [st["calls"][k] for st in sets], nb, reps)
            log(f"  fp32 {name:32s} call {ops[name]['call_median_us']:9.1f} us  {ops[name]['GBps']:8.1f} GB/s")
        calls_meta += meta
        del sets
        torch.cuda.empty_cache()
    return {"ops": ops, "fwbw": fwbw_summary(parts, calls_meta, ops)}


def cpu_baseline(workload, parts, step_bytes):
    """The oracle timed on the host cores over a bounded sample of the step (about 10 s of CPU
    work in all), scaled to the step's bytes."""
    import oracle
    log("timing the oracle on the host cores")
    if workload == "w2":
        frac, sample = 1.0, "one whole step: softmax fw+bw [32,8,256,256] and LayerNorm fw+bw [8192,256]"
        cut = lambda n: n
    else:
        frac = 1.0 / 8
        sample = ("1/8 of a step: softmax fw+bw [8,16,512,512], LayerNorm fw+bw [4096,1024] and "
                  "[4096,4096]")
        cut = lambda n: n // 8
    work = []
    for kind, c in parts:
        if kind == "softmax":
            b = cut(c.B)
            work.append(("softmax", c.x[:b], c.dy[:b], None if c.mask is None else c.mask[:b], c.causal))
        else:
            n = cut(c.N)
            work.append(("layernorm", c.x[:n], c.dy[:n], c.gamma, c.beta, c.eps))
    times = []
    t_start = time.perf_counter()
    while True:
        c0 = time.perf_counter()
        for w in work:
            if w[0] == "softmax":
                y = oracle.softmax_fw(w[1], w[3], w[4])
                oracle.softmax_bw(y, w[2])
                del y
            else:
                oracle.layernorm_fw(w[1], w[3], w[4], w[5])
                oracle.layernorm_bw(w[1], w[2], w[3], w[5])
        times.append(time.perf_counter() - c0)
        spent = time.perf_counter() - t_start
        if (len(times) >= 3 and spent >= 10.0) or spent >= 30.0:
            break
    tmed = statistics.median(times)
    cpu = {"value": round(step_bytes * frac / tmed / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
           "cpu_model": cpu_model(), "kind": "oracle", "sample": f"{sample}, repeated {len(times)} times",
           "seconds_per_sample": round(tmed, 3), "repeats": len(times),
           "seconds_total": round(sum(times), 1),
           "note": "fp64 correctness oracle, not a tuned CPU kernel; the median sample is reported"}
    log(f"oracle: {tmed:.2f} s per sample on {cpu['cores']} threads -> {cpu['value']} GB/s")
    return cpu


if __name__ == "__main__":
    main()
