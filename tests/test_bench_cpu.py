"""Host logic of bench.py that runs without a GPU: the one-GPU contract, the loud failure where
no GPU is visible, the fw+bw summary arithmetic, and the freshness of the committed traffic
records that the bench reports as roofline.traffic."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest
import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env, cwd=ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = run_bench("--gpus", str(n))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = run_bench("--steps", "1", "--warmup", "0", env=env)
    assert r.returncode == 2
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the bench would run")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "no GPU" in r.stderr and r.stdout == ""


def test_fwbw_summary_is_bytes_over_summed_call_times():
    f16 = SimpleNamespace(dtype=torch.float16)
    f32 = SimpleNamespace(dtype=torch.float32)
    parts = [("softmax", f16), ("layernorm", f32)]
    meta = [("attn_softmax_fw [2,3,4,4]", 100), ("attn_softmax_bw [2,3,4,4]", 150),
            ("layernorm_fw [8,16]", 40), ("layernorm_bw [8,16]", 60)]
    ops = {"attn_softmax_fw [2,3,4,4]": {"bytes": 100e6, "call_median_us": 10.0},
           "attn_softmax_bw [2,3,4,4]": {"bytes": 150e6, "call_median_us": 15.0},
           "layernorm_fw [8,16]": {"bytes": 40e6, "call_median_us": 4.0},
           "layernorm_bw [8,16]": {"bytes": 60e6, "call_median_us": 16.0}}
    out = bench.fwbw_summary(parts, meta, ops)
    sm, ln = out["softmax [2,3,4,4] fp16"], out["layernorm [8,16] fp32"]
    # 250 MB in 25 us = 10000 GB/s; 100 MB in 20 us = 5000 GB/s
    assert sm["bytes"] == 250e6 and sm["us"] == 25.0 and sm["GBps"] == 10000.0
    assert sm["frac_of_peak"] == 1.25
    assert ln["bytes"] == 100e6 and ln["us"] == 20.0 and ln["GBps"] == 5000.0
    assert ln["frac_of_peak"] == 0.625


@pytest.mark.parametrize("workload", ["w5", "w2"])
def test_committed_traffic_record_matches_the_softmax_sources(workload):
    """The bench reports a traffic record only for the kernel sources it was measured on; the
    committed records must be those of the current softmax backward."""
    with open(os.path.join(ROOT, "profiles", f"traffic_softmax_bw_{workload}.json")) as fh:
        rec = json.load(fh)
    assert rec["source_sha256"] == bench.source_digest()
    algorithmic = {"w5": 3 * 64 * 16 * 512 * 512 * 2, "w2": 3 * 32 * 8 * 256 * 256 * 2}[workload]
    # counted bytes within 0.1% of the algorithmic three passes over the scores
    assert abs(rec["bytes_per_launch"] / algorithmic - 1) < 1e-3


def _csv(path, header, rows):
    """A CSV file as rocprofv3 writes it (fields with commas, such as kernel names, quoted)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_traffic_record_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    """summarize_profiles on synthetic rocprofv3 output with known counts: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are scaled by what they read for the 1 GiB copy (only the
    copy at the calibration grid counts), and the fp16 softmax backward's scaled bytes become
    the record the bench reports as roofline.traffic."""
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    os.symlink(os.path.join(ROOT, "layernorm_reduction_amd"), root / "layernorm_reduction_amd")
    monkeypatch.setattr(bench, "ROOT", str(root))
    out = tmp_path / "out"
    dom16 = "_ZN3lnr14softmax_bw_vecIDF16_Li64ELi1ELi64EEEvPT_PKS1_S4_li"
    dom32 = "void lnr::softmax_bw_vec<float, 64, 2, 64>(float*, float const*, float const*, long, int)"
    copy = "lnr::copy16(float __vector(4)*, float __vector(4) const*, long)"
    _csv(str(out / "prof_w5" / "w5_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
         [[dom16, 67, 241000.0, 237000.0, 248000.0, 12.8]])
    calib = bench.CALIB_GRID
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Value"]
    # the copy reads 1 GiB but FETCH_SIZE counts 512 MiB (scale 2) and WRITE_SIZE 1 GiB (scale
    # 1); a same-size-ceiling copy at another grid carries other counts and must be ignored
    _csv(str(out / "pmc_fetch_w5" / "w5_counter_collection.csv"), hdr,
         [[copy, calib, 512 * 1024], [copy, calib // 4, 1], [dom16, 1 << 24, 500000], [dom16, 1 << 24, 500002],
          [dom32, 1 << 24, 999999]])
    _csv(str(out / "pmc_write_w5" / "w5_counter_collection.csv"), hdr,
         [[copy, calib, 1024 * 1024], [copy, calib // 4, 7], [dom16, 1 << 24, 250000], [dom32, 1 << 24, 1]])
    bench.summarize_profiles(str(out), "w5")
    with open(root / "profiles" / "traffic_softmax_bw_w5.json") as fh:
        rec = json.load(fh)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 500001 * 1024 * 2      # mean over the fp16 dispatches, scaled
    assert rec["write_bytes"] == 250000 * 1024
    assert rec["bytes_per_launch"] == 500001 * 2048 + 250000 * 1024
    assert rec["source_sha256"] == bench.source_digest()
    trace = (root / "profiles" / "w5_kernel_trace.md").read_text()
    assert "| 67 | 241.00 | 237.00 | 248.00 | 12.8% |" in trace
