"""Host logic of the division by a launch-invariant divisor that the softmax forward uses for
its row -> (batch, query) index math: the magic numbers of lnr_fastdiv.h reproduce n / d for
edge and random numerators over thousands of divisors, and for every 32-bit numerator with
two divisors. Compiled with the host C++ compiler; no GPU involved."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fastdiv_matches_integer_division(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "layernorm_reduction_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
