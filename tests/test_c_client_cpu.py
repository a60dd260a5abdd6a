"""The C ABI from a plain C99 program (tests/native/c_client.c), with no Python in the loop:
argument validation returns the documented statuses, the status strings and the build string
are reachable. No device is touched."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "native", "c_client")


def test_c_client_validation_without_a_gpu():
    if not os.path.exists(CLIENT):
        from layernorm_reduction_amd import build
        if not os.path.exists(os.path.join(ROOT, "layernorm_reduction_amd", "liblnr.so")):
            build.build()
        build.build_c_client()
    r = subprocess.run([CLIENT, "validate"], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 failed" in r.stdout
