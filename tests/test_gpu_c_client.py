"""The C ABI driven by a plain C99 program (tests/native/c_client.c, built by
__graft_entry__.build()): device memory and a stream from the HIP runtime directly, masked
causal softmax forward and backward and LayerNorm forward and backward, checked against
properties of the operations (rows of probabilities sum to 1 with exact zeros at masked and
future keys, gradient rows sum to 0, LayerNorm rows have mean 0 and second moment v/(v+eps),
the saved statistics are the row's, dbeta is the column sum of dy)."""
import os
import subprocess

import pytest

from parity_utils import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "native", "c_client")


def test_c_client_on_the_gpu():
    assert os.path.exists(CLIENT), "tests/native/c_client is not built (run __graft_entry__.build())"
    say("c_client gpu")
    r = subprocess.run([CLIENT, "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert ", 0 failed" in r.stdout
