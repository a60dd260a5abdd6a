"""The entry module's contract on a host without a GPU: smoke() refuses to run rather than
pass on anything but the HIP library, and the product path has no CPU fallback."""
import pytest
import torch

import __graft_entry__
import layernorm_reduction_amd as lnr


def test_smoke_needs_a_gpu():
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: smoke() would run")
    with pytest.raises(RuntimeError, match="GPU"):
        __graft_entry__.smoke()


def test_ops_refuse_host_tensors():
    x = torch.zeros(4, 64, dtype=torch.float16)
    g = torch.ones(64, dtype=torch.float16)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        lnr.layernorm_fw(x, g, g, 1e-8)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        lnr.attn_softmax_fw(torch.zeros(1, 1, 4, 64, dtype=torch.float16))
