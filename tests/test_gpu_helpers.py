"""GPU checks of the two measurement helpers the benchmark's ceilings come from: lnr_copy and
lnr_xor2 must move exactly the bytes they claim, including a size that leaves a partial last
workgroup."""
import pytest
import torch

import layernorm_reduction_amd as lnr
from parity_utils import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20])
def test_copy_and_xor_move_exact_bytes(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    a = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    b = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    ad, bd = a.to(DEV), b.to(DEV)
    say("helpers", nbytes)
    c = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    lnr.copy_bytes(c, ad)
    x = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    lnr.xor_bytes(x, ad, bd)
    torch.cuda.synchronize()
    assert torch.equal(c[:nbytes].cpu(), a) and int(c[nbytes:].count_nonzero()) == 0
    assert torch.equal(x[:nbytes].cpu(), a ^ b) and int(x[nbytes:].count_nonzero()) == 0
