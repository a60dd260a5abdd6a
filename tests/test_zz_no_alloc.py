"""layernorm_bw_noalloc (the column partials in the library's own device array instead of a
caller workspace) against layernorm_bw, through the C ABI.

Both entry points run the same kernels with the same partial rows in the same order, so their
outputs must be bitwise equal; both are also compared with the oracle's backward on the same
fp32 statistics at the plain tolerance (1e-3 fp16, 1e-5 fp32). Two calls in a row on one
device share the array: the second, smaller call must not see the first call's partials."""
import pytest
import torch

import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import assert_close, assert_grad_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_pair(case):
    x64, g64, dy64 = case.x.double().numpy(), case.gamma.double().numpy(), case.dy.double().numpy()
    _, mean_ref, rstd_ref = oracle.layernorm_fw(x64, g64, case.beta.double().numpy(), case.eps)
    m32 = torch.from_numpy(mean_ref).float()
    r32 = torch.from_numpy(rstd_ref).float()
    dx_ref, dg_ref, db_ref = oracle.layernorm_bw_given_stats(x64, dy64, g64, m32, r32)
    xd, gd, dyd, md, rd = (t.to(DEV) for t in (case.x, case.gamma, case.dy, m32, r32))
    say(case.name, "layernorm_bw and layernorm_bw_noalloc")
    a = lnr.layernorm_bw(dyd, xd, gd, md, rd)
    # outputs pre-filled with NaN: every element must be written
    outs = [torch.full_like(xd, float("nan")), torch.full_like(gd, float("nan")),
            torch.full_like(gd, float("nan"))]
    b = lnr.layernorm_bw_noalloc(dyd, xd, gd, md, rd, *outs)
    torch.cuda.synchronize()
    for u, v, nm in zip(a, b, ("dx", "dgamma", "dbeta")):
        assert torch.equal(u, v), f"{case.name} {nm}: noalloc differs from the workspace entry point"
    gm = (dy64 * g64.reshape(1, -1))
    gmax = abs(gm).max(axis=1)
    assert_grad_close(b[0], dx_ref, case.dtype, f"{case.name} noalloc dx", r32.double().numpy(), gmax)
    assert_close(b[1], dg_ref, case.dtype, f"{case.name} noalloc dgamma")
    assert_close(b[2], db_ref, case.dtype, f"{case.name} noalloc dbeta")


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_noalloc_equals_workspace_entry_point_twice(dtype):
    big = W.workload5_layernorm(1024, dtype) if dtype == torch.float16 else \
        W.layernorm_case("noalloc-8192x4096-f32", 8192, 4096, dtype=dtype, seed_base=9810, row_offset_var=1.0)
    check_pair(big)
    small = W.layernorm_case(f"noalloc-1031x1000-{dtype}", 1031, 1000, dtype=dtype, seed_base=9820,
                             row_offset_var=1.0)
    check_pair(small)


def test_noalloc_rejects_shapes_beyond_its_array():
    N, C = 1024, 8192            # fp32 partials: 256 x 2 x 8192 x 8 bytes > 16 MiB
    x = torch.zeros(N, C, dtype=torch.float32, device=DEV)
    g = torch.ones(C, dtype=torch.float32, device=DEV)
    m = torch.zeros(N, dtype=torch.float32, device=DEV)
    with pytest.raises(lnr.LnrError) as e:
        lnr.layernorm_bw_noalloc(x, x, g, m, m)
    assert e.value.status == 9


def test_noalloc_zero_rows_give_zero_parameter_gradients():
    C = 1024
    x = torch.empty(0, C, dtype=torch.float16, device=DEV)
    g = torch.ones(C, dtype=torch.float16, device=DEV)
    m = torch.empty(0, dtype=torch.float32, device=DEV)
    dg = torch.full((C,), 7.0, dtype=torch.float16, device=DEV)
    db = torch.full((C,), 7.0, dtype=torch.float16, device=DEV)
    say("N=0 noalloc backward")
    lnr.layernorm_bw_noalloc(x, x, g, m, m, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(db == 0)
