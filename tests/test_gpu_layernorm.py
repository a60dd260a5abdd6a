"""GPU parity of layernorm_fw / layernorm_bw (through the C ABI) against the fp64 oracle.

  * forward: y, mean and rstd on the seeded inputs of each workload, every element;
  * backward on identical stored inputs: the GPU receives the oracle's mean/rstd rounded to
    fp32 (the ABI's statistics format) and is compared, element by element, with the oracle's
    backward evaluated on those same fp32 statistics (dx, dgamma, dbeta);
  * chained: GPU forward statistics feeding the GPU backward, against the true gradient (the
    oracle recomputes the statistics from x in fp64).
Workloads 1, 2, 4 and 5 run at their full sizes, in the launch configuration the benchmark uses.

Every comparison uses the plain element-wise bound atol + rtol * |ref| (1e-3 fp16, 1e-5 fp32),
with two exceptions, both printed when they apply:
  * near-constant rows of the edge-case tests (parity_utils.assert_grad_close): dx of a row
    with rstd >= 8 may add the fp32 formula's own rounding term;
  * the chained dgamma at fp32 storage over 32768 rows is compared norm-wise, max |err| <=
    atol + rtol * max |ref|, with its element-wise pass rate printed: every row's fp32
    statistics carry about 1e-7 relative rounding, random over rows, and a column sum over
    32768 rows accumulates that to about 1e-5 absolute, so near-zero columns can miss an
    element-wise 1e-5 however exactly the sum itself is taken.
"""
import numpy as np
import pytest
import torch

import gpu_cases
import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import TOL, assert_close, assert_grad_close, say, to_host64, violations

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gmax_of(dy64, g64):
    """Per row, max_j |gamma_j * dy_ij|: the largest term the dx formula subtracts from."""
    return np.max(np.abs(dy64 * g64.reshape(1, -1)), axis=1)


def run_ln(case, chain=True, chain_dgamma_normwise=False, edge=False):
    atol, rtol = TOL[case.dtype]
    say(case.name, "oracle forward")
    x64 = case.x.double().numpy()
    g64 = case.gamma.double().numpy()
    y_ref, mean_ref, rstd_ref = oracle.layernorm_fw(x64, g64, case.beta.double().numpy(), case.eps)

    say(case.name, "GPU forward")
    xd, gd, bd = case.x.to(DEV), case.gamma.to(DEV), case.beta.to(DEV)
    y, mean, rstd = lnr.layernorm_fw(xd, gd, bd, case.eps)
    torch.cuda.synchronize()
    assert_close(y, y_ref, case.dtype, f"{case.name} y")
    assert_close(mean, mean_ref, case.dtype, f"{case.name} mean")
    assert_close(rstd, rstd_ref, case.dtype, f"{case.name} rstd")
    del y_ref, y

    say(case.name, "oracle backward (given fp32 statistics)")
    dy64 = case.dy.double().numpy()
    m32 = torch.from_numpy(mean_ref).float()
    r32 = torch.from_numpy(rstd_ref).float()
    dx_ref, dg_ref, db_ref = oracle.layernorm_bw_given_stats(x64, dy64, g64, m32, r32)
    say(case.name, "GPU backward")
    dyd = case.dy.to(DEV)
    dx, dg, db = lnr.layernorm_bw(dyd, xd, gd, m32.to(DEV), r32.to(DEV))
    torch.cuda.synchronize()
    gm = gmax_of(dy64, g64)
    assert_grad_close(dx, dx_ref, case.dtype, f"{case.name} dx", r32.double().numpy(), gm,
                      allow_near_constant=edge)
    assert_close(dg, dg_ref, case.dtype, f"{case.name} dgamma")
    assert_close(db, db_ref, case.dtype, f"{case.name} dbeta")
    del dx_ref, dg_ref, db_ref, dx, dg, db

    if chain:
        say(case.name, "oracle backward (exact) and GPU chained fw -> bw")
        tdx, tdg, tdb = oracle.layernorm_bw(x64, dy64, g64, case.eps)
        dx2, dg2, db2 = lnr.layernorm_bw(dyd, xd, gd, mean, rstd)
        torch.cuda.synchronize()
        assert_grad_close(dx2, tdx, case.dtype, f"{case.name} chain dx", rstd_ref, gm,
                          allow_near_constant=edge)
        assert_close(db2, tdb, case.dtype, f"{case.name} chain dbeta")
        if chain_dgamma_normwise:
            got = to_host64(dg2)
            bad, _ = violations(got, tdg, atol, rtol)
            print(f"[info] {case.name} chained dgamma element-wise: {case.C - bad}/{case.C} within "
                  f"atol=rtol={atol}", flush=True)
            err = np.max(np.abs(got - tdg))
            assert err <= atol + rtol * np.max(np.abs(tdg)), err
        else:
            assert_close(dg2, tdg, case.dtype, f"{case.name} chain dgamma")
    del xd, gd, bd, dyd
    torch.cuda.empty_cache()


def test_workload1_tiny_fp32():
    _, [case] = W.workload1()
    run_ln(case)


def test_workload2_gpt2_fp16():
    _, [case] = W.workload2()
    run_ln(case)


@pytest.mark.parametrize("C", W.LAYERNORM_C_SWEEP)
def test_workload4_hidden_size_sweep(C):
    run_ln(W.workload4_case(C))


@pytest.mark.parametrize("C", [1024, 4096])
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_workload5_encoder_layer(C, dtype):
    run_ln(W.workload5_layernorm(C, dtype), chain_dgamma_normwise=(dtype == torch.float32))


# ------------------------------------------------------------------------- edge cases

EDGE_C = gpu_cases.NORM_EDGE_C


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("C", EDGE_C)
def test_bucket_boundaries_and_ragged_rows(C, dtype):
    for N in (1, 7, 1031):
        case = W.layernorm_case(f"edge-N{N}-C{C}-{dtype}", N, C, dtype=dtype,
                                seed_base=7000 + C, row_offset_var=1.0)
        run_ln(case, chain=False, edge=True)


def odd_trip_count(N, C, dtype):
    """Rows each backward workgroup walks per row group (its loop trip count), from the plan:
    about N / 256 rows per workgroup, rounded up to whole row groups."""
    code = lnr.LNR_F16 if dtype == torch.float16 else lnr.LNR_F32
    _, G, _, WG, blocks = lnr.layernorm_plan(N, C, code, backward=True)
    groups = WG // G
    per_block = -(-N // 256)                      # ceil(N / 256)
    rpb = -(-per_block // groups) * groups        # whole row groups
    assert blocks == -(-N // rpb), (blocks, rpb)
    return G, rpb // groups


# Backward plans whose row sits inside one wave store each row after the next row's fetch,
# through a loop unrolled by two: with an odd trip count of three or more, the last live row
# is stored from the second half of the loop and a dead row follows it. Ragged last
# workgroups as well.
ODD_TRIPS = [(49151, 64, torch.float16), (12283, 256, torch.float16), (10237, 1000, torch.float16),
             (6141, 500, torch.float32)]


@pytest.mark.parametrize("N,C,dtype", ODD_TRIPS)
def test_backward_odd_row_loop_trip_counts(N, C, dtype):
    G, trips = odd_trip_count(N, C, dtype)
    assert G <= 64 and trips >= 3 and trips % 2 == 1, (G, trips)
    case = W.layernorm_case(f"odd-trips-N{N}-C{C}-{dtype}", N, C, dtype=dtype,
                            seed_base=7700 + C, row_offset_var=1.0)
    run_ln(case, chain=False)


@pytest.mark.parametrize("N,C", gpu_cases.NORM_LONG_F16)
def test_long_ragged_launch(N, C):
    """Long launches with a ragged row count (not whole row groups, a partial last band), at a
    width with idle lanes and at the bucket's full width."""
    case = W.layernorm_case(f"long-N{N}-C{C}", N, C, dtype=torch.float16, seed_base=7900 + C,
                            row_offset_var=1.0)
    run_ln(case)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_constant_rows_give_beta(dtype):
    N, C = 16, 256
    x = torch.full((N, C), 0.5, dtype=dtype, device=DEV)
    g = W.uniform((C,), 7100, 0.5, 1.5).to(dtype).to(DEV)
    b = W.normal((C,), 7101).to(dtype).to(DEV)
    say("constant rows", dtype)
    y, mean, rstd = lnr.layernorm_fw(x, g, b, 1e-8)
    torch.cuda.synchronize()
    assert torch.equal(y, b.expand(N, C))
    assert torch.all(mean == 0.5)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_and_bitwise_determinism(dtype):
    case = W.layernorm_case("det", 3000, 1024, dtype=dtype, seed_base=7200, row_offset_var=4.0)
    x, g, b, dy = (t.to(DEV) for t in (case.x, case.gamma, case.beta, case.dy))
    say(case.name, dtype)
    y1, m1, r1 = lnr.layernorm_fw(x, g, b)
    y2, m2, r2 = lnr.layernorm_fw(x, g, b)
    xi = x.clone()
    yi, mi, ri = lnr.layernorm_fw(xi, g, b, y=xi)
    a = lnr.layernorm_bw(dy, x, g, m1, r1)
    c = lnr.layernorm_bw(dy, x, g, m1, r1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, xi)
    assert torch.equal(m1, m2) and torch.equal(r1, r2) and torch.equal(m1, mi)
    for u, v in zip(a, c):
        assert torch.equal(u, v)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_unaligned_buffers_take_the_fallback(dtype):
    case = W.layernorm_case("unaligned", 300, 512, dtype=dtype, seed_base=7300, row_offset_var=1.0)
    N, C = case.N, case.C

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:].copy_(t.reshape(-1).to(DEV))
        return buf[1:].view(t.shape)

    x, g, b, dy = shifted(case.x), shifted(case.gamma), shifted(case.beta), shifted(case.dy)
    say(case.name, dtype)
    y, mean, rstd = lnr.layernorm_fw(x, g, b, case.eps)
    dx, dg, db = lnr.layernorm_bw(dy, x, g, mean, rstd)
    torch.cuda.synchronize()
    x64, g64 = case.x.double().numpy(), case.gamma.double().numpy()
    y_ref, _, _ = oracle.layernorm_fw(x64, g64, case.beta.double().numpy(), case.eps)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bw(x64, case.dy.double().numpy(), g64, case.eps)
    assert_close(y, y_ref, dtype, "unaligned y")
    assert_close(dx, dx_ref, dtype, "unaligned dx")
    assert_close(dg, dg_ref, dtype, "unaligned dgamma")
    assert_close(db, db_ref, dtype, "unaligned dbeta")


def test_zero_rows_give_zero_parameter_gradients():
    C = 1024
    x = torch.empty(0, C, dtype=torch.float16, device=DEV)
    g = torch.ones(C, dtype=torch.float16, device=DEV)
    m = torch.empty(0, dtype=torch.float32, device=DEV)
    dg = torch.full((C,), 7.0, dtype=torch.float16, device=DEV)
    db = torch.full((C,), 7.0, dtype=torch.float16, device=DEV)
    say("N=0 backward")
    lnr.layernorm_bw(x, x, g, m, m, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(db == 0)


def test_small_workspace_is_rejected():
    N, C = 512, 1024
    x = torch.zeros(N, C, dtype=torch.float16, device=DEV)
    g = torch.ones(C, dtype=torch.float16, device=DEV)
    m = torch.zeros(N, dtype=torch.float32, device=DEV)
    need = lnr.layernorm_bw_workspace_bytes(N, C, lnr.LNR_F16)
    ws = torch.empty(need - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(lnr.LnrError) as e:
        lnr.layernorm_bw(x, x, g, m, m, workspace=ws)
    assert e.value.status == 7
