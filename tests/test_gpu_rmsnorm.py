"""GPU parity of rmsnorm_fw / rmsnorm_bw (through the C ABI) against the fp64 oracle.

RMSNorm as the FastTransformer page defines it (section 5.4): y = x * rsqrt(mean(x^2) + eps)
* weight, eps = 1e-6, no bias. Same structure as the LayerNorm tests:
  * forward: y and rstd on seeded inputs, every element;
  * backward on identical stored inputs: the GPU receives the oracle's rstd rounded to fp32
    and is compared with the oracle's backward evaluated on that same rstd;
  * chained: GPU forward rstd feeding the GPU backward, against the true gradient.

Plain element-wise bounds throughout (1e-3 fp16, 1e-5 fp32), with the LayerNorm tests' two
printed exceptions: near-constant rows of the edge-case tests (rstd >= 8; here also the zero
rows, rstd = 1/sqrt(eps)) may add the fp32 formula's rounding term to dx, 16 * 2^-24 * rstd_i
* max_j (|g_ij| + |xhat_ij b_i|) with b = mean(g * xhat); and the chained dgamma over 32768
fp32 rows is norm-wise.
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
def rms_gmax(x64, dy64, g64, rstd):
    """Per row, max_j (|g_ij| + |xhat_ij * b_i|): the terms the dx formula subtracts."""
    r = np.asarray(rstd, np.float64).reshape(-1, 1)
    gd = dy64 * g64.reshape(1, -1)
    xh = x64 * r
    b = np.mean(gd * xh, axis=1, keepdims=True)
    return np.max(np.abs(gd) + np.abs(xh * b), axis=1)


def run_rms(case, chain=True, chain_dgamma_normwise=False, edge=False):
    atol, rtol = TOL[case.dtype]
    say(case.name, "oracle forward")
    x64 = case.x.double().numpy()
    g64 = case.gamma.double().numpy()
    y_ref, rr_ref = oracle.rmsnorm_fw(x64, g64, case.eps)

    say(case.name, "GPU forward")
    xd, gd = case.x.to(DEV), case.gamma.to(DEV)
    y, rstd = lnr.rmsnorm_fw(xd, gd, case.eps)
    torch.cuda.synchronize()
    assert_close(y, y_ref, case.dtype, f"{case.name} y")
    assert_close(rstd, rr_ref, case.dtype, f"{case.name} rstd")
    del y_ref, y

    say(case.name, "oracle backward (given fp32 rstd)")
    dy64 = case.dy.double().numpy()
    r32 = torch.from_numpy(rr_ref).float()
    dx_ref, dg_ref = oracle.rmsnorm_bw_given_rstd(x64, dy64, g64, r32.numpy())
    say(case.name, "GPU backward")
    dyd = case.dy.to(DEV)
    dx, dg = lnr.rmsnorm_bw(dyd, xd, gd, r32.to(DEV))
    torch.cuda.synchronize()
    r64 = r32.double().numpy()
    assert_grad_close(dx, dx_ref, case.dtype, f"{case.name} dx", r64, rms_gmax(x64, dy64, g64, r64),
                      allow_near_constant=edge)
    assert_close(dg, dg_ref, case.dtype, f"{case.name} dgamma")
    del dx_ref, dg_ref, dx, dg

    if chain:
        say(case.name, "oracle backward (exact) and GPU chained fw -> bw")
        tdx, tdg = oracle.rmsnorm_bw(x64, dy64, g64, case.eps)
        dx2, dg2 = lnr.rmsnorm_bw(dyd, xd, gd, rstd)
        torch.cuda.synchronize()
        assert_grad_close(dx2, tdx, case.dtype, f"{case.name} chain dx", rr_ref,
                          rms_gmax(x64, dy64, g64, rr_ref), allow_near_constant=edge)
        if chain_dgamma_normwise:
            got = to_host64(dg2)
            bad, _ = violations(got, tdg, atol, rtol)
            print(f"[info] {case.name} chained dgamma element-wise: {case.C - bad}/{case.C} within "
                  f"atol=rtol={atol}", flush=True)
            err = np.max(np.abs(got - tdg))
            assert err <= atol + rtol * np.max(np.abs(tdg)), err
        else:
            assert_close(dg2, tdg, case.dtype, f"{case.name} chain dgamma")
    del xd, gd, dyd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_pages_model_shape(dtype):
    run_rms(W.rmsnorm_gpt2_case(dtype))


@pytest.mark.parametrize("C", W.LAYERNORM_C_SWEEP)
def test_hidden_size_sweep(C):
    run_rms(W.rmsnorm_sweep_case(16384, C))


def test_encoder_rows_fp32():
    # fp32 over 32768 rows: the chained dgamma carries the fp32 rounding of every row's rstd;
    # see the LayerNorm tests for why that comparison is norm-wise.
    run_rms(W.rmsnorm_sweep_case(32768, 1024, torch.float32), chain_dgamma_normwise=True)


EDGE_C = gpu_cases.NORM_EDGE_C


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("C", EDGE_C)
def test_bucket_boundaries_and_ragged_rows(C, dtype):
    for N in (1, 7, 1031):
        case = W.layernorm_case(f"rms-edge-N{N}-C{C}-{dtype}", N, C, dtype=dtype,
                                seed_base=7500 + C, row_offset_var=1.0, eps=W.RMS_EPS)
        run_rms(case, chain=False, edge=True)


@pytest.mark.parametrize("N,C,dtype", [(6141, 512, torch.float16), (10237, 1000, torch.float16)])
def test_backward_odd_row_loop_trip_counts(N, C, dtype):
    """One-wave backward rows with deferred stores and an odd trip count of three or more
    (the row loop is unrolled by two): see the LayerNorm test of the same name."""
    case = W.layernorm_case(f"rms-odd-trips-N{N}-C{C}-{dtype}", N, C, dtype=dtype,
                            seed_base=7800 + C, row_offset_var=1.0, eps=W.RMS_EPS)
    run_rms(case, chain=False)


@pytest.mark.parametrize("N,C", gpu_cases.NORM_LONG_F16)
def test_long_ragged_launch(N, C):
    """Long launches with ragged row counts: see the LayerNorm test of the same name."""
    case = W.layernorm_case(f"rms-long-N{N}-C{C}", N, C, dtype=torch.float16, seed_base=7950 + C,
                            row_offset_var=1.0, eps=W.RMS_EPS)
    run_rms(case)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_zero_rows(dtype):
    """x = 0: y = 0, rstd = 1/sqrt(eps), and dx = rstd * gamma * dy exactly in form."""
    N, C = 16, 512
    x = torch.zeros(N, C, dtype=dtype, device=DEV)
    g = W.uniform((C,), 7600, 0.5, 1.5).to(dtype).to(DEV)
    dy = W.normal((N, C), 7601).to(dtype).to(DEV)
    say("zero rows", dtype)
    y, rstd = lnr.rmsnorm_fw(x, g, W.RMS_EPS)
    dx, dg = lnr.rmsnorm_bw(dy, x, g, rstd)
    torch.cuda.synchronize()
    assert int(y.count_nonzero()) == 0
    r = 1.0 / np.sqrt(np.float32(W.RMS_EPS))
    np.testing.assert_allclose(rstd.cpu().numpy(), r, rtol=1e-6)
    ref = r * g.double().cpu().numpy().reshape(1, C) * dy.double().cpu().numpy()
    assert_close(dx, ref, dtype, "zero-row dx")
    assert int(dg.count_nonzero()) == 0


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_and_bitwise_determinism(dtype):
    case = W.rmsnorm_sweep_case(3000, 1024, dtype)
    x, g, dy = (t.to(DEV) for t in (case.x, case.gamma, case.dy))
    say(case.name, dtype)
    y1, r1 = lnr.rmsnorm_fw(x, g, case.eps)
    y2, r2 = lnr.rmsnorm_fw(x, g, case.eps)
    xi = x.clone()
    yi, ri = lnr.rmsnorm_fw(xi, g, case.eps, y=xi)
    a = lnr.rmsnorm_bw(dy, x, g, r1)
    c = lnr.rmsnorm_bw(dy, x, g, r1)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, xi)
    assert torch.equal(r1, r2) and torch.equal(r1, ri)
    for u, v in zip(a, c):
        assert torch.equal(u, v)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_unaligned_buffers_take_the_fallback(dtype):
    case = W.layernorm_case("rms-unaligned", 300, 512, dtype=dtype, seed_base=7700,
                            row_offset_var=1.0, eps=W.RMS_EPS)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:].copy_(t.reshape(-1).to(DEV))
        return buf[1:].view(t.shape)

    x, g, dy = shifted(case.x), shifted(case.gamma), shifted(case.dy)
    say(case.name, dtype)
    y, rstd = lnr.rmsnorm_fw(x, g, case.eps)
    dx, dg = lnr.rmsnorm_bw(dy, x, g, rstd)
    torch.cuda.synchronize()
    x64, g64, dy64 = case.x.double().numpy(), case.gamma.double().numpy(), case.dy.double().numpy()
    y_ref, _ = oracle.rmsnorm_fw(x64, g64, case.eps)
    dx_ref, dg_ref = oracle.rmsnorm_bw(x64, dy64, g64, case.eps)
    assert_close(y, y_ref, dtype, "unaligned y")
    assert_close(dx, dx_ref, dtype, "unaligned dx")
    assert_close(dg, dg_ref, dtype, "unaligned dgamma")


def test_zero_rows_count_gives_zero_dgamma():
    C = 1024
    x = torch.empty(0, C, dtype=torch.float16, device=DEV)
    g = torch.ones(C, dtype=torch.float16, device=DEV)
    r = torch.empty(0, dtype=torch.float32, device=DEV)
    dg = torch.full((C,), 7.0, dtype=torch.float16, device=DEV)
    say("N=0 rmsnorm backward")
    lnr.rmsnorm_bw(x, x, g, r, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)
