"""GPU parity of attn_softmax_fw / attn_softmax_bw (through the C ABI) against the fp64 oracle.

Every element of every output is compared with the oracle on the same stored inputs:
  * forward: the seeded scores and mask of each workload;
  * backward: y = the oracle's forward output rounded to the storage dtype, and the seeded dy,
    so both sides see identical bits and masked positions hold exact zeros on both;
  * chained: the GPU forward feeding the GPU backward, against oracle forward -> backward.
Workloads 1-3 and 5 run at their full sizes, in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import gpu_cases
import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import TOL, assert_close, say, to_host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(t):
    return None if t is None else t.to(DEV)


def run_case(case, check_chain=True):
    """Forward, backward and chained parity for one SoftmaxCase at its full size."""
    say(case.name, "oracle forward")
    x64 = case.x.double().numpy()
    m64 = None if case.mask is None else case.mask.double().numpy()
    y_ref = oracle.softmax_fw(x64, m64, case.causal)
    del x64

    say(case.name, "GPU forward")
    xd, md = _dev(case.x), _dev(case.mask)
    y = lnr.attn_softmax_fw(xd, md, case.causal)
    torch.cuda.synchronize()
    assert_close(y, y_ref, case.dtype, f"{case.name} fw")
    # masked and future positions are exact zeros
    yh = y.cpu()
    assert torch.all(yh[torch.from_numpy(y_ref == 0.0)] == 0)

    # backward on identical stored inputs: y_T = oracle y rounded to the storage dtype
    y_t = torch.from_numpy(y_ref).to(case.dtype)
    del y_ref
    say(case.name, "oracle backward")
    dx_ref = oracle.softmax_bw(y_t.double().numpy(), case.dy.double().numpy())
    say(case.name, "GPU backward")
    dyd = _dev(case.dy)
    dx = lnr.attn_softmax_bw(dyd, _dev(y_t))
    torch.cuda.synchronize()
    assert_close(dx, dx_ref, case.dtype, f"{case.name} bw")
    del dx_ref, dx

    if check_chain:
        say(case.name, "chained fw -> bw")
        dx_chain = lnr.attn_softmax_bw(dyd, y)
        torch.cuda.synchronize()
        # oracle chain: fp64 y (never rounded) into the fp64 backward
        yc = oracle.softmax_fw(case.x.double().numpy(), m64, case.causal)
        dxc_ref = oracle.softmax_bw(yc, case.dy.double().numpy())
        del yc
        atol, rtol = TOL[case.dtype]
        # the GPU chain also carries the storage rounding of y into the backward: allow it
        scale = 2.0 if case.dtype == torch.float16 else 1.0
        assert_close(dx_chain, dxc_ref, case.dtype, f"{case.name} chain", atol=atol * scale,
                     rtol=rtol * scale)
    del xd, md, dyd, y
    torch.cuda.empty_cache()


def test_workload1_tiny_fp32():
    [case], _ = W.workload1()
    run_case(case)


def test_workload2_gpt2_fp16():
    [case], _ = W.workload2()
    run_case(case)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tk", W.SOFTMAX_TK_SWEEP)
def test_workload3_row_length_sweep(Tk, causal):
    run_case(W.workload3_case(Tk, causal), check_chain=False)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_workload5_encoder_layer(dtype):
    run_case(W.workload5_softmax(dtype), check_chain=False)


# ------------------------------------------------------------------------- edge cases

EDGE_TK = gpu_cases.SOFTMAX_EDGE_TK


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("Tk", EDGE_TK)
def test_bucket_boundaries_and_ragged_rows(Tk, dtype):
    # B*H*Tq = 3*5*Tq rows: not a multiple of any rows-per-block, a ragged last block.
    for causal, B, H in ((True, 3, 5), (False, 2, 3)):
        Tq = Tk if causal else 7
        lo = max(1, Tk // 2)
        case = W.softmax_case(f"edge-Tk{Tk}-{'causal' if causal else 'full'}-{dtype}", B, H, Tq, Tk,
                              causal=causal, dtype=dtype, seed_base=9000 + Tk, len_range=(lo, Tk))
        run_case(case, check_chain=False)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_equals_out_of_place_and_runs_are_bitwise_identical(dtype):
    case = W.softmax_case("inplace", 4, 4, 128, 128, causal=True, dtype=dtype, seed_base=9100,
                          len_range=(64, 128))
    say(case.name, dtype, "GPU")
    x, m, dy = _dev(case.x), _dev(case.mask), _dev(case.dy)
    y1 = lnr.attn_softmax_fw(x, m, True)
    y2 = lnr.attn_softmax_fw(x, m, True)
    xi = x.clone()
    lnr.attn_softmax_fw(xi, m, True, out=xi)
    d1 = lnr.attn_softmax_bw(dy, y1)
    d2 = lnr.attn_softmax_bw(dy, y1)
    dyi = dy.clone()
    lnr.attn_softmax_bw(dyi, y1, dinp=dyi)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, xi)
    assert torch.equal(d1, d2) and torch.equal(d1, dyi)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_unaligned_buffers_take_the_fallback_with_the_same_results(dtype):
    # Offset every buffer by one element: not 16-byte aligned, so the element-wise kernel runs.
    case = W.softmax_case("unaligned", 2, 2, 64, 64, causal=False, dtype=dtype, seed_base=9200,
                          len_range=(20, 64))
    n = case.x.numel()
    say(case.name, dtype, "GPU")
    xb = torch.empty(n + 1, dtype=dtype, device=DEV)
    xb[1:].copy_(case.x.reshape(-1).to(DEV))
    x_un = xb[1:].view(case.x.shape)
    yb = torch.empty(n + 1, dtype=dtype, device=DEV)
    y_un = yb[1:].view(case.x.shape)
    m = _dev(case.mask)
    lnr.attn_softmax_fw(x_un, m, False, out=y_un)
    torch.cuda.synchronize()
    y_ref = oracle.softmax_fw(case.x.double().numpy(), case.mask.double().numpy(), False)
    assert_close(y_un, y_ref, dtype, "unaligned fw")


def test_fully_masked_rows_are_zero_and_finite_masks_shift_scores():
    B, H, T = 2, 3, 64
    x = W.normal((B, H, T, T), 9300).to(torch.float32)
    mask = torch.zeros(B, T)
    mask[0, :] = float("-inf")                         # batch 0: every key removed
    mask[1, :] = torch.linspace(-3.0, 2.0, T)          # batch 1: finite additive values
    say("fully-masked", "GPU")
    y = lnr.attn_softmax_fw(x.to(DEV), mask.to(DEV), False)
    torch.cuda.synchronize()
    assert torch.all(y[0] == 0)
    y_ref = oracle.softmax_fw(x.double().numpy(), mask.double().numpy(), False)
    assert_close(y, y_ref, torch.float32, "finite mask")


def test_large_magnitude_scores_fp32():
    x = (W.normal((2, 4, 256, 256), 9400) * 1e4).to(torch.float32)
    say("large-magnitude", "GPU")
    y = lnr.attn_softmax_fw(x.to(DEV), None, True)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    assert_close(y, oracle.softmax_fw(x.double().numpy(), None, True), torch.float32, "1e4 scores")


def test_empty_inputs_launch_nothing():
    for shape in ((0, 2, 4, 4), (2, 0, 4, 4), (2, 2, 0, 4)):
        x = torch.empty(shape, dtype=torch.float16, device=DEV)
        y = lnr.attn_softmax_fw(x, None, False)
        d = lnr.attn_softmax_bw(x, y)
        assert y.shape == shape and d.shape == shape
    torch.cuda.synchronize()


def test_row_sums_at_full_size_workload5():
    # Property that holds at any size: every unmasked row sums to 1 (fp16 rounding allowed).
    case = W.workload5_softmax(torch.float16)
    say(case.name, "row sums")
    y = lnr.attn_softmax_fw(case.x.to(DEV), case.mask.to(DEV), False)
    s = y.float().sum(-1)
    torch.cuda.synchronize()
    # each stored probability carries at most 2^-11 relative rounding, and they sum to 1
    assert torch.all((s - 1.0).abs() <= 2.0 ** -11 + 1e-4)
    Lb = case.lengths.to(DEV)
    j = torch.arange(case.Tk, device=DEV)
    padded = (j.view(1, 1, 1, -1) >= Lb.view(-1, 1, 1, 1)).expand_as(y)
    assert torch.all(y[padded] == 0)
