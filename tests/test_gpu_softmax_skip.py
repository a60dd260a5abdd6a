"""GPU parity of attn_softmax_fw_skip / attn_softmax_bw_skip (through the C ABI).

These entry points compute the same softmax as attn_softmax_fw / attn_softmax_bw but do not read
16-byte score runs whose keys are all masked (after the query when causal, or under -inf mask
entries). Checked here:
  * against the fp64 oracle, element by element, at the storage tolerance: the forward on the
    seeded inputs, the backward on identical stored inputs (y = the oracle's output rounded to
    the storage type), and the chained pass;
  * equality with the dense entry points on the same inputs (a property of the design: the
    skipped runs contribute exactly 0 either way; equality is numeric, so -0 equals +0). Both
    directions are equal where the two use the same lanes per row and vectors per lane
    (lnr_softmax_plan). Where they do not, a row's sum adds the same terms in another order:
    two such fp32 sums of Tk terms differ by at most 2(Tk - 1) u relative (u = 2^-24), so the
    forward outputs (each term times the reciprocal sum) agree to (2 Tk + 4) u relative, or
    one unit in the last place of the storage type where that is larger; the backward
    outputs agree to one unit in the last place;
  * that skipped runs are really not read: NaN planted in them leaves the outputs finite and
    equal to the oracle's on clean inputs, where a read would poison the row (NaN + -inf and
    0 * NaN are NaN);
  * fully masked batches, every bucket with ragged row counts, unaligned buffers (the dense
    fallback), in place.
"""
import numpy as np
import pytest
import torch

import gpu_cases
import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import TOL, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(t):
    return None if t is None else t.to(DEV)


def assert_equal_or_one_ulp(a, b, what):
    """a == b element by element, or within one unit in the last place of b's storage type."""
    if torch.equal(a, b):
        return
    an = a.detach().cpu().numpy()
    bn = b.detach().cpu().numpy()
    ulp = np.spacing(np.abs(bn)).astype(np.float64)
    diff = np.abs(an.astype(np.float64) - bn.astype(np.float64))
    bad = ~(diff <= ulp)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ by more than one ulp"


def assert_same_sum_reordered(a, b, Tk, what):
    """a and b are the same softmax rows normalised by two fp32 sums of the same Tk terms in
    different orders: |a - b| <= max(ulp(b), (2 Tk + 4) u |b|), u = 2^-24."""
    if torch.equal(a, b):
        return
    an = a.detach().cpu().double().numpy()
    bn = b.detach().cpu().numpy()
    ulp = np.spacing(np.abs(bn)).astype(np.float64)
    bound = np.maximum(ulp, (2 * Tk + 4) * 2.0 ** -24 * np.abs(bn.astype(np.float64)))
    diff = np.abs(an - bn.astype(np.float64))
    worst = float(np.max(diff / bound))
    print(f"[parity] {what}: worst difference / bound {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{what}: {int((diff > bound).sum())} elements beyond the reordering bound"


def same_plan(case, backward):
    """Whether the dense and the skipping kernel reduce a row of this case in the same order
    (the same lanes per row and vectors per lane)."""
    code = lnr.LNR_F16 if case.dtype == torch.float16 else lnr.LNR_F32
    Tk = case.x.shape[-1]
    return (lnr.softmax_plan(Tk, code, backward=backward)[1:]
            == lnr.softmax_plan(Tk, code, backward=backward, skip=True)[1:])


def run_skip(case, check_chain=True):
    say(case.name, "oracle forward")
    x64 = case.x.double().numpy()
    m64 = None if case.mask is None else case.mask.double().numpy()
    y_ref = oracle.softmax_fw(x64, m64, case.causal)
    del x64

    say(case.name, "GPU forward (skip and dense)")
    xd, md = _dev(case.x), _dev(case.mask)
    y = lnr.attn_softmax_fw_skip(xd, md, case.causal)
    y_dense = lnr.attn_softmax_fw(xd, md, case.causal)
    torch.cuda.synchronize()
    assert_close(y, y_ref, case.dtype, f"{case.name} fw_skip")
    if same_plan(case, backward=False):
        assert torch.equal(y, y_dense), f"{case.name}: fw_skip differs from the dense forward"
    else:
        assert_same_sum_reordered(y, y_dense, case.x.shape[-1],
                                  f"{case.name}: fw_skip against the dense forward")
    del y_dense

    y_t = torch.from_numpy(y_ref).to(case.dtype)
    del y_ref
    say(case.name, "oracle backward")
    dx_ref = oracle.softmax_bw(y_t.double().numpy(), case.dy.double().numpy())
    say(case.name, "GPU backward (skip and dense)")
    dyd, ytd = _dev(case.dy), _dev(y_t)
    dx = lnr.attn_softmax_bw_skip(dyd, ytd, md, case.causal)
    dx_dense = lnr.attn_softmax_bw(dyd, ytd)
    torch.cuda.synchronize()
    assert_close(dx, dx_ref, case.dtype, f"{case.name} bw_skip")
    if same_plan(case, backward=True):
        assert torch.equal(dx, dx_dense), f"{case.name}: bw_skip differs from the dense backward"
    else:
        assert_equal_or_one_ulp(dx, dx_dense, f"{case.name}: bw_skip against the dense backward")
    del dx_ref, dx, dx_dense, ytd

    if check_chain:
        say(case.name, "chained fw_skip -> bw_skip")
        dxc = lnr.attn_softmax_bw_skip(dyd, y, md, case.causal)
        torch.cuda.synchronize()
        yc = oracle.softmax_fw(case.x.double().numpy(), m64, case.causal)
        dxc_ref = oracle.softmax_bw(yc, case.dy.double().numpy())
        del yc
        atol, rtol = TOL[case.dtype]
        scale = 2.0 if case.dtype == torch.float16 else 1.0
        assert_close(dxc, dxc_ref, case.dtype, f"{case.name} chain", atol=atol * scale,
                     rtol=rtol * scale)
    del xd, md, dyd, y
    torch.cuda.empty_cache()


def test_workload1_tiny_fp32():
    [case], _ = W.workload1()
    run_skip(case)


def test_workload2_gpt2_causal_fp16():
    [case], _ = W.workload2()
    run_skip(case)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Tk", W.SOFTMAX_TK_SWEEP)
def test_workload3_row_length_sweep(Tk, causal):
    run_skip(W.workload3_case(Tk, causal), check_chain=False)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_workload5_padded_encoder(dtype):
    run_skip(W.workload5_softmax(dtype), check_chain=False)


EDGE_TK = gpu_cases.SKIP_EDGE_TK


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("Tk", EDGE_TK)
def test_buckets_ragged_rows_and_odd_lengths(Tk, dtype):
    # 3*5*Tq rows: a ragged last block. Odd Tk (1, 31, 33, 100, 2047 at fp16) takes the dense
    # element-wise path through the same entry point.
    for causal, B, H in ((True, 3, 5), (False, 2, 3)):
        Tq = Tk if causal else 7
        case = W.softmax_case(f"skip-edge-Tk{Tk}-{'causal' if causal else 'full'}-{dtype}", B, H, Tq,
                              Tk, causal=causal, dtype=dtype, seed_base=9700 + Tk,
                              len_range=(max(1, Tk // 3), Tk))
        run_skip(case, check_chain=False)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_fully_masked_batches_and_no_mask(dtype):
    """A batch whose every key is masked reads no scores and writes zero rows; a causal call
    without a mask skips by index alone."""
    B, H, T = 3, 4, 96
    case = W.softmax_case("skip-fully-masked", B, H, T, T, causal=False, dtype=dtype,
                          seed_base=9800, len_range=(1, T))
    case.mask[1, :] = float("-inf")
    run_skip(case)
    case2 = W.softmax_case("skip-causal-nomask", B, H, T, T, causal=True, dtype=dtype,
                           seed_base=9810)
    run_skip(case2)


def _skipped_runs(case, V):
    """Boolean [B, H, Tq, Tk]: elements of 16-byte runs whose keys are all masked."""
    B, H, Tq, Tk = case.B, case.H, case.Tq, case.Tk
    j = np.arange(Tk)
    closed = np.zeros((B, 1, Tq, Tk), bool)
    if case.mask is not None:
        closed |= (case.mask.numpy() == -np.inf)[:, None, None, :]
    if case.causal:
        closed |= (j[None, :] > np.arange(Tq)[:, None])[None, None]
    runs = closed.reshape(B, 1, Tq, Tk // V, V).all(axis=-1)
    return np.broadcast_to(np.repeat(runs, V, axis=-1), (B, H, Tq, Tk))


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_skipped_runs_are_not_read(causal, dtype):
    V = 8 if dtype == torch.float16 else 4
    B, H, T = 4, 3, 256
    case = W.softmax_case(f"skip-nan-{'causal' if causal else 'full'}", B, H, T, T, causal=causal,
                          dtype=dtype, seed_base=9900, len_range=(40, 200))
    sk = _skipped_runs(case, V)
    assert sk.any() and not sk.all()
    say(case.name, dtype, f"{int(sk.sum())} planted NaN")
    m64 = case.mask.double().numpy()
    y_ref = oracle.softmax_fw(case.x.double().numpy(), m64, causal)
    x_nan = case.x.clone()
    x_nan.numpy()[sk] = np.nan
    md = _dev(case.mask)
    y = lnr.attn_softmax_fw_skip(_dev(x_nan), md, causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    assert_close(y, y_ref, dtype, f"{case.name} fw with NaN in skipped runs")

    y_t = torch.from_numpy(y_ref).to(dtype)
    dx_ref = oracle.softmax_bw(y_t.double().numpy(), case.dy.double().numpy())
    y_nan, dy_nan = y_t.clone(), case.dy.clone()
    y_nan.numpy()[sk] = np.nan
    dy_nan.numpy()[sk] = np.nan
    dx = lnr.attn_softmax_bw_skip(_dev(dy_nan), _dev(y_nan), md, causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dx).all())
    assert_close(dx, dx_ref, dtype, f"{case.name} bw with NaN in skipped runs")
    assert bool((dx.cpu().numpy()[sk] == 0).all())


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_and_unaligned_fallback(dtype):
    case = W.softmax_case("skip-inplace", 2, 4, 128, 128, causal=True, dtype=dtype, seed_base=9950,
                          len_range=(64, 128))
    say(case.name, dtype)
    x, m, dy = _dev(case.x), _dev(case.mask), _dev(case.dy)
    y = lnr.attn_softmax_fw_skip(x, m, True)
    xi = x.clone()
    lnr.attn_softmax_fw_skip(xi, m, True, out=xi)
    dx = lnr.attn_softmax_bw_skip(dy, y, m, True)
    dyi = dy.clone()
    lnr.attn_softmax_bw_skip(dyi, y, m, True, dinp=dyi)
    # one element past a 16-byte boundary: the dense element-wise kernels run
    buf = torch.empty(x.numel() + 8, dtype=dtype, device=DEV)
    xs = buf[1:1 + x.numel()].view(x.shape)
    xs.copy_(x)
    ys = lnr.attn_softmax_fw_skip(xs, m, True)
    torch.cuda.synchronize()
    assert torch.equal(y, xi) and torch.equal(dx, dyi)
    y_ref = oracle.softmax_fw(case.x.double().numpy(), case.mask.double().numpy(), True)
    assert_close(ys, y_ref, dtype, "unaligned fw_skip")
    assert_close(y, y_ref, dtype, "fw_skip")
