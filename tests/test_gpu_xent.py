"""GPU parity of cross_entropy_fw / cross_entropy_bw (through the C ABI) against the fp64
oracle: the textbook softmax cross-entropy over a vocabulary (the L10 page's third reduce
kernel; no formula on the pages).

  * forward: loss and lse (fp32 outputs) on identical stored logits, every row, at
    atol = rtol = 1e-5 for both storage types: the outputs are fp32 computed from exactly
    representable inputs, and the fp32 sum of V terms is relatively accurate to about
    1e-6 (at most ~1.3e-5 for V = 50001), so lse and loss (magnitude ~10) meet 1e-5 + 1e-5*|ref|;
  * backward on identical inputs: the GPU receives the oracle's lse rounded to fp32 and is
    compared, element by element, with the oracle's backward on that same lse, at the
    storage type's tolerance; plus the relative accuracy of the probabilities, which the
    absolute tolerance alone would not see (p ~ 1/V ~ 2e-5): |gpu - ref| <= r * (|ref| +
    |g| p) + floor, with r = 2e-3 and floor = 2^-24 for fp16 storage (half-ulp rounding,
    subnormals included) and r = 1e-4, floor = 1e-12 for fp32 (exp2 of an fp32 argument);
    the |g| p term covers the cancellation in g (p - 1) at the target when p is near 1;
  * each gradient row sums to zero up to storage rounding: |sum_j dz_ij| <= c |g_i| + V 2^-25
    (the last term only for fp16: most entries g p are fp16 subnormals, each rounded by up
    to half the subnormal step 2^-24, and because those values cluster at small magnitudes
    within a step the rounding errors need not cancel across the row).
"""
import numpy as np
import pytest
import torch

import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import TOL, assert_close, say, to_host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OUT_TOL = 1e-5  # fp32 loss / lse


def check_dz(dz, ref, dtype, what, z64, lse64, g):
    """g: the per-row factor dloss_i * scale, 0 for ignored rows."""
    assert_close(dz, ref, dtype, what)
    got = to_host64(dz) if isinstance(dz, torch.Tensor) else dz
    rt, floor = (2e-3, 2.0 ** -24) if dtype == torch.float16 else (1e-4, 1e-12)
    gp = np.abs(np.asarray(g, np.float64)).reshape(-1, 1) * np.exp(z64 - lse64.reshape(-1, 1))
    err = np.abs(got - ref)
    lim = rt * (np.abs(ref) + gp) + floor
    bad = ~(err <= lim)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - lim, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the relative bound; worst "
                             f"at {i}: gpu={got[i]!r} oracle={ref[i]!r}")
    V = got.shape[1]
    rs = np.abs(got.sum(axis=1))
    if dtype == torch.float16:
        lim_rows = 3e-3 * np.abs(g) + V * 2.0 ** -25
    else:
        lim_rows = 3e-5 * np.abs(g) + 1e-9
    assert np.all(rs <= lim_rows), float(np.max(rs - lim_rows))


def run_xent(case, with_dloss=True, scale=1.0):
    say(case.name, "oracle forward")
    z64 = case.logits.double().numpy()
    t = case.target.numpy()
    loss_ref, lse_ref = oracle.xent_fw(z64, t, case.ignore_index)

    say(case.name, "GPU forward")
    zd, td = case.logits.to(DEV), case.target.to(DEV)
    loss, lse = lnr.cross_entropy_fw(zd, td, case.ignore_index)
    torch.cuda.synchronize()
    assert_close(loss, loss_ref, torch.float32, f"{case.name} loss", atol=OUT_TOL, rtol=OUT_TOL)
    assert_close(lse, lse_ref, torch.float32, f"{case.name} lse", atol=OUT_TOL, rtol=OUT_TOL)

    say(case.name, "oracle backward (given fp32 lse)")
    l32 = torch.from_numpy(lse_ref).float()
    dl = case.dloss if with_dloss else torch.ones(case.N)
    g = dl.double().numpy() * scale
    dz_ref = oracle.xent_bw_given_lse(z64, t, l32.numpy(), g, case.ignore_index)
    say(case.name, "GPU backward")
    dz = lnr.cross_entropy_bw(zd, td, l32.to(DEV), case.dloss.to(DEV) if with_dloss else None,
                              scale, case.ignore_index)
    torch.cuda.synchronize()
    g_rows = np.where(t == case.ignore_index, 0.0, g)
    check_dz(dz, dz_ref, case.dtype, f"{case.name} dlogits", z64, l32.double().numpy(), g_rows)
    del zd, dz
    torch.cuda.empty_cache()


@pytest.mark.parametrize("V", W.XENT_VOCABS)
def test_tokens_fp16(V):
    run_xent(W.xent_tokens_case(V, torch.float16))


def test_tokens_fp32():
    run_xent(W.xent_tokens_case(32000, torch.float32, N=2048), with_dloss=False, scale=1.0 / 2048)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("V", W.XENT_VOCABS)
def test_few_rows_split_over_workgroups(V, dtype):
    """64 rows (a decoding batch): the backward splits each row over several workgroups; the
    forward streams each row in one workgroup (rows of up to 256 KB are not split)."""
    assert lnr.cross_entropy_fw_workspace_bytes(64, V, dtype) == 0
    run_xent(W.xent_case(f"xent-split-64x{V}-{dtype}", 64, V, dtype=dtype, seed_base=7800 + V % 97))


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("N", [1, 5])
def test_long_rows_split_forward(N, dtype):
    """Rows above 256 KB (140001 logits) with few rows: the forward splits each row over
    workgroups and combines the chunk partials in a second kernel, in chunk order."""
    assert lnr.cross_entropy_fw_workspace_bytes(N, 140001, dtype) > 0
    run_xent(W.xent_case(f"xent-long-{N}x140001-{dtype}", N, 140001, dtype=dtype, seed_base=7700 + N))


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 64, 1000, 1024, 4097, 65536])
def test_vocabulary_edges(V, dtype):
    for N in (1, 3, 33):
        run_xent(W.xent_case(f"xent-edge-{N}x{V}-{dtype}", N, V, dtype=dtype,
                             seed_base=7900 + V % 89, logit_std=3.0, ignore_frac=0.2))


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_backward_and_determinism(dtype):
    case = W.xent_case("xent-inplace", 300, 4099, dtype=dtype, seed_base=8100)
    zd, td = case.logits.to(DEV), case.target.to(DEV)
    say(case.name, dtype)
    l1, s1 = lnr.cross_entropy_fw(zd, td)
    l2, s2 = lnr.cross_entropy_fw(zd, td)
    d1 = lnr.cross_entropy_bw(zd, td, s1, None, 0.5)
    d2 = lnr.cross_entropy_bw(zd, td, s1, None, 0.5)
    zi = zd.clone()
    di = lnr.cross_entropy_bw(zi, td, s1, None, 0.5, dlogits=zi)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(s1, s2)
    assert torch.equal(d1, d2) and torch.equal(d1, di)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("NV", [(50, 1001), (20, 20011), (3, 140001)])
@pytest.mark.parametrize("dz_phase", ["line", "16B", "scalar"])
def test_unaligned_and_phase_shifted_buffers(dz_phase, NV, dtype):
    """Logits one element past a 16-byte boundary (vector middle after a scalar head of up to
    a 128-byte line), and the gradient buffer at the logits' 128-byte phase ("line"), at their
    16-byte phase only ("16B": 16-byte vectors from dz's first 16-byte boundary), or at
    another 16-byte phase ("scalar": every element on its own). 20 x 20011 splits each row
    of the backward over several workgroups, 3 x 140001 those of both passes; inner chunk
    boundaries are rounded to lines."""
    N, V = NV
    case = W.xent_case(f"xent-unaligned-{N}x{V}", N, V, dtype=dtype, seed_base=8200 + N)
    es = torch.empty((), dtype=dtype).element_size()
    buf = torch.empty(case.N * case.V + 8, dtype=dtype, device=DEV)
    zd = buf[1:1 + case.N * case.V].view(case.N, case.V)
    zd.copy_(case.logits.to(DEV))
    td = case.target.to(DEV)
    say(case.name, dtype, dz_phase)
    loss, lse = lnr.cross_entropy_fw(zd, td)
    k = {"line": 1, "16B": 1 + 16 // es, "scalar": 2}[dz_phase]
    out = torch.empty(case.N * case.V + 80, dtype=dtype, device=DEV)
    dz = out[k:k + case.N * case.V].view(case.N, case.V)
    shift = (dz.data_ptr() - zd.data_ptr()) % 128
    assert {"line": shift == 0, "16B": shift == 16, "scalar": shift % 16 != 0}[dz_phase]
    lnr.cross_entropy_bw(zd, td, lse, case.dloss.to(DEV), 1.0, dlogits=dz)
    torch.cuda.synchronize()
    z64, t = case.logits.double().numpy(), case.target.numpy()
    loss_ref, lse_ref = oracle.xent_fw(z64, t)
    assert_close(loss, loss_ref, torch.float32, "unaligned loss", atol=OUT_TOL, rtol=OUT_TOL)
    l64 = lse.cpu().double().numpy()
    dz_ref = oracle.xent_bw_given_lse(z64, t, l64, case.dloss.double().numpy())
    g_rows = np.where(t == case.ignore_index, 0.0, case.dloss.double().numpy())
    check_dz(dz, dz_ref, dtype, f"{dz_phase} dlogits", z64, l64, g_rows)


def test_large_logits_and_invalid_targets():
    """+-1e4 logits stay finite; a target outside [0, V) (other than the ignore index) gives a
    NaN loss and a NaN gradient row, found by the kernel's own bounds check."""
    z = torch.tensor([[1e4, -1e4, 0.0, 1e4 - 1.0], [-1e4, -1e4 + 2.0, -1e4 + 1.0, -1e4],
                      [0.5, 0.25, 0.125, 0.0], [1.0, 2.0, 3.0, 4.0]], dtype=torch.float32)
    t = torch.tensor([3, 0, 4, -7], dtype=torch.int64)
    say("large logits / invalid targets")
    loss, lse = lnr.cross_entropy_fw(z.to(DEV), t.to(DEV))
    dz = lnr.cross_entropy_bw(z.to(DEV), t.to(DEV), lse)
    torch.cuda.synchronize()
    loss_ref, lse_ref = oracle.xent_fw(z.double().numpy(), t.numpy())
    lo = loss.cpu().double().numpy()
    assert np.all(np.isfinite(lo[:2])) and np.all(np.isnan(lo[2:]))
    np.testing.assert_allclose(lo[:2], loss_ref[:2], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(lse.cpu().double().numpy(), lse_ref, rtol=1e-6)
    d = dz.cpu().double().numpy()
    assert np.all(np.isfinite(d[:2])) and np.all(np.isnan(d[2:]))
    # the reference takes the kernel's own fp32 lse: at |z| ~ 1e4 the fp32 rounding of lse
    # alone moves p by ~5e-4, which is the saved statistic, not the backward, speaking
    ref = oracle.xent_bw_given_lse(z.double().numpy()[:2], t.numpy()[:2],
                                   lse.cpu().double().numpy()[:2], np.ones(2))
    np.testing.assert_allclose(d[:2], ref, rtol=1e-5, atol=1e-6)


def test_zero_rows():
    z = torch.empty(0, 100, dtype=torch.float16, device=DEV)
    t = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, lse = lnr.cross_entropy_fw(z, t)
    dz = lnr.cross_entropy_bw(z, t, lse)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and dz.numel() == 0
