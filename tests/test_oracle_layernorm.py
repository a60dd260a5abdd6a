"""Pins for the oracle's LayerNorm and RMSNorm (forward and backward), CPU only.

What the pages fix ("CMU 11-868 L10 ...", "Technique 2"; "CMU 11-868 HW4 ...", "Problem
structure and scoring"): sigma = sqrt(mu(x^2) - mu(x)^2 + eps) with eps = 1e-8, the input
gradient built from the two row sums of gamma*dy and gamma*dy*xhat, and dgamma/dbeta as sums
across rows. RMSNorm follows "FastTransformer ...", section 5.4. The oracle is pinned against
closed forms, invariants, central finite differences and independent fp64 library routines
(torch.nn.functional.layer_norm / rms_norm and their autograd).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from layernorm_reduction_amd import workloads as W

EPS = 1e-8


def _case(N, C, seed, offset_std=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, C)) + offset_std * rng.standard_normal((N, 1))
    gamma = rng.uniform(0.5, 1.5, C)
    beta = rng.normal(0.0, 0.3, C)
    dy = rng.standard_normal((N, C))
    return x, gamma, beta, dy


# ---------------------------------------------------------------- forward

def test_unit_affine_output_has_zero_mean_and_closed_form_second_moment():
    x, _, _, _ = _case(37, 53, 1, offset_std=3.0)
    C = x.shape[1]
    y, mean, rstd = oracle.layernorm_fw(x, np.ones(C), np.zeros(C), EPS)
    v = x.var(axis=1)                                    # biased variance (numpy routine)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), v / (v + EPS), rtol=1e-13)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-14)


def test_one_pass_sigma_identity():
    # The L10 rewrite: sigma = sqrt(mu(x^2) - mu(x)^2 + eps) equals the two-pass sigma.
    x, g, b, _ = _case(64, 1024, 2, offset_std=2.0)
    _, _, rstd = oracle.layernorm_fw(x, g, b, EPS)
    one_pass = np.sqrt(np.mean(x * x, axis=1) - np.mean(x, axis=1) ** 2 + EPS)
    np.testing.assert_allclose(1.0 / rstd, one_pass, rtol=1e-10)


def test_affine_invariance_of_normalised_output():
    x, g, b, _ = _case(9, 33, 3)
    y0, _, _ = oracle.layernorm_fw(x, g, b, EPS)
    y1, _, _ = oracle.layernorm_fw(3.5 * x - 11.0, g, b, EPS)
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-7)    # differs only through eps


def test_closed_forms_for_one_and_two_columns():
    rng = np.random.default_rng(4)
    x1 = rng.standard_normal((5, 1))
    beta1 = np.array([0.25])
    y1, _, _ = oracle.layernorm_fw(x1, np.array([2.0]), beta1, EPS)
    assert np.all(y1 == 0.25)                             # C = 1: y = beta exactly
    x2 = rng.standard_normal((6, 2))
    y2, _, _ = oracle.layernorm_fw(x2, np.ones(2), np.zeros(2), EPS)
    d = (x2[:, 0] - x2[:, 1]) / 2.0
    np.testing.assert_allclose(y2[:, 0], d / np.sqrt(d * d + EPS), rtol=1e-14)
    np.testing.assert_allclose(y2[:, 1], -d / np.sqrt(d * d + EPS), rtol=1e-14)


@pytest.mark.parametrize("N,C", [(7, 19), (64, 64), (3, 300)])
def test_forward_matches_torch_layer_norm(N, C):
    x, g, b, _ = _case(N, C, 5, offset_std=1.0)
    ref = F.layer_norm(torch.from_numpy(x), (C,), torch.from_numpy(g), torch.from_numpy(b), eps=EPS)
    y, _, _ = oracle.layernorm_fw(x, g, b, EPS)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_workload1_forward_matches_torch():
    _, [ln] = W.workload1()
    x, g, b = ln.x.double(), ln.gamma.double(), ln.beta.double()
    ref = F.layer_norm(x, (ln.C,), g, b, eps=ln.eps).numpy()
    y, _, _ = oracle.layernorm_fw(x.numpy(), g.numpy(), b.numpy(), ln.eps)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- backward

def _ln_loss(x, g, b, dy):
    y, _, _ = oracle.layernorm_fw(x, g, b, EPS)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("N,C", [(4, 8), (3, 5)])
def test_backward_matches_central_finite_differences(N, C):
    x, g, b, dy = _case(N, C, 6, offset_std=0.5)
    dx, dg, db = oracle.layernorm_bw(x, dy, g, EPS)
    h = 1e-6
    fdx = np.zeros_like(x)
    for i in range(N):
        for j in range(C):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fdx[i, j] = (_ln_loss(xp, g, b, dy) - _ln_loss(xm, g, b, dy)) / (2 * h)
    fdg = np.zeros(C)
    fdb = np.zeros(C)
    for j in range(C):
        gp = g.copy(); gp[j] += h
        gm = g.copy(); gm[j] -= h
        fdg[j] = (_ln_loss(x, gp, b, dy) - _ln_loss(x, gm, b, dy)) / (2 * h)
        bp = b.copy(); bp[j] += h
        bm = b.copy(); bm[j] -= h
        fdb[j] = (_ln_loss(x, g, bp, dy) - _ln_loss(x, g, bm, dy)) / (2 * h)
    np.testing.assert_allclose(dx, fdx, rtol=0, atol=2e-7)
    np.testing.assert_allclose(dg, fdg, rtol=0, atol=2e-7)
    np.testing.assert_allclose(db, fdb, rtol=0, atol=2e-7)


def test_backward_row_invariants():
    # sum_j dx_j = 0 and sum_j dx_j xhat_j = (1/sigma) (eps/(v+eps)) sum_j g_j xhat_j per row.
    x, g, _, dy = _case(21, 40, 7, offset_std=1.0)
    x[:, :] *= 1e-4                        # small variance makes the eps term visible
    dx = oracle.layernorm_bw_dx(x, dy, g, EPS)
    mu = x.mean(axis=1, keepdims=True)
    v = x.var(axis=1, keepdims=True)
    sigma = np.sqrt(v + EPS)
    xhat = (x - mu) / sigma
    gg = g * dy
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-9 * np.abs(dx).max())
    lhs = (dx * xhat).sum(axis=1)
    rhs = (1.0 / sigma[:, 0]) * (EPS / (v[:, 0] + EPS)) * (gg * xhat).sum(axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-7, atol=1e-9 * np.abs(dx).max())


def test_dbeta_is_column_sum_and_zero_gamma_gives_zero_dx():
    x, g, _, dy = _case(50, 17, 8)
    dx, dg, db = oracle.layernorm_bw(x, dy, g, EPS)
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-14, atol=1e-13)
    dx0 = oracle.layernorm_bw_dx(x, dy, np.zeros(17), EPS)
    assert np.all(dx0 == 0.0)


@pytest.mark.parametrize("N,C", [(6, 10), (64, 64), (33, 129)])
def test_backward_matches_torch_autograd(N, C):
    x, g, b, dy = _case(N, C, 9, offset_std=2.0)
    xt = torch.from_numpy(x).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    bt = torch.from_numpy(b).requires_grad_(True)
    F.layer_norm(xt, (C,), gt, bt, eps=EPS).backward(torch.from_numpy(dy))
    dx, dg, db = oracle.layernorm_bw(x, dy, g, EPS)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_dgamma_is_not_transposed():
    # N != C and distinct per-column dy scales: a swapped index would mix columns.
    x, g, _, dy = _case(11, 4, 10)
    dy = dy * np.array([1.0, 10.0, 100.0, 1000.0])
    _, dg, db = oracle.layernorm_bw(x, dy, g, EPS)
    xhat = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, keepdims=True) + EPS)
    np.testing.assert_allclose(dg, np.einsum("ij,ij->j", dy, xhat), rtol=1e-12)
    np.testing.assert_allclose(db, np.einsum("ij->j", dy), rtol=1e-14)


def test_given_stats_backward_equals_recomputing_backward_with_exact_stats():
    x, g, b, dy = _case(40, 70, 13, offset_std=2.0)
    _, mean, rstd = oracle.layernorm_fw(x, g, b, EPS)
    got = oracle.layernorm_bw_given_stats(x, dy, g, mean, rstd)
    ref = oracle.layernorm_bw(x, dy, g, EPS)
    for u, v in zip(got, ref):
        np.testing.assert_allclose(u, v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,C", [(9, 2), (17, 33), (64, 256)])
def test_given_stats_backward_matches_aten_layer_norm_backward(N, C):
    # aten's native layer-norm backward also takes mean and rstd as inputs: feed both the
    # fp32-rounded statistics (what a forward kernel stores), independent of recomputation.
    x, g, b, dy = _case(N, C, 14, offset_std=3.0)
    _, mean, rstd = oracle.layernorm_fw(x, g, b, EPS)
    mean32 = mean.astype(np.float32).astype(np.float64)
    rstd32 = rstd.astype(np.float32).astype(np.float64)
    dx_t, dg_t, db_t = torch.ops.aten.native_layer_norm_backward(
        torch.from_numpy(dy), torch.from_numpy(x), [C], torch.from_numpy(mean32).view(N, 1),
        torch.from_numpy(rstd32).view(N, 1), torch.from_numpy(g), torch.from_numpy(b),
        [True, True, True])
    dx, dg, db = oracle.layernorm_bw_given_stats(x, dy, g, mean32, rstd32)
    np.testing.assert_allclose(dx, dx_t.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dg, dg_t.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, db_t.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RMSNorm

RMS_EPS = 1e-6


def test_rmsnorm_forward_matches_torch_rms_norm_and_closed_form():
    x, g, _, _ = _case(13, 31, 11, offset_std=1.0)
    ref = F.rms_norm(torch.from_numpy(x), (31,), torch.from_numpy(g), eps=RMS_EPS).numpy()
    y, rr = oracle.rmsnorm_fw(x, g, RMS_EPS)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    c = 0.7
    yc, _ = oracle.rmsnorm_fw(np.full((2, 5), c), np.ones(5), RMS_EPS)
    np.testing.assert_allclose(yc, c / np.sqrt(c * c + RMS_EPS), rtol=1e-15)


def test_rmsnorm_backward_matches_autograd_and_finite_differences():
    x, g, _, dy = _case(5, 9, 12, offset_std=1.0)
    xt = torch.from_numpy(x).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    F.rms_norm(xt, (9,), gt, eps=RMS_EPS).backward(torch.from_numpy(dy))
    dx, dg = oracle.rmsnorm_bw(x, dy, g, RMS_EPS)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    h = 1e-6
    i, j = 2, 4
    xp = x.copy(); xp[i, j] += h
    xm = x.copy(); xm[i, j] -= h
    fd = (np.sum(dy * oracle.rmsnorm_fw(xp, g, RMS_EPS)[0]) -
          np.sum(dy * oracle.rmsnorm_fw(xm, g, RMS_EPS)[0])) / (2 * h)
    assert abs(fd - dx[i, j]) <= 1e-7


def test_rmsnorm_backward_given_rstd_pins():
    """Backward from a saved rstd (what the GPU kernel receives):
    (1) with the exact fp64 rstd it equals the recomputing backward (itself pinned to autograd
        and finite differences above);
    (2) with an fp32-rounded rstd (not the exact statistic) it equals aten's LayerNorm
        backward taking mean = 0 and that rstd as inputs, plus rstd_i * mean_j(gamma_j dy_ij):
        RMSNorm's gradient is LayerNorm's with the mean removed and without the sum_k g_ik
        term that the mean's derivative contributes;
    (3) C = 1 closed form: xhat = x*r and dx = r*g*(1 - xhat^2)."""
    N, C = 41, 37
    x, g, _, dy = _case(N, C, 15, offset_std=1.0)
    _, rr = oracle.rmsnorm_fw(x, g, RMS_EPS)
    dx_e, dg_e = oracle.rmsnorm_bw_given_rstd(x, dy, g, rr)
    dx_r, dg_r = oracle.rmsnorm_bw(x, dy, g, RMS_EPS)
    np.testing.assert_allclose(dx_e, dx_r, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg_e, dg_r, rtol=1e-12, atol=1e-13)

    r32 = rr.astype(np.float32).astype(np.float64)
    dx_t, dg_t, _ = torch.ops.aten.native_layer_norm_backward(
        torch.from_numpy(dy), torch.from_numpy(x), [C], torch.zeros(N, 1, dtype=torch.float64),
        torch.from_numpy(r32).view(N, 1), torch.from_numpy(g), torch.zeros(C, dtype=torch.float64),
        [True, True, False])
    dx, dg = oracle.rmsnorm_bw_given_rstd(x, dy, g, r32)
    gdy = g.reshape(1, C) * dy
    np.testing.assert_allclose(dx, dx_t.numpy() + r32.reshape(N, 1) * gdy.mean(axis=1, keepdims=True),
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dg, dg_t.numpy(), rtol=1e-11, atol=1e-11)

    x1 = np.array([[0.3], [-2.0], [1e-4]])
    dy1 = np.array([[1.5], [-0.25], [2.0]])
    g1 = np.array([0.8])
    r1 = np.array([1.7, 0.4, 3.0])
    dx1, dg1 = oracle.rmsnorm_bw_given_rstd(x1, dy1, g1, r1)
    xh = x1[:, 0] * r1
    np.testing.assert_allclose(dx1[:, 0], r1 * g1[0] * dy1[:, 0] * (1 - xh * xh), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dg1, [np.sum(dy1[:, 0] * xh)], rtol=1e-14)


def test_results_do_not_depend_on_the_thread_count():
    """The CPU baseline times the oracle at several thread counts; every output element is
    computed by one thread in a fixed order, so the values must be bitwise identical."""
    x, g, b, dy = _case(300, 96, 14, offset_std=1.0)
    n0 = oracle.threads()
    try:
        ref = [*oracle.layernorm_fw(x, g, b), *oracle.layernorm_bw(x, dy, g)]
        oracle.set_threads(1)
        assert oracle.threads() == 1
        one = [*oracle.layernorm_fw(x, g, b), *oracle.layernorm_bw(x, dy, g)]
    finally:
        oracle.set_threads(n0)
    for u, v in zip(ref, one):
        assert np.array_equal(u, v)
