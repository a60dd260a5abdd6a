"""Pins of the oracle's softmax cross-entropy over a vocabulary (CPU only).

The pages name the kernel (L10 "Technique 1": cross entropy is one of the custom reduce
kernels) but print no formula, so the oracle is the textbook definition: lse - z_target per
row, gradient dloss * (softmax - onehot). Pinned here against independent fp64 library
routines (torch's cross_entropy, logsumexp and autograd), closed forms and finite
differences, so that a dropped max shift, a wrong target index, a missing one-hot term or a
sign error fails a test.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

IGN = -100


def _case(N, V, seed, scale=3.0, ignore_rows=()):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((N, V)) * scale
    t = rng.integers(0, V, N)
    for r in ignore_rows:
        t[r] = IGN
    dloss = rng.standard_normal(N)
    return z, t, dloss


def test_forward_matches_torch_cross_entropy_and_logsumexp():
    z, t, _ = _case(37, 101, 1, ignore_rows=(3, 20))
    loss, lse = oracle.xent_fw(z, t, IGN)
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(t), reduction="none",
                          ignore_index=IGN).numpy()
    np.testing.assert_allclose(loss, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(z), dim=1).numpy(),
                               rtol=1e-14, atol=1e-14)
    assert loss[3] == 0.0 and loss[20] == 0.0


def test_closed_forms():
    V = 64
    loss, lse = oracle.xent_fw(np.full((3, V), 2.5), [0, 17, 63])
    np.testing.assert_allclose(loss, math.log(V), rtol=1e-15)            # uniform logits
    np.testing.assert_allclose(lse, 2.5 + math.log(V), rtol=1e-15)
    loss1, lse1 = oracle.xent_fw(np.array([[7.0], [-3.0]]), [0, 0])      # one class
    assert np.all(loss1 == 0.0) and np.allclose(lse1, [7.0, -3.0])
    a, b = 1.3, -0.4                                                     # two classes: softplus
    loss2, _ = oracle.xent_fw(np.array([[a, b]]), [0])
    np.testing.assert_allclose(loss2, [math.log1p(math.exp(b - a))], rtol=1e-14)


def test_large_logits_are_stable():
    z = np.array([[1e4, -1e4, 0.0, 1e4 - 1.0], [-1e4, -1e4 + 2.0, -1e4 + 1.0, -1e4]])
    t = np.array([3, 0])
    loss, lse = oracle.xent_fw(z, t)
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(t), reduction="none").numpy()
    assert np.all(np.isfinite(loss))
    np.testing.assert_allclose(loss, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(loss[0], math.log1p(math.exp(1.0)) + math.log1p(0.0), rtol=1e-12)


def test_out_of_range_target_is_nan_and_ignored_row_is_zero():
    z, _, dloss = _case(3, 10, 2)
    loss, lse = oracle.xent_fw(z, [10, IGN, -1], IGN)
    assert math.isnan(loss[0]) and loss[1] == 0.0 and math.isnan(loss[2])
    dz = oracle.xent_bw_given_lse(z, [10, IGN, -1], lse, dloss, IGN)
    assert np.all(np.isnan(dz[0])) and np.all(dz[1] == 0.0) and np.all(np.isnan(dz[2]))


def test_backward_matches_autograd():
    z, t, dloss = _case(29, 77, 3, ignore_rows=(5,))
    zt = torch.from_numpy(z).requires_grad_(True)
    l = F.cross_entropy(zt, torch.from_numpy(t), reduction="none", ignore_index=IGN)
    (l * torch.from_numpy(dloss)).sum().backward()
    dz = oracle.xent_bw(z, t, dloss, IGN)
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-12, atol=1e-14)
    assert np.all(dz[5] == 0.0)


def test_backward_finite_differences_and_row_sums():
    z, t, dloss = _case(4, 13, 4)
    dz = oracle.xent_bw(z, t, dloss)
    # each row of softmax - onehot sums to zero
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-14)
    h = 1e-6
    for (i, j) in [(0, int(t[0])), (1, 3), (3, 12)]:
        zp = z.copy(); zp[i, j] += h
        zm = z.copy(); zm[i, j] -= h
        fp = np.dot(dloss, oracle.xent_fw(zp, t)[0])
        fm = np.dot(dloss, oracle.xent_fw(zm, t)[0])
        assert abs((fp - fm) / (2 * h) - dz[i, j]) < 1e-7


def test_given_lse_is_the_recomputing_backward_and_is_linear_in_lse_error():
    z, t, dloss = _case(11, 50, 5)
    _, lse = oracle.xent_fw(z, t)
    np.testing.assert_allclose(oracle.xent_bw_given_lse(z, t, lse, dloss), oracle.xent_bw(z, t, dloss),
                               rtol=0, atol=0)
    # a shifted lse scales the softmax part by exp(-delta): check one element exactly
    d = 0.25
    dz = oracle.xent_bw_given_lse(z, t, lse + d, dloss)
    i, j = 2, (int(t[2]) + 1) % 50
    np.testing.assert_allclose(dz[i, j], dloss[i] * math.exp(z[i, j] - lse[i] - d), rtol=1e-14)
