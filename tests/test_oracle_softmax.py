"""Pins for the oracle's attention softmax (forward and backward), CPU only.

The oracle is checked against things other than itself: invariants that the definition on
the HW4 page fixes ("CMU 11-868 HW4 ...", "Problem structure and scoring": the attention mask
is added, future tokens are set to -inf, then a max and a sum of exponentials), closed forms,
an independent fp64 library routine (torch.softmax / autograd on the CPU), and central
finite differences for the backward formula, which the pages never print.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from layernorm_reduction_amd import workloads as W


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_softmax_ref(x, mask, causal):
    """softmax(inp + mask) in fp64 with a triu(-inf) future mask: the HW4 baseline's form."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    B, H, Tq, Tk = xt.shape
    z = xt.clone()
    if mask is not None:
        z = z + torch.from_numpy(np.asarray(mask, np.float64)).view(B, 1, 1, Tk)
    if causal:
        fut = torch.triu(torch.ones(Tq, Tk, dtype=torch.bool), diagonal=1)
        z = z.masked_fill(fut, float("-inf"))
    return torch.softmax(z, dim=-1).numpy()


def _mask_from_lengths(lengths, Tk):
    m = np.zeros((len(lengths), Tk))
    for b, L in enumerate(lengths):
        m[b, L:] = -np.inf
    return m


# ---------------------------------------------------------------- forward: invariants

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_masked_positions_are_exact_zeros(causal):
    B, H, T = 3, 2, 12
    x = _rand((B, H, T, T), 1)
    lengths = [12, 7, 1]
    mask = _mask_from_lengths(lengths, T)
    y = oracle.softmax_fw(x, mask, causal)
    assert np.all(np.abs(y.sum(-1) - 1.0) <= 1e-13)
    for b, L in enumerate(lengths):
        assert np.all(y[b, :, :, L:] == 0.0)          # padded keys: exact zeros
    if causal:
        fut = np.triu(np.ones((T, T), bool), 1)
        assert np.all(y[:, :, fut] == 0.0)             # future keys: exact zeros
    assert np.all(y >= 0.0)


@pytest.mark.parametrize("c", [-30.0, 7.0, 1e3])
def test_shift_invariance(c):
    x = _rand((2, 3, 9, 9), 2)
    mask = _mask_from_lengths([9, 5], 9)
    y0 = oracle.softmax_fw(x, mask, True)
    y1 = oracle.softmax_fw(x + c, mask, True)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-15)


def test_fully_masked_row_is_zero():
    x = _rand((1, 1, 3, 4), 3)
    mask = np.full((1, 4), -np.inf)
    y = oracle.softmax_fw(x, mask, False)
    assert np.all(y == 0.0)


def test_large_magnitude_scores_do_not_overflow():
    x = _rand((2, 2, 8, 8), 4) * 1e4
    y = oracle.softmax_fw(x, None, True)
    assert np.all(np.isfinite(y))
    np.testing.assert_allclose(y.sum(-1), 1.0, atol=1e-13)
    np.testing.assert_allclose(y, _torch_softmax_ref(x, None, True), rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- forward: closed forms

def test_closed_form_logs_of_integers():
    # softmax([0, ln 2, ln 3, ln 4]) = [1, 2, 3, 4] / 10
    x = np.log(np.array([1.0, 2.0, 3.0, 4.0])).reshape(1, 1, 1, 4)
    y = oracle.softmax_fw(x, None, False)
    np.testing.assert_allclose(y.reshape(4), [0.1, 0.2, 0.3, 0.4], rtol=1e-15, atol=1e-16)


def test_closed_form_one_and_two_valid_keys():
    x = _rand((2, 1, 1, 6), 5)
    mask = _mask_from_lengths([1, 2], 6)
    y = oracle.softmax_fw(x, mask, False)
    assert y[0, 0, 0, 0] == 1.0 and np.all(y[0, 0, 0, 1:] == 0.0)
    d = x[1, 0, 0, 1] - x[1, 0, 0, 0]
    np.testing.assert_allclose(y[1, 0, 0, 0], 1.0 / (1.0 + math.exp(d)), rtol=1e-15)
    np.testing.assert_allclose(y[1, 0, 0, 1], 1.0 / (1.0 + math.exp(-d)), rtol=1e-15)


def test_closed_form_equal_scores_and_causal_first_row():
    T = 7
    x = np.full((1, 1, T, T), 0.3)
    y = oracle.softmax_fw(x, None, True)
    for i in range(T):
        np.testing.assert_allclose(y[0, 0, i, : i + 1], 1.0 / (i + 1), rtol=1e-15)
    assert y[0, 0, 0, 0] == 1.0


def test_additive_mask_with_finite_values():
    # A finite additive mask m shifts scores: softmax(x + m) with m = log(w) weights keys by w.
    x = np.zeros((1, 1, 1, 3))
    w = np.array([1.0, 2.0, 5.0])
    y = oracle.softmax_fw(x, np.log(w).reshape(1, 3), False)
    np.testing.assert_allclose(y.reshape(3), w / w.sum(), rtol=1e-15)


# ---------------------------------------------------------------- forward: library routine

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_fp64_softmax_of_inp_plus_mask(causal):
    B, H, T = 3, 2, 17
    x = _rand((B, H, T, T), 6)
    mask = _mask_from_lengths([17, 9, 4], T)
    np.testing.assert_allclose(oracle.softmax_fw(x, mask, causal), _torch_softmax_ref(x, mask, causal),
                               rtol=1e-13, atol=1e-15)


def test_mask_is_indexed_by_batch_and_broadcast_over_heads_and_queries():
    # Non-square, non-causal: a swapped index (b vs h, Tq vs Tk) changes the result.
    B, H, Tq, Tk = 3, 2, 5, 7
    x = _rand((B, H, Tq, Tk), 7)
    mask = _rand((B, Tk), 8)
    np.testing.assert_allclose(oracle.softmax_fw(x, mask, False), _torch_softmax_ref(x, mask, False),
                               rtol=1e-13, atol=1e-15)


def test_workload1_matches_torch():
    [s], _ = W.workload1()
    x = s.x.double().numpy()
    m = s.mask.double().numpy()
    np.testing.assert_allclose(oracle.softmax_fw(x, m, True), _torch_softmax_ref(x, m, True),
                               rtol=1e-13, atol=1e-15)


def test_selected_rows_agree_with_whole_tensor():
    B, H, T = 2, 3, 11
    x = _rand((B, H, T, T), 9)
    mask = _mask_from_lengths([11, 6], T)
    y = oracle.softmax_fw(x, mask, True).reshape(-1, T)
    rows = np.array([0, 5, 12, 33, 65])
    b = rows // (H * T)
    q = rows % T
    yr = oracle.softmax_fw_rows(x.reshape(-1, T)[rows], mask[b], q, True)
    np.testing.assert_array_equal(yr, y[rows])


# ---------------------------------------------------------------- backward

def _loss(x, dy, mask, causal):
    return float(np.sum(dy * oracle.softmax_fw(x, mask, causal)))


@pytest.mark.parametrize("shape,causal,lengths", [((1, 1, 4, 4), True, None),
                                                  ((2, 2, 16, 16), True, [16, 9]),
                                                  ((2, 1, 3, 5), False, [5, 2])])
def test_backward_matches_central_finite_differences(shape, causal, lengths):
    rng = np.random.default_rng(10)
    x = rng.standard_normal(shape)
    dy = rng.standard_normal(shape)
    mask = None if lengths is None else _mask_from_lengths(lengths, shape[-1])
    y = oracle.softmax_fw(x, mask, causal)
    dx = oracle.softmax_bw(y, dy)
    h = 1e-6
    fd = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy()
        xp[idx] += h
        xm = x.copy()
        xm[idx] -= h
        fd[idx] = (_loss(xp, dy, mask, causal) - _loss(xm, dy, mask, causal)) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=0, atol=1e-7)


def test_backward_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 2, 9, 9))
    mask = _mask_from_lengths([9, 4], 9)
    y = oracle.softmax_fw(x, mask, True)
    dy = rng.standard_normal(x.shape)
    dx = oracle.softmax_bw(y, dy)
    np.testing.assert_allclose(dx.sum(-1), 0.0, atol=1e-14)     # rows of dx sum to 0
    assert np.all(dx[y == 0.0] == 0.0)                          # masked positions: exact 0
    dxc = oracle.softmax_bw(y, np.full_like(y, 2.5))            # constant dy: no gradient
    assert np.max(np.abs(dxc)) <= 1e-14


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(12)
    B, H, T = 2, 3, 10
    x = rng.standard_normal((B, H, T, T))
    dy = rng.standard_normal(x.shape)
    mask = _mask_from_lengths([10, 3], T)
    xt = torch.from_numpy(x).requires_grad_(True)
    z = xt + torch.from_numpy(mask).view(B, 1, 1, T)
    z = z.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    torch.softmax(z, -1).backward(torch.from_numpy(dy))
    y = oracle.softmax_fw(x, mask, True)
    np.testing.assert_allclose(oracle.softmax_bw(y, dy), xt.grad.numpy(), rtol=1e-12, atol=1e-14)
