"""Pins of the oracle's bias + dropout + residual feeding LayerNorm (CPU only).

The L10 page lists "bias + dropout + residual" among the elementwise kernels, followed by
the LayerNorm reduce kernel; it gives no RNG or dropout rule, so the keep-mask is an input
bit mask (bit j % 8 of byte j / 8, least significant first) and kept elements are scaled by
1 / (1 - p). Pinned against torch's layer_norm and autograd through the composition,
numpy's packbits for the bit order, and the p = 0 reduction to plain LayerNorm.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle

EPS = 1e-8


def _case(N, C, seed, p):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, C))
    r = rng.standard_normal((N, C)) * 2.0 + 1.0
    b = rng.standard_normal(C) * 0.5
    g = rng.uniform(0.5, 1.5, C)
    be = rng.normal(0.0, 0.3, C)
    keep = rng.random((N, C)) >= p
    bits = np.packbits(keep, axis=1, bitorder="little")
    dy = rng.standard_normal((N, C))
    de = rng.standard_normal((N, C))
    return x, r, b, g, be, keep, bits, dy, de


def test_p_zero_all_kept_is_layernorm_of_the_sum():
    x, r, b, g, be, _, _, _, _ = _case(9, 37, 1, 0.0)
    bits = np.packbits(np.ones((9, 37), bool), axis=1, bitorder="little")
    s, y, mean, rstd = oracle.bdr_ln_fw(x, r, b, bits, 0.0, g, be, EPS)
    np.testing.assert_array_equal(s, r + (x + b))
    ref = F.layer_norm(torch.from_numpy(s), (37,), torch.from_numpy(g), torch.from_numpy(be), EPS)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, s.mean(axis=1), rtol=1e-14)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(s.var(axis=1) + EPS), rtol=1e-13)


def test_mask_bit_order_and_scaling():
    N, C, p = 4, 21, 0.25
    x, r, b, g, be, keep, bits, _, _ = _case(N, C, 2, p)
    s, _, _, _ = oracle.bdr_ln_fw(x, r, b, bits, p, g, be, EPS)
    added = s - r                          # (r + a) - r: one rounding of r's size
    np.testing.assert_allclose(added[keep], ((x + b) / (1 - p))[keep], rtol=1e-12, atol=1e-14)
    assert np.all(added[~keep] == 0.0)
    one = np.zeros((N, C), bool)
    one[2, 13] = True                      # a single kept element: byte 1, bit 5 of row 2
    s1, _, _, _ = oracle.bdr_ln_fw(x, r, b, np.packbits(one, axis=1, bitorder="little"), p, g, be, EPS)
    d = s1 - r
    assert np.count_nonzero(d) == 1
    np.testing.assert_allclose(d[2, 13], (x[2, 13] + b[13]) / (1 - p), rtol=1e-12, atol=1e-14)


def test_backward_matches_autograd_through_the_composition():
    N, C, p = 11, 29, 0.3
    x, r, b, g, be, keep, bits, dy, de = _case(N, C, 3, p)
    s, y, mean, rstd = oracle.bdr_ln_fw(x, r, b, bits, p, g, be, EPS)
    tx, tr, tb = (torch.from_numpy(v).requires_grad_(True) for v in (x, r, b))
    tg, tbe = torch.from_numpy(g).requires_grad_(True), torch.from_numpy(be).requires_grad_(True)
    km = torch.from_numpy(keep.astype(np.float64))
    ts = tr + km * (tx + tb) / (1 - p)
    ty = F.layer_norm(ts, (C,), tg, tbe, EPS)
    ((ty * torch.from_numpy(dy)).sum() + (ts * torch.from_numpy(de)).sum()).backward()
    dres, dx, dg, db, dbias = oracle.bdr_ln_bw(s, dy, de, bits, p, g, mean, rstd)
    np.testing.assert_allclose(dres, tr.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dbias, tb.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(db, tbe.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_identities_and_no_extra_gradient():
    N, C, p = 6, 16, 0.5
    x, r, b, g, be, keep, bits, dy, _ = _case(N, C, 4, p)
    s, _, mean, rstd = oracle.bdr_ln_fw(x, r, b, bits, p, g, be, EPS)
    dres, dx, _, _, dbias = oracle.bdr_ln_bw(s, dy, None, bits, p, g, mean, rstd)
    np.testing.assert_allclose(dx, np.where(keep, dres / (1 - p), 0.0), rtol=1e-15)
    np.testing.assert_allclose(dbias, dx.sum(axis=0), rtol=1e-13, atol=1e-14)
    # without the extra gradient, dresidual is the LayerNorm input gradient: rows sum to 0
    np.testing.assert_allclose(dres.sum(axis=1), 0.0, atol=1e-12)
