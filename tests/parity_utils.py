"""Helpers shared by the GPU parity tests: tolerances, element-wise comparison, case logging.

Tolerances (|gpu - oracle| <= atol + rtol * |oracle|, element by element, the allclose
convention of the HW4 page's kernel tests):
  * fp16 storage: atol = rtol = 1e-3 (the HW4 page, "Faster than what?").
  * fp32 storage: atol = rtol = 1e-5.
Column sums over N rows of products formed in fp32 (dgamma = sum_i dy * xhat) carry the fp32
rounding of every term, random over rows: about 2^-24 * sqrt(sum_i (dy * xhat)^2) per column,
which reaches 1e-5 on near-zero columns from a few thousand rows up. Their bound adds six
times that (colsum_slack; see assert_close's `slack`).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {torch.float16: (1e-3, 1e-3), torch.float32: (1e-5, 1e-5)}


def say(*msg):
    """Name the case before each GPU step, flushed, so a failing run says where it was."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def violations(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float, chunk: int = 1 << 24):
    """Count elements outside the bound and return (count, worst index, worst excess)."""
    g = got.reshape(-1)
    r = ref.reshape(-1)
    bad = 0
    worst = (-1, 0.0)
    for s in range(0, g.size, chunk):
        gs = g[s:s + chunk]
        rs = r[s:s + chunk]
        with np.errstate(invalid="ignore"):
            err = np.abs(gs - rs)
            lim = atol + rtol * np.abs(rs)
            over = ~(err <= lim)          # NaN counts as a violation
        n = int(over.sum())
        if n:
            bad += n
            ex = np.where(over, np.nan_to_num(err - lim, nan=np.inf), -np.inf)
            i = int(np.argmax(ex))
            if ex[i] > worst[1] or worst[0] < 0:
                worst = (s + i, float(ex[i]))
    return bad, worst


def colsum_slack(dy64: np.ndarray, xhat64: np.ndarray, rows: int = 4096) -> np.ndarray:
    """Per-column allowance for the fp32 rounding of the N terms of sum_i dy_ij * xhat_ij: xhat
    (two fp32 operations) and the product (one) each round with relative error below 2^-24,
    independently over rows, so the sum's error has a standard deviation of about
    2^-24 * sqrt(sum_i (dy * xhat)^2); the allowance is six of those."""
    sq = np.zeros(dy64.shape[1])
    for s in range(0, dy64.shape[0], rows):
        sq += np.sum((dy64[s:s + rows] * xhat64[s:s + rows]) ** 2, axis=0)
    return 6.0 * 2.0 ** -24 * np.sqrt(sq)


def assert_close(got, ref, dtype, what: str, atol=None, rtol=None, slack=None):
    """Element-wise |got - ref| <= atol + rtol * |ref| (+ slack, a per-element array)."""
    a0, r0 = TOL[dtype]
    atol = a0 if atol is None else atol
    rtol = r0 if rtol is None else rtol
    got = to_host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if slack is not None:
        atol = atol + np.asarray(slack, np.float64).reshape(-1)
        assert atol.size == got.size, (what, atol.size, got.size)
        got, ref = got.reshape(-1), ref.reshape(-1)
        bad = ~(np.abs(got - ref) <= atol + rtol * np.abs(ref))
        if bad.any():
            idx = int(np.argmax(np.where(bad, np.abs(got - ref) - atol - rtol * np.abs(ref), -np.inf)))
            raise AssertionError(
                f"{what}: {int(bad.sum())} of {got.size} elements outside atol={TOL[dtype][0]} + "
                f"fp32 column-sum slack, rtol={rtol}; worst at index {idx}: gpu={got[idx]!r} "
                f"oracle={ref[idx]!r} |diff|={abs(got[idx] - ref[idx]):.3e} slack="
                f"{float(atol[idx]) - TOL[dtype][0]:.3e}")
        return
    bad, (idx, ex) = violations(got, ref, atol, rtol)
    if bad:
        gi = got.reshape(-1)[idx]
        ri = ref.reshape(-1)[idx]
        raise AssertionError(
            f"{what}: {bad} of {got.size} elements outside atol={atol} rtol={rtol}; worst at flat "
            f"index {idx}: gpu={gi!r} oracle={ri!r} |diff|={abs(gi - ri):.3e}")


def max_abs_err(got, ref) -> float:
    got = to_host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    return float(np.max(np.abs(got - np.asarray(ref, np.float64)))) if got.size else 0.0
