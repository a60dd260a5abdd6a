"""Helpers shared by the GPU parity tests: tolerances, element-wise comparison, case logging.

Tolerances (|gpu - oracle| <= atol + rtol * |oracle|, element by element, the allclose
convention of the HW4 page's kernel tests):
  * fp16 storage: atol = rtol = 1e-3 (the HW4 page, "Faster than what?").
  * fp32 storage: atol = rtol = 1e-5.
Every comparison prints the largest ratio of error to bound it saw, so the margin is on record.

Input gradients of the normalisations (assert_grad_close): dx = rstd * (g - mean(g) - xhat *
mean(g * xhat)) is formed in fp32 from terms as large as rstd * |g|, so its rounding error is a
few units of fp32 roundoff times rstd * max_j |g_ij| for its row. Below rstd = 8 (a row
variance above 1/64) that is under 1e-5 for the workloads' gradients and the plain bound holds.
Only near-constant rows (a C = 2 row with nearly equal entries, a zero row) have an exact dx
that is a tiny remainder of much larger terms; the edge-case tests, and only they, let those
rows add the rounding term 16 * 2^-24 * rstd_i * max_j |g_ij| to the bound, and print how many
elements needed it.
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


def worst_ratio(got: np.ndarray, ref: np.ndarray, atol: float, rtol: float, chunk: int = 1 << 24) -> float:
    """Largest |got - ref| / (atol + rtol * |ref|) over all elements (inf if any is NaN)."""
    g = got.reshape(-1)
    r = ref.reshape(-1)
    w = 0.0
    for s in range(0, g.size, chunk):
        with np.errstate(invalid="ignore"):
            q = np.abs(g[s:s + chunk] - r[s:s + chunk]) / (atol + rtol * np.abs(r[s:s + chunk]))
        if q.size:
            m = float(np.max(q)) if not np.isnan(q).any() else float("inf")
            w = max(w, m)
    return w


def assert_close(got, ref, dtype, what: str, atol=None, rtol=None):
    """Element-wise |got - ref| <= atol + rtol * |ref|; prints the worst error-to-bound ratio."""
    a0, r0 = TOL[dtype]
    atol = a0 if atol is None else atol
    rtol = r0 if rtol is None else rtol
    got = to_host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    print(f"[parity] {what}: worst err/bound {worst_ratio(got, ref, atol, rtol):.3f} "
          f"(atol={atol:g} rtol={rtol:g})", flush=True)
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


U32 = 2.0 ** -24
NEAR_CONSTANT_RSTD = 8.0


def assert_grad_close(got_t, ref, dtype, what: str, rstd, gmax, allow_near_constant: bool = False,
                      factor: float = 1.0):
    """Element-wise plain bound atol + rtol * |ref| on a normalisation's input gradient.

    rstd [N] and gmax [N] (max_j of the magnitudes the row's fp32 formula subtracts) give the
    rounding term 16 * 2^-24 * rstd_i * gmax_i (times `factor` for a gradient scaled after it is
    formed). That term is added only where allow_near_constant is set and only on rows with
    rstd_i >= NEAR_CONSTANT_RSTD; the number of elements that needed it is printed."""
    atol, rtol = TOL[dtype]
    got = to_host64(got_t) if isinstance(got_t, torch.Tensor) else np.asarray(got_t, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    r = np.asarray(rstd, np.float64).reshape(-1, 1)
    err = np.abs(got - ref)
    lim0 = atol + rtol * np.abs(ref)
    plain_bad = ~(err <= lim0)
    ratio = float(np.max(err / lim0)) if err.size else 0.0
    n_allow = 0
    if allow_near_constant:
        term = factor * 16.0 * U32 * r * np.asarray(gmax, np.float64).reshape(-1, 1)
        term = np.where(r >= NEAR_CONSTANT_RSTD, term, 0.0)
        lim = lim0 + term
        bad = ~(err <= lim)
        n_allow = int(np.sum(plain_bad & ~bad))
    else:
        lim = lim0
        bad = plain_bad
    print(f"[parity] {what}: worst err/plain bound {ratio:.3f}; {n_allow} of {err.size} elements "
          f"(near-constant rows) needed the rounding term", flush=True)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - lim, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements outside the bound; "
                             f"worst at {i}: gpu={got[i]!r} oracle={ref[i]!r} bound={lim[i]:.3e} "
                             f"rstd={float(r[i[0], 0]):.3e}")
