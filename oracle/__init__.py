"""fp64 CPU oracle for the fused softmax / LayerNorm row reductions.

TEST INFRASTRUCTURE ONLY. The product package (``layernorm_reduction_amd``) never imports
this module. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it. It shares no code with the HIP path.

The arithmetic lives in ``lnr_oracle.c`` (plain loops, double precision, two-pass
statistics). This wrapper only converts numpy arrays: every input is widened to float64,
which is exact for values stored as fp16 or fp32, and every output is float64, never
rounded to a storage type.

Citations (page titles and sections; see ``lnr_oracle.c`` for the formulas):
  * softmax forward: "CMU 11-868 HW4: Softmax and LayerNorm as fused CUDA kernels",
    "Problem structure and scoring" (attention mask added, future tokens set to -inf,
    a max then a sum of exponentials) and "Faster than what?" (softmax(inp + mask));
    "CMU 11-868 L10 ...", "Technique 2" (two reductions).
  * softmax backward: named in the HW4 page's table; formula = textbook softmax Jacobian.
  * LayerNorm forward/backward: L10 "Technique 2" (mu(x), mu(x^2); the two backward sums),
    HW4 "Problem structure and scoring" (eps = 1e-8 inside the root; dgamma/dbeta summed
    across rows).
  * RMSNorm: "FastTransformer: Breaking the Compiler Ceiling ...", section 5.4 (forward,
    backward recomputing rstd from x, and backward from a given rstd).
  * Bias + dropout + residual feeding LayerNorm: L10 "Technique 1" (the elementwise kernel
    "bias + dropout + residual", then the LayerNorm reduce kernel); the dropout keep-mask is
    an input bit mask.
  * Softmax cross-entropy over a vocabulary: L10 "Technique 1" names the reduce kernel and
    the inference section the whole-vocabulary softmax; no formula is printed, so this is
    the textbook definition (lse - z_target; gradient softmax - onehot), no label smoothing.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed forms,
invariants, finite differences and independent fp64 library routines.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblnr_oracle.so")
SRC_PATH = os.path.join(_HERE, "lnr_oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile lnr_oracle.c with gcc (IEEE double, no FMA contraction, OpenMP)."""
    import subprocess

    cmd = [
        "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
        SRC_PATH, "-o", LIB_PATH + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    d = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.lnr_oracle_softmax_fw.argtypes = [d, d, i64, i64, i64, i64, ctypes.c_int, d]
    lib.lnr_oracle_softmax_fw_rows.argtypes = [d, d, ctypes.POINTER(i64), i64, i64, ctypes.c_int, d]
    lib.lnr_oracle_softmax_bw.argtypes = [d, d, i64, i64, d]
    lib.lnr_oracle_layernorm_fw.argtypes = [d, d, d, i64, i64, ctypes.c_double, d, d, d]
    lib.lnr_oracle_layernorm_bw_dx.argtypes = [d, d, d, i64, i64, ctypes.c_double, d]
    lib.lnr_oracle_layernorm_bw_dgamma_dbeta.argtypes = [d, d, i64, i64, ctypes.c_double, d, d, d, d]
    lib.lnr_oracle_rmsnorm_fw.argtypes = [d, d, i64, i64, ctypes.c_double, d, d]
    lib.lnr_oracle_rmsnorm_bw.argtypes = [d, d, d, i64, i64, ctypes.c_double, d, d]
    lib.lnr_oracle_rmsnorm_bw_given_rstd.argtypes = [d, d, d, d, i64, i64, d, d]
    lib.lnr_oracle_layernorm_bw_given_stats.argtypes = [d, d, d, d, d, i64, i64, d, d, d]
    lib.lnr_oracle_layernorm_bw_given_stats.restype = None
    pi64 = ctypes.POINTER(ctypes.c_int64)
    lib.lnr_oracle_xent_fw.argtypes = [d, pi64, i64, i64, i64, d, d]
    lib.lnr_oracle_xent_fw.restype = None
    lib.lnr_oracle_xent_bw_given_lse.argtypes = [d, pi64, d, d, i64, i64, i64, d]
    lib.lnr_oracle_xent_bw_given_lse.restype = None
    pu8 = ctypes.POINTER(ctypes.c_uint8)
    lib.lnr_oracle_bdr_ln_fw.argtypes = [d, d, d, pu8, ctypes.c_double, d, d, i64, i64,
                                         ctypes.c_double, d, d, d, d]
    lib.lnr_oracle_bdr_ln_fw.restype = None
    lib.lnr_oracle_bdr_ln_bw.argtypes = [d, d, d, pu8, ctypes.c_double, d, d, d, i64, i64,
                                         d, d, d, d, d]
    lib.lnr_oracle_bdr_ln_bw.restype = None
    lib.lnr_oracle_threads.argtypes = []
    lib.lnr_oracle_threads.restype = ctypes.c_int
    lib.lnr_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.lnr_oracle_set_threads.restype = None
    for f in (lib.lnr_oracle_softmax_fw, lib.lnr_oracle_softmax_fw_rows, lib.lnr_oracle_softmax_bw,
              lib.lnr_oracle_layernorm_fw, lib.lnr_oracle_layernorm_bw_dx,
              lib.lnr_oracle_layernorm_bw_dgamma_dbeta, lib.lnr_oracle_rmsnorm_fw,
              lib.lnr_oracle_rmsnorm_bw, lib.lnr_oracle_rmsnorm_bw_given_rstd):
        f.restype = None
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().lnr_oracle_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads from now on (timing only: each output element is computed by one
    thread in a fixed order, so results do not depend on n)."""
    _load().lnr_oracle_set_threads(int(n))


def _f64(a) -> np.ndarray:
    """Widen to a C-contiguous float64 array (exact for fp16 / fp32 stored values)."""
    if hasattr(a, "detach"):  # a CPU torch tensor
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray | None):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def softmax_fw(x, mask=None, causal: bool = False) -> np.ndarray:
    """x: [B, H, Tq, Tk]; mask: additive [B, Tk] or None. Returns y as float64."""
    x = _f64(x)
    B, H, Tq, Tk = x.shape
    if causal and Tq != Tk:
        raise ValueError("causal softmax needs Tq == Tk")
    m = None if mask is None else _f64(mask).reshape(B, Tk)
    y = np.empty_like(x)
    _load().lnr_oracle_softmax_fw(_p(x), _p(m), B, H, Tq, Tk, int(bool(causal)), _p(y))
    return y


def softmax_fw_rows(x_rows, mask_rows, qidx, causal: bool = False) -> np.ndarray:
    """Selected rows: x_rows [n, Tk]; mask_rows [n, Tk] or None; qidx [n] query positions."""
    x = _f64(x_rows)
    n, Tk = x.shape
    m = None if mask_rows is None else _f64(mask_rows).reshape(n, Tk)
    q = np.ascontiguousarray(np.asarray(qidx, dtype=np.int64).reshape(n))
    y = np.empty_like(x)
    _load().lnr_oracle_softmax_fw_rows(
        _p(x), _p(m), q.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, Tk,
        int(bool(causal)), _p(y))
    return y


def softmax_bw(y, dy) -> np.ndarray:
    """y, dy: [..., Tk] (y = forward output). Returns dx as float64 with the same shape."""
    y = _f64(y)
    dy = _f64(dy)
    if y.shape != dy.shape:
        raise ValueError("y and dy shapes differ")
    Tk = y.shape[-1]
    rows = y.size // Tk if Tk else 0
    dx = np.empty_like(y)
    _load().lnr_oracle_softmax_bw(_p(y), _p(dy), rows, Tk, _p(dx))
    return dx


def layernorm_fw(x, gamma, beta, eps: float = 1e-8):
    """x: [N, C]; gamma, beta: [C]. Returns (y, mean, rstd) as float64."""
    x = _f64(x)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    b = _f64(beta).reshape(C)
    y = np.empty_like(x)
    mean = np.empty(N, np.float64)
    rstd = np.empty(N, np.float64)
    _load().lnr_oracle_layernorm_fw(_p(x), _p(g), _p(b), N, C, float(eps), _p(y), _p(mean), _p(rstd))
    return y, mean, rstd


def layernorm_bw_dx(x, dy, gamma, eps: float = 1e-8) -> np.ndarray:
    x = _f64(x)
    dy = _f64(dy)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    dx = np.empty_like(x)
    _load().lnr_oracle_layernorm_bw_dx(_p(x), _p(dy), _p(g), N, C, float(eps), _p(dx))
    return dx


def layernorm_bw_dgamma_dbeta(x, dy, eps: float = 1e-8):
    x = _f64(x)
    dy = _f64(dy)
    N, C = x.shape
    mu = np.empty(N, np.float64)
    sg = np.empty(N, np.float64)
    dg = np.empty(C, np.float64)
    db = np.empty(C, np.float64)
    _load().lnr_oracle_layernorm_bw_dgamma_dbeta(_p(x), _p(dy), N, C, float(eps), _p(mu), _p(sg), _p(dg), _p(db))
    return dg, db


def layernorm_bw(x, dy, gamma, eps: float = 1e-8):
    """Returns (dx, dgamma, dbeta) as float64."""
    dx = layernorm_bw_dx(x, dy, gamma, eps)
    dg, db = layernorm_bw_dgamma_dbeta(x, dy, eps)
    return dx, dg, db


def layernorm_bw_given_stats(x, dy, gamma, mean, rstd):
    """Backward from saved statistics (mean, rstd per row, e.g. the fp32 values a forward
    kernel stored). Returns (dx, dgamma, dbeta) as float64."""
    x = _f64(x)
    dy = _f64(dy)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    m = _f64(mean).reshape(N)
    r = _f64(rstd).reshape(N)
    dx = np.empty_like(x)
    dg = np.empty(C, np.float64)
    db = np.empty(C, np.float64)
    _load().lnr_oracle_layernorm_bw_given_stats(_p(x), _p(dy), _p(g), _p(m), _p(r), N, C, _p(dx), _p(dg), _p(db))
    return dx, dg, db


def rmsnorm_fw(x, gamma, eps: float = 1e-6):
    """Returns (y, rrms) as float64."""
    x = _f64(x)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    y = np.empty_like(x)
    r = np.empty(N, np.float64)
    _load().lnr_oracle_rmsnorm_fw(_p(x), _p(g), N, C, float(eps), _p(y), _p(r))
    return y, r


def rmsnorm_bw_given_rstd(x, dy, gamma, rstd):
    """RMSNorm backward from a saved rstd per row (e.g. the fp32 values a forward kernel
    stored). Returns (dx, dgamma) as float64."""
    x = _f64(x)
    dy = _f64(dy)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    r = _f64(rstd).reshape(N)
    dx = np.empty_like(x)
    dg = np.empty(C, np.float64)
    _load().lnr_oracle_rmsnorm_bw_given_rstd(_p(x), _p(dy), _p(g), _p(r), N, C, _p(dx), _p(dg))
    return dx, dg


def rmsnorm_bw(x, dy, gamma, eps: float = 1e-6):
    """Returns (dx, dgamma) as float64."""
    x = _f64(x)
    dy = _f64(dy)
    N, C = x.shape
    g = _f64(gamma).reshape(C)
    dx = np.empty_like(x)
    dg = np.empty(C, np.float64)
    _load().lnr_oracle_rmsnorm_bw(_p(x), _p(dy), _p(g), N, C, float(eps), _p(dx), _p(dg))
    return dx, dg


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a CPU torch tensor
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def xent_fw(z, target, ignore_index: int = -100):
    """Softmax cross-entropy per row: returns (loss, lse) as float64. z [N, V]; target [N]."""
    z = _f64(z)
    N, V = z.shape
    t = _i64(target).reshape(N)
    loss = np.empty(N, np.float64)
    lse = np.empty(N, np.float64)
    _load().lnr_oracle_xent_fw(_p(z), t.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, V,
                               int(ignore_index), _p(loss), _p(lse))
    return loss, lse


def xent_bw_given_lse(z, target, lse, dloss, ignore_index: int = -100):
    """Gradient of sum_i dloss_i * loss_i with respect to z, from a given lse per row."""
    z = _f64(z)
    N, V = z.shape
    t = _i64(target).reshape(N)
    l = _f64(lse).reshape(N)
    g = _f64(dloss).reshape(N)
    dz = np.empty_like(z)
    _load().lnr_oracle_xent_bw_given_lse(_p(z), t.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         _p(l), _p(g), N, V, int(ignore_index), _p(dz))
    return dz


def xent_bw(z, target, dloss, ignore_index: int = -100):
    """Gradient with lse recomputed from z in fp64."""
    _, lse = xent_fw(z, target, ignore_index)
    return xent_bw_given_lse(z, target, lse, dloss, ignore_index)


def _u8(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.uint8)


def bdr_ln_fw(x, residual, bias, mask_bits, p, gamma, beta, eps: float = 1e-8):
    """s = residual + keep * (x + bias) / (1 - p), y = LayerNorm(s). mask_bits: uint8
    [N, ceil(C/8)], bit j % 8 of byte j / 8 keeps element j. Returns (s, y, mean, rstd)."""
    x = _f64(x)
    N, C = x.shape
    r = _f64(residual).reshape(N, C)
    b = _f64(bias).reshape(C)
    m = _u8(mask_bits).reshape(N, (C + 7) // 8)
    g = _f64(gamma).reshape(C)
    be = _f64(beta).reshape(C)
    s = np.empty_like(x)
    y = np.empty_like(x)
    mean = np.empty(N, np.float64)
    rstd = np.empty(N, np.float64)
    _load().lnr_oracle_bdr_ln_fw(_p(x), _p(r), _p(b), m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                                 float(p), _p(g), _p(be), N, C, float(eps), _p(s), _p(y), _p(mean),
                                 _p(rstd))
    return s, y, mean, rstd


def bdr_ln_bw(s, dy, ds_extra, mask_bits, p, gamma, mean, rstd):
    """Backward from the saved s, mean, rstd. ds_extra may be None. Returns
    (dresidual, dx, dgamma, dbeta, dbias)."""
    s = _f64(s)
    N, C = s.shape
    dy = _f64(dy).reshape(N, C)
    de = None if ds_extra is None else _f64(ds_extra).reshape(N, C)
    m = _u8(mask_bits).reshape(N, (C + 7) // 8)
    g = _f64(gamma).reshape(C)
    mu = _f64(mean).reshape(N)
    rs = _f64(rstd).reshape(N)
    dres = np.empty_like(s)
    dx = np.empty_like(s)
    dg = np.empty(C, np.float64)
    db = np.empty(C, np.float64)
    dbias = np.empty(C, np.float64)
    _load().lnr_oracle_bdr_ln_bw(_p(s), _p(dy), None if de is None else _p(de),
                                 m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), float(p), _p(g),
                                 _p(mu), _p(rs), N, C, _p(dres), _p(dx), _p(dg), _p(db), _p(dbias))
    return dres, dx, dg, db, dbias
