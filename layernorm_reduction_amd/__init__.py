"""layernorm_reduction_amd -- fused attention-softmax and LayerNorm row reductions for MI355X.

A thin binding over the C ABI of ``liblnr.so`` (declared in ``include/lnr.h``). Every step of
every operation runs in the library's HIP kernels; this module only checks tensors, picks
the dtype code, passes raw device pointers and torch's current HIP stream, and turns a
nonzero status into ``LnrError``. There is no CPU fallback: if the library is missing or a
tensor is not on the GPU, the call raises.

Functions mirror the C entry points:
    attn_softmax_fw(inp, mask=None, causal=False, out=None) -> out
    attn_softmax_bw(dout, out_fw, dinp=None) -> dinp
    layernorm_fw(x, gamma, beta, eps=1e-8, y=None, mean=None, rstd=None) -> (y, mean, rstd)
    layernorm_bw(dy, x, gamma, mean, rstd, dx=None, dgamma=None, dbeta=None,
                 workspace=None) -> (dx, dgamma, dbeta)
    layernorm_bw_workspace_bytes(N, C, dtype) -> int
    layernorm_bw_noalloc(dy, x, gamma, mean, rstd, dx=None, dgamma=None, dbeta=None)
                 -> (dx, dgamma, dbeta)   (the library's own scratch array, no workspace)
    rmsnorm_fw(x, gamma, eps=1e-6, y=None, rstd=None) -> (y, rstd)
    rmsnorm_bw(dy, x, gamma, rstd, dx=None, dgamma=None, workspace=None) -> (dx, dgamma)
    rmsnorm_bw_workspace_bytes(N, C, dtype) -> int
    cross_entropy_fw(logits, target, ignore_index=-100, loss=None, lse=None,
                     workspace=None) -> (loss, lse)
    cross_entropy_bw(logits, target, lse, dloss=None, scale=1.0, ignore_index=-100,
                     dlogits=None) -> dlogits
    cross_entropy_fw_workspace_bytes(N, V, dtype) -> int
    bdr_layernorm_fw(x, residual, bias, keep_mask, p, gamma, beta, eps=1e-8, s=None, y=None,
                     mean=None, rstd=None) -> (s, y, mean, rstd)
    bdr_layernorm_bw(dy, s, keep_mask, p, gamma, mean, rstd, ds_extra=None, ...)
                     -> (dresidual, dx, dgamma, dbeta, dbias)
    bdr_layernorm_bw_workspace_bytes(N, C, dtype) -> int
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LnrError", "load", "library_path", "attn_softmax_fw", "attn_softmax_bw", "layernorm_fw",
    "layernorm_bw", "layernorm_bw_workspace_bytes", "layernorm_bw_noalloc", "rmsnorm_fw", "rmsnorm_bw",
    "rmsnorm_bw_workspace_bytes", "cross_entropy_fw", "cross_entropy_bw",
    "cross_entropy_fw_workspace_bytes", "bdr_layernorm_fw", "bdr_layernorm_bw",
    "bdr_layernorm_bw_workspace_bytes", "copy_bytes", "xor_bytes", "softmax_plan",
    "layernorm_plan", "LNR_F32", "LNR_F16", "SOFTMAX_MAX_TK", "LAYERNORM_MAX_C",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "liblnr.so")

LNR_F32, LNR_F16 = 0, 1
SOFTMAX_MAX_TK = 2048
LAYERNORM_MAX_C = 8192

STATUS_NAMES = {
    0: "LNR_OK", 1: "LNR_ERR_NULL", 2: "LNR_ERR_SHAPE", 3: "LNR_ERR_UNSUPPORTED",
    4: "LNR_ERR_DTYPE", 5: "LNR_ERR_ALIGN", 6: "LNR_ERR_ALIAS", 7: "LNR_ERR_WORKSPACE",
    8: "LNR_ERR_HIP", 9: "LNR_ERR_SCRATCH",
}


class LnrError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({text})")


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load liblnr.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m layernorm_reduction_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.attn_softmax_fw.argtypes = [vp, vp, vp, i64, i64, i64, i64, ci, ci, vp]
    lib.attn_softmax_bw.argtypes = [vp, vp, vp, i64, i64, i64, i64, ci, vp]
    lib.attn_softmax_fw_skip.argtypes = [vp, vp, vp, i64, i64, i64, i64, ci, ci, vp]
    lib.attn_softmax_bw_skip.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, vp]
    lib.layernorm_fw.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, ctypes.c_float, ci, vp]
    lib.layernorm_bw_workspace_bytes.argtypes = [i64, i64, ci]
    lib.layernorm_bw_workspace_bytes.restype = sz
    lib.layernorm_bw.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, vp, sz, vp]
    lib.layernorm_bw_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, ci, vp]
    lib.rmsnorm_fw.argtypes = [vp, vp, vp, vp, i64, i64, ctypes.c_float, ci, vp]
    lib.rmsnorm_bw_workspace_bytes.argtypes = [i64, i64, ci]
    lib.rmsnorm_bw_workspace_bytes.restype = sz
    lib.rmsnorm_bw.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, ci, vp, sz, vp]
    fl = ctypes.c_float
    lib.bdr_layernorm_fw.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, fl, vp, vp, i64, i64, fl, ci, vp]
    lib.bdr_layernorm_bw_workspace_bytes.argtypes = [i64, i64, ci]
    lib.bdr_layernorm_bw_workspace_bytes.restype = sz
    lib.bdr_layernorm_bw.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, fl, vp, vp, vp, i64, i64,
                                     ci, vp, sz, vp]
    lib.cross_entropy_fw_workspace_bytes.argtypes = [i64, i64, ci]
    lib.cross_entropy_fw_workspace_bytes.restype = sz
    lib.cross_entropy_fw.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, sz, vp]
    lib.cross_entropy_bw.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, i64, i64, i64, ci, vp]
    lib.lnr_copy.argtypes = [vp, vp, sz, vp]
    lib.lnr_xor2.argtypes = [vp, vp, vp, sz, vp]
    lib.lnr_time_next_launch.argtypes = [vp, vp]
    lib.lnr_time_next_launch.restype = ci
    lib.lnr_strerror.argtypes = [ci]
    lib.lnr_strerror.restype = ctypes.c_char_p
    lib.lnr_build_info.restype = ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    lib.lnr_softmax_plan.argtypes = [i64, ci, ci, ip, ip, ip]
    lib.lnr_layernorm_plan.argtypes = [i64, i64, ci, ci, ip, ip, ip, ip, ctypes.POINTER(i64)]
    for f in ("attn_softmax_fw", "attn_softmax_bw", "layernorm_fw", "layernorm_bw",
              "layernorm_bw_noalloc", "rmsnorm_fw",
              "rmsnorm_bw", "cross_entropy_fw", "cross_entropy_bw", "bdr_layernorm_fw",
              "bdr_layernorm_bw", "lnr_copy",
              "lnr_xor2", "lnr_softmax_plan", "lnr_layernorm_plan"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise LnrError(status, where, load().lnr_strerror(status).decode())


# ------------------------------------------------------------------------------------------
# Tensor marshalling (torch is used for device memory and streams only).
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return LNR_F16
    if t.dtype == torch.float32:
        return LNR_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use float16 or float32 storage")


def _dev(t, name: str, like=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None:
        if t.device != like.device:
            raise ValueError(f"{name} is on {t.device}, expected {like.device}")
        if t.dtype != like.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {like.dtype}")
    return t


def _f32(t, name: str, like):
    torch = _torch()
    _dev(t, name)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    return t


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------------------------------------
# Operations.
# ------------------------------------------------------------------------------------------

def attn_softmax_fw(inp, mask=None, causal: bool = False, out=None):
    """Masked / causal softmax over the last axis of inp [B, H, Tq, Tk].

    mask: additive [B, Tk] (0 keeps a key, -inf removes it) or None. out may be inp.
    """
    torch = _torch()
    _dev(inp, "inp")
    if inp.dim() != 4:
        raise ValueError("inp must be [B, H, Tq, Tk]")
    B, H, Tq, Tk = inp.shape
    if mask is not None:
        _dev(mask, "mask", like=inp)
        if tuple(mask.shape) != (B, Tk):
            raise ValueError(f"mask must be [B, Tk] = [{B}, {Tk}], got {tuple(mask.shape)}")
    if out is None:
        out = torch.empty_like(inp)
    else:
        _dev(out, "out", like=inp)
        if out.shape != inp.shape:
            raise ValueError("out must have the shape of inp")
    st = load().attn_softmax_fw(_ptr(out), _ptr(inp), _ptr(mask), B, H, Tq, Tk, int(bool(causal)),
                                _dtype_code(inp), _stream(inp))
    _check(st, "attn_softmax_fw")
    return out


def attn_softmax_bw(dout, out_fw, dinp=None):
    """Gradient of attn_softmax_fw: dinp = y * (dout - sum(y * dout)). dinp may be dout."""
    torch = _torch()
    _dev(dout, "dout")
    _dev(out_fw, "out_fw", like=dout)
    if dout.dim() != 4 or out_fw.shape != dout.shape:
        raise ValueError("dout and out_fw must both be [B, H, Tq, Tk]")
    B, H, Tq, Tk = dout.shape
    if dinp is None:
        dinp = torch.empty_like(dout)
    else:
        _dev(dinp, "dinp", like=dout)
        if dinp.shape != dout.shape:
            raise ValueError("dinp must have the shape of dout")
    st = load().attn_softmax_bw(_ptr(dinp), _ptr(dout), _ptr(out_fw), B, H, Tq, Tk,
                                _dtype_code(dout), _stream(dout))
    _check(st, "attn_softmax_bw")
    return dinp


def _softmax_mask(mask, like, B, Tk):
    if mask is not None:
        _dev(mask, "mask", like=like)
        if tuple(mask.shape) != (B, Tk):
            raise ValueError(f"mask must be [B, Tk] = [{B}, {Tk}], got {tuple(mask.shape)}")


def attn_softmax_fw_skip(inp, mask=None, causal: bool = False, out=None):
    """attn_softmax_fw that does not read 16-byte score runs whose keys are all masked
    (after the query when causal, or under -inf mask entries); writes every element."""
    torch = _torch()
    _dev(inp, "inp")
    if inp.dim() != 4:
        raise ValueError("inp must be [B, H, Tq, Tk]")
    B, H, Tq, Tk = inp.shape
    _softmax_mask(mask, inp, B, Tk)
    if out is None:
        out = torch.empty_like(inp)
    else:
        _dev(out, "out", like=inp)
        if out.shape != inp.shape:
            raise ValueError("out must have the shape of inp")
    st = load().attn_softmax_fw_skip(_ptr(out), _ptr(inp), _ptr(mask), B, H, Tq, Tk,
                                     int(bool(causal)), _dtype_code(inp), _stream(inp))
    _check(st, "attn_softmax_fw_skip")
    return out


def attn_softmax_bw_skip(dout, out_fw, mask=None, causal: bool = False, dinp=None):
    """attn_softmax_bw that neither reads y nor dout on 16-byte runs whose keys the forward
    masked (same mask and causal flag as the forward); writes zeros there."""
    torch = _torch()
    _dev(dout, "dout")
    _dev(out_fw, "out_fw", like=dout)
    if dout.dim() != 4 or out_fw.shape != dout.shape:
        raise ValueError("dout and out_fw must both be [B, H, Tq, Tk]")
    B, H, Tq, Tk = dout.shape
    _softmax_mask(mask, dout, B, Tk)
    if dinp is None:
        dinp = torch.empty_like(dout)
    else:
        _dev(dinp, "dinp", like=dout)
        if dinp.shape != dout.shape:
            raise ValueError("dinp must have the shape of dout")
    st = load().attn_softmax_bw_skip(_ptr(dinp), _ptr(dout), _ptr(out_fw), _ptr(mask), B, H, Tq,
                                     Tk, int(bool(causal)), _dtype_code(dout), _stream(dout))
    _check(st, "attn_softmax_bw_skip")
    return dinp


def layernorm_fw(x, gamma, beta, eps: float = 1e-8, y=None, mean=None, rstd=None):
    """LayerNorm over the last axis of x [N, C]; returns (y, mean, rstd) (fp32 stats)."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    N, C = x.shape
    _dev(gamma, "gamma", like=x)
    _dev(beta, "beta", like=x)
    if gamma.numel() != C or beta.numel() != C:
        raise ValueError("gamma and beta must have C elements")
    if y is None:
        y = torch.empty_like(x)
    else:
        _dev(y, "y", like=x)
        if y.shape != x.shape:
            raise ValueError("y must have the shape of x")
    if mean is None:
        mean = torch.empty(N, dtype=torch.float32, device=x.device)
    if rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _f32(mean, "mean", x)
    _f32(rstd, "rstd", x)
    if mean.numel() != N or rstd.numel() != N:
        raise ValueError("mean and rstd must have N elements")
    st = load().layernorm_fw(_ptr(y), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(gamma), _ptr(beta),
                             N, C, float(eps), _dtype_code(x), _stream(x))
    _check(st, "layernorm_fw")
    return y, mean, rstd


def layernorm_bw_workspace_bytes(N: int, C: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (LNR_F16 if str(dtype).endswith("float16") else LNR_F32)
    return int(load().layernorm_bw_workspace_bytes(int(N), int(C), code))


def layernorm_bw(dy, x, gamma, mean, rstd, dx=None, dgamma=None, dbeta=None, workspace=None):
    """LayerNorm backward; returns (dx, dgamma, dbeta).

    workspace: a uint8 GPU tensor of at least layernorm_bw_workspace_bytes(N, C, dtype) bytes,
    16-byte aligned (a fresh allocation is); allocated here when not given.
    """
    torch = _torch()
    _dev(x, "x")
    _dev(dy, "dy", like=x)
    if x.dim() != 2 or dy.shape != x.shape:
        raise ValueError("x and dy must both be [N, C]")
    N, C = x.shape
    _dev(gamma, "gamma", like=x)
    if gamma.numel() != C:
        raise ValueError("gamma must have C elements")
    _f32(mean, "mean", x)
    _f32(rstd, "rstd", x)
    if mean.numel() != N or rstd.numel() != N:
        raise ValueError("mean and rstd must have N elements")
    if dx is None:
        dx = torch.empty_like(x)
    else:
        _dev(dx, "dx", like=x)
    if dgamma is None:
        dgamma = torch.empty(C, dtype=x.dtype, device=x.device)
    else:
        _dev(dgamma, "dgamma", like=x)
    if dbeta is None:
        dbeta = torch.empty(C, dtype=x.dtype, device=x.device)
    else:
        _dev(dbeta, "dbeta", like=x)
    code = _dtype_code(x)
    need = int(load().layernorm_bw_workspace_bytes(N, C, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        _dev(workspace, "workspace")
    st = load().layernorm_bw(_ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dy), _ptr(x), _ptr(gamma),
                             _ptr(mean), _ptr(rstd), N, C, code, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(x))
    _check(st, "layernorm_bw")
    return dx, dgamma, dbeta


def layernorm_bw_noalloc(dy, x, gamma, mean, rstd, dx=None, dgamma=None, dbeta=None):
    """layernorm_bw with the column partials in the library's own device array instead of a
    workspace (for callers that cannot allocate: pass dx, dgamma and dbeta, and this function
    allocates nothing either). Calls that overlap in time on one GPU race on that array.
    Returns (dx, dgamma, dbeta)."""
    torch = _torch()
    _dev(x, "x")
    _dev(dy, "dy", like=x)
    if x.dim() != 2 or dy.shape != x.shape:
        raise ValueError("x and dy must both be [N, C]")
    N, C = x.shape
    _dev(gamma, "gamma", like=x)
    if gamma.numel() != C:
        raise ValueError("gamma must have C elements")
    _f32(mean, "mean", x)
    _f32(rstd, "rstd", x)
    if mean.numel() != N or rstd.numel() != N:
        raise ValueError("mean and rstd must have N elements")
    dx = torch.empty_like(x) if dx is None else dx
    dgamma = torch.empty(C, dtype=x.dtype, device=x.device) if dgamma is None else dgamma
    dbeta = torch.empty(C, dtype=x.dtype, device=x.device) if dbeta is None else dbeta
    for t, nm in ((dx, "dx"), (dgamma, "dgamma"), (dbeta, "dbeta")):
        _dev(t, nm, like=x)
    st = load().layernorm_bw_noalloc(_ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dy), _ptr(x),
                                     _ptr(gamma), _ptr(mean), _ptr(rstd), N, C, _dtype_code(x),
                                     _stream(x))
    _check(st, "layernorm_bw_noalloc")
    return dx, dgamma, dbeta


def rmsnorm_fw(x, gamma, eps: float = 1e-6, y=None, rstd=None):
    """RMSNorm over the last axis of x [N, C]; returns (y, rstd) (fp32 rstd)."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    N, C = x.shape
    _dev(gamma, "gamma", like=x)
    if gamma.numel() != C:
        raise ValueError("gamma must have C elements")
    if y is None:
        y = torch.empty_like(x)
    else:
        _dev(y, "y", like=x)
        if y.shape != x.shape:
            raise ValueError("y must have the shape of x")
    if rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _f32(rstd, "rstd", x)
    if rstd.numel() != N:
        raise ValueError("rstd must have N elements")
    st = load().rmsnorm_fw(_ptr(y), _ptr(rstd), _ptr(x), _ptr(gamma), N, C, float(eps),
                           _dtype_code(x), _stream(x))
    _check(st, "rmsnorm_fw")
    return y, rstd


def rmsnorm_bw_workspace_bytes(N: int, C: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (LNR_F16 if str(dtype).endswith("float16") else LNR_F32)
    return int(load().rmsnorm_bw_workspace_bytes(int(N), int(C), code))


def rmsnorm_bw(dy, x, gamma, rstd, dx=None, dgamma=None, workspace=None):
    """RMSNorm backward; returns (dx, dgamma).

    workspace: a uint8 GPU tensor of at least rmsnorm_bw_workspace_bytes(N, C, dtype) bytes,
    16-byte aligned; allocated here when not given.
    """
    torch = _torch()
    _dev(x, "x")
    _dev(dy, "dy", like=x)
    if x.dim() != 2 or dy.shape != x.shape:
        raise ValueError("x and dy must both be [N, C]")
    N, C = x.shape
    _dev(gamma, "gamma", like=x)
    if gamma.numel() != C:
        raise ValueError("gamma must have C elements")
    _f32(rstd, "rstd", x)
    if rstd.numel() != N:
        raise ValueError("rstd must have N elements")
    if dx is None:
        dx = torch.empty_like(x)
    else:
        _dev(dx, "dx", like=x)
    if dgamma is None:
        dgamma = torch.empty(C, dtype=x.dtype, device=x.device)
    else:
        _dev(dgamma, "dgamma", like=x)
    code = _dtype_code(x)
    need = int(load().rmsnorm_bw_workspace_bytes(N, C, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        _dev(workspace, "workspace")
    st = load().rmsnorm_bw(_ptr(dx), _ptr(dgamma), _ptr(dy), _ptr(x), _ptr(gamma), _ptr(rstd), N, C,
                           code, _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(x))
    _check(st, "rmsnorm_bw")
    return dx, dgamma


def _keep_mask(keep_mask, N, C, like):
    torch = _torch()
    if not keep_mask.is_cuda or keep_mask.device != like.device:
        raise ValueError("keep_mask must be on the same GPU as x")
    if keep_mask.dtype != torch.uint8 or not keep_mask.is_contiguous() or \
            keep_mask.numel() != N * ((C + 7) // 8):
        raise ValueError("keep_mask must be a contiguous uint8 tensor of N * ceil(C/8) bytes")


def bdr_layernorm_bw_workspace_bytes(N: int, C: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (LNR_F16 if str(dtype).endswith("float16") else LNR_F32)
    return int(load().bdr_layernorm_bw_workspace_bytes(int(N), int(C), code))


def bdr_layernorm_fw(x, residual, bias, keep_mask, p, gamma, beta, eps: float = 1e-8, s=None,
                     y=None, mean=None, rstd=None):
    """s = residual + keep * (x + bias) / (1 - p); y = LayerNorm(s). keep_mask: uint8
    [N, ceil(C/8)], bit j % 8 of byte j / 8 keeps element j. Returns (s, y, mean, rstd)."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    N, C = x.shape
    _dev(residual, "residual", like=x)
    if residual.shape != x.shape:
        raise ValueError("residual must have the shape of x")
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _dev(t, nm, like=x)
        if t.numel() != C:
            raise ValueError(f"{nm} must have C elements")
    _keep_mask(keep_mask, N, C, x)
    s = torch.empty_like(x) if s is None else s
    y = torch.empty_like(x) if y is None else y
    _dev(s, "s", like=x)
    _dev(y, "y", like=x)
    if mean is None:
        mean = torch.empty(N, dtype=torch.float32, device=x.device)
    if rstd is None:
        rstd = torch.empty(N, dtype=torch.float32, device=x.device)
    _f32(mean, "mean", x)
    _f32(rstd, "rstd", x)
    st = load().bdr_layernorm_fw(_ptr(s), _ptr(y), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(residual),
                                 _ptr(bias), _ptr(keep_mask), float(p), _ptr(gamma), _ptr(beta), N,
                                 C, float(eps), _dtype_code(x), _stream(x))
    _check(st, "bdr_layernorm_fw")
    return s, y, mean, rstd


def bdr_layernorm_bw(dy, s, keep_mask, p, gamma, mean, rstd, ds_extra=None, dresidual=None,
                     dx=None, dgamma=None, dbeta=None, dbias=None, workspace=None):
    """Backward of bdr_layernorm_fw from the saved s, mean, rstd; ds_extra is a gradient
    reaching s by another path (None: none). Returns (dresidual, dx, dgamma, dbeta, dbias).
    workspace: a uint8 GPU tensor of at least bdr_layernorm_bw_workspace_bytes(N, C, dtype)
    bytes, 16-byte aligned; allocated here when not given."""
    torch = _torch()
    _dev(s, "s")
    if s.dim() != 2:
        raise ValueError("s must be [N, C]")
    N, C = s.shape
    _dev(dy, "dy", like=s)
    if dy.shape != s.shape:
        raise ValueError("dy must have the shape of s")
    if ds_extra is not None:
        _dev(ds_extra, "ds_extra", like=s)
    _dev(gamma, "gamma", like=s)
    _keep_mask(keep_mask, N, C, s)
    _f32(mean, "mean", s)
    _f32(rstd, "rstd", s)
    dresidual = torch.empty_like(s) if dresidual is None else dresidual
    dx = torch.empty_like(s) if dx is None else dx
    dgamma = torch.empty(C, dtype=s.dtype, device=s.device) if dgamma is None else dgamma
    dbeta = torch.empty(C, dtype=s.dtype, device=s.device) if dbeta is None else dbeta
    dbias = torch.empty(C, dtype=s.dtype, device=s.device) if dbias is None else dbias
    code = _dtype_code(s)
    need = int(load().bdr_layernorm_bw_workspace_bytes(N, C, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=s.device)
    st = load().bdr_layernorm_bw(_ptr(dresidual), _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dbias),
                                 _ptr(dy), _ptr(ds_extra), _ptr(s), _ptr(keep_mask), float(p),
                                 _ptr(gamma), _ptr(mean), _ptr(rstd), N, C, code, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(s))
    _check(st, "bdr_layernorm_bw")
    return dresidual, dx, dgamma, dbeta, dbias


def _targets(target, N, like):
    torch = _torch()
    if not target.is_cuda or target.device != like.device:
        raise ValueError("target must be on the same GPU as the logits")
    if target.dtype != torch.int64 or not target.is_contiguous() or target.numel() != N:
        raise ValueError("target must be a contiguous int64 tensor of N elements")


def cross_entropy_fw_workspace_bytes(N: int, V: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (LNR_F16 if str(dtype).endswith("float16") else LNR_F32)
    return int(load().cross_entropy_fw_workspace_bytes(int(N), int(V), code))


def cross_entropy_fw(logits, target, ignore_index: int = -100, loss=None, lse=None, workspace=None):
    """Softmax cross-entropy per row of logits [N, V]; returns (loss, lse), both fp32 [N]."""
    torch = _torch()
    _dev(logits, "logits")
    if logits.dim() != 2:
        raise ValueError("logits must be [N, V]")
    N, V = logits.shape
    _targets(target, N, logits)
    if loss is None:
        loss = torch.empty(N, dtype=torch.float32, device=logits.device)
    if lse is None:
        lse = torch.empty(N, dtype=torch.float32, device=logits.device)
    _f32(loss, "loss", logits)
    _f32(lse, "lse", logits)
    if loss.numel() != N or lse.numel() != N:
        raise ValueError("loss and lse must have N elements")
    code = _dtype_code(logits)
    need = int(load().cross_entropy_fw_workspace_bytes(N, V, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().cross_entropy_fw(_ptr(loss), _ptr(lse), _ptr(logits), _ptr(target), N, V,
                                 int(ignore_index), code, _ptr(workspace), wb, _stream(logits))
    _check(st, "cross_entropy_fw")
    return loss, lse


def cross_entropy_bw(logits, target, lse, dloss=None, scale: float = 1.0, ignore_index: int = -100,
                     dlogits=None):
    """Gradient of sum_i scale * dloss_i * loss_i with respect to logits (dloss None: ones)."""
    torch = _torch()
    _dev(logits, "logits")
    if logits.dim() != 2:
        raise ValueError("logits must be [N, V]")
    N, V = logits.shape
    _targets(target, N, logits)
    _f32(lse, "lse", logits)
    if dloss is not None:
        _f32(dloss, "dloss", logits)
        if dloss.numel() != N:
            raise ValueError("dloss must have N elements")
    if dlogits is None:
        dlogits = torch.empty_like(logits)
    else:
        _dev(dlogits, "dlogits", like=logits)
    st = load().cross_entropy_bw(_ptr(dlogits), _ptr(logits), _ptr(target), _ptr(lse), _ptr(dloss),
                                 float(scale), N, V, int(ignore_index), _dtype_code(logits),
                                 _stream(logits))
    _check(st, "cross_entropy_bw")
    return dlogits


def copy_bytes(dst, src):
    """Streaming 16-byte-vector copy of src into dst (measurement helper)."""
    _dev(src, "src")
    _dev(dst, "dst")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(load().lnr_copy(_ptr(dst), _ptr(src), n, _stream(src)), "lnr_copy")
    return dst


def xor_bytes(dst, a, b):
    """dst = a XOR b bytewise: reads two buffers, writes one (measurement helper)."""
    for t, nm in ((a, "a"), (b, "b"), (dst, "dst")):
        _dev(t, nm)
    n = a.numel() * a.element_size()
    if b.numel() * b.element_size() < n or dst.numel() * dst.element_size() < n:
        raise ValueError("b and dst must be at least as large as a")
    _check(load().lnr_xor2(_ptr(dst), _ptr(a), _ptr(b), n, _stream(a)), "lnr_xor2")
    return dst


def softmax_plan(Tk: int, dtype_code: int, backward: bool = False, skip: bool = False):
    """(bucket, lanes per row, 16-byte vectors per lane) of the forward or backward kernel (of
    the read-skipping entry points with skip=True) for aligned buffers; bucket 0 means the
    element-wise fallback."""
    b, g, it = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    which = int(bool(backward)) + (2 if skip else 0)
    _check(load().lnr_softmax_plan(int(Tk), int(dtype_code), which, ctypes.byref(b),
                                   ctypes.byref(g), ctypes.byref(it)), "lnr_softmax_plan")
    return b.value, g.value, it.value


def layernorm_plan(N: int, C: int, dtype_code: int, backward: bool = False):
    """(bucket, lanes per row, vectors per lane, workgroup size, blocks) of the LayerNorm
    forward or backward kernel."""
    b, g, it, wg = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    blocks = ctypes.c_int64()
    _check(load().lnr_layernorm_plan(int(N), int(C), int(dtype_code), int(bool(backward)),
                                     ctypes.byref(b), ctypes.byref(g), ctypes.byref(it),
                                     ctypes.byref(wg), ctypes.byref(blocks)), "lnr_layernorm_plan")
    return b.value, g.value, it.value, wg.value, blocks.value


# ------------------------------------------------------------------------------------------
# Bound calls: validate tensors once, then re-issue the same C call with no Python checks.
# For launch-bound loops (benchmarks, training steps with fixed buffers). The tensors must
# stay alive and unchanged in shape while the bound call is used.
# ------------------------------------------------------------------------------------------

class BoundCall:
    """A C-ABI call with fixed arguments; calling it enqueues the kernels again."""
    __slots__ = ("name", "_fn", "_args", "_keep")

    def __init__(self, name, fn, args, keep):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            _check(st, self.name)


def bind_attn_softmax_fw(inp, mask, causal, out):
    attn_softmax_fw(inp, mask, causal, out)          # full validation once
    B, H, Tq, Tk = inp.shape
    args = (out.data_ptr(), inp.data_ptr(), _ptr(mask), B, H, Tq, Tk, int(bool(causal)),
            _dtype_code(inp), _stream(inp))
    return BoundCall("attn_softmax_fw", load().attn_softmax_fw, args, (inp, mask, out))


def bind_attn_softmax_bw(dout, out_fw, dinp):
    attn_softmax_bw(dout, out_fw, dinp)
    B, H, Tq, Tk = dout.shape
    args = (dinp.data_ptr(), dout.data_ptr(), out_fw.data_ptr(), B, H, Tq, Tk, _dtype_code(dout),
            _stream(dout))
    return BoundCall("attn_softmax_bw", load().attn_softmax_bw, args, (dout, out_fw, dinp))


def bind_attn_softmax_fw_skip(inp, mask, causal, out):
    attn_softmax_fw_skip(inp, mask, causal, out)
    B, H, Tq, Tk = inp.shape
    args = (out.data_ptr(), inp.data_ptr(), _ptr(mask), B, H, Tq, Tk, int(bool(causal)),
            _dtype_code(inp), _stream(inp))
    return BoundCall("attn_softmax_fw_skip", load().attn_softmax_fw_skip, args, (inp, mask, out))


def bind_attn_softmax_bw_skip(dout, out_fw, mask, causal, dinp):
    attn_softmax_bw_skip(dout, out_fw, mask, causal, dinp)
    B, H, Tq, Tk = dout.shape
    args = (dinp.data_ptr(), dout.data_ptr(), out_fw.data_ptr(), _ptr(mask), B, H, Tq, Tk,
            int(bool(causal)), _dtype_code(dout), _stream(dout))
    return BoundCall("attn_softmax_bw_skip", load().attn_softmax_bw_skip, args,
                     (dout, out_fw, mask, dinp))


def bind_layernorm_fw(x, gamma, beta, eps, y, mean, rstd):
    layernorm_fw(x, gamma, beta, eps, y, mean, rstd)
    N, C = x.shape
    args = (y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), x.data_ptr(), gamma.data_ptr(),
            beta.data_ptr(), N, C, float(eps), _dtype_code(x), _stream(x))
    return BoundCall("layernorm_fw", load().layernorm_fw, args, (x, gamma, beta, y, mean, rstd))


def bind_layernorm_bw(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace):
    layernorm_bw(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace)
    N, C = x.shape
    args = (dx.data_ptr(), dgamma.data_ptr(), dbeta.data_ptr(), dy.data_ptr(), x.data_ptr(),
            gamma.data_ptr(), mean.data_ptr(), rstd.data_ptr(), N, C, _dtype_code(x),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(x))
    return BoundCall("layernorm_bw", load().layernorm_bw, args,
                     (dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace))


def bind_bdr_layernorm_fw(x, residual, bias, keep_mask, p, gamma, beta, eps, s, y, mean, rstd):
    bdr_layernorm_fw(x, residual, bias, keep_mask, p, gamma, beta, eps, s, y, mean, rstd)
    N, C = x.shape
    args = (s.data_ptr(), y.data_ptr(), mean.data_ptr(), rstd.data_ptr(), x.data_ptr(),
            residual.data_ptr(), bias.data_ptr(), keep_mask.data_ptr(), float(p), gamma.data_ptr(),
            beta.data_ptr(), N, C, float(eps), _dtype_code(x), _stream(x))
    return BoundCall("bdr_layernorm_fw", load().bdr_layernorm_fw, args,
                     (x, residual, bias, keep_mask, gamma, beta, s, y, mean, rstd))


def bind_bdr_layernorm_bw(dy, s, keep_mask, p, gamma, mean, rstd, ds_extra, dresidual, dx, dgamma,
                          dbeta, dbias, workspace):
    bdr_layernorm_bw(dy, s, keep_mask, p, gamma, mean, rstd, ds_extra, dresidual, dx, dgamma, dbeta,
                     dbias, workspace)
    N, C = s.shape
    args = (dresidual.data_ptr(), dx.data_ptr(), dgamma.data_ptr(), dbeta.data_ptr(), dbias.data_ptr(),
            dy.data_ptr(), _ptr(ds_extra), s.data_ptr(), keep_mask.data_ptr(), float(p),
            gamma.data_ptr(), mean.data_ptr(), rstd.data_ptr(), N, C, _dtype_code(s),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(s))
    return BoundCall("bdr_layernorm_bw", load().bdr_layernorm_bw, args,
                     (dy, s, keep_mask, gamma, mean, rstd, ds_extra, dresidual, dx, dgamma, dbeta,
                      dbias, workspace))


def bind_cross_entropy_fw(logits, target, ignore_index, loss, lse, workspace):
    cross_entropy_fw(logits, target, ignore_index, loss, lse, workspace)
    N, V = logits.shape
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (loss.data_ptr(), lse.data_ptr(), logits.data_ptr(), target.data_ptr(), N, V,
            int(ignore_index), _dtype_code(logits), _ptr(workspace), wb, _stream(logits))
    return BoundCall("cross_entropy_fw", load().cross_entropy_fw, args,
                     (logits, target, loss, lse, workspace))


def bind_cross_entropy_bw(logits, target, lse, dloss, scale, ignore_index, dlogits):
    cross_entropy_bw(logits, target, lse, dloss, scale, ignore_index, dlogits)
    N, V = logits.shape
    args = (dlogits.data_ptr(), logits.data_ptr(), target.data_ptr(), lse.data_ptr(), _ptr(dloss),
            float(scale), N, V, int(ignore_index), _dtype_code(logits), _stream(logits))
    return BoundCall("cross_entropy_bw", load().cross_entropy_bw, args,
                     (logits, target, lse, dloss, dlogits))


def bind_rmsnorm_fw(x, gamma, eps, y, rstd):
    rmsnorm_fw(x, gamma, eps, y, rstd)
    N, C = x.shape
    args = (y.data_ptr(), rstd.data_ptr(), x.data_ptr(), gamma.data_ptr(), N, C, float(eps),
            _dtype_code(x), _stream(x))
    return BoundCall("rmsnorm_fw", load().rmsnorm_fw, args, (x, gamma, y, rstd))


def bind_rmsnorm_bw(dy, x, gamma, rstd, dx, dgamma, workspace):
    rmsnorm_bw(dy, x, gamma, rstd, dx, dgamma, workspace)
    N, C = x.shape
    args = (dx.data_ptr(), dgamma.data_ptr(), dy.data_ptr(), x.data_ptr(), gamma.data_ptr(),
            rstd.data_ptr(), N, C, _dtype_code(x), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), _stream(x))
    return BoundCall("rmsnorm_bw", load().rmsnorm_bw, args, (dy, x, gamma, rstd, dx, dgamma, workspace))
