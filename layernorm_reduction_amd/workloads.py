"""Seeded synthetic inputs and algorithmic byte counts for the five benchmark workloads.

This module draws random tensors and counts bytes; it holds none of the softmax or
LayerNorm arithmetic. The HIP path and the CPU oracle both take their inputs from here
and from nowhere else, so both sides see identical stored bits.

Recipe (every tensor drawn on the CPU in float32 with its own ``torch.Generator``, then
cast to the storage dtype; the oracle reads the cast values):
  seed = 1000 * workload + 10 * variant + k, with k naming the tensor:
    0 scores, 1 valid key lengths, 2 softmax upstream grad, 3 LayerNorm input,
    4 per-row offset, 5 gamma, 6 beta, 7 LayerNorm upstream grad.
  * "N(m, v)" in a workload description is read as mean m and VARIANCE v, so the
    per-row offset N(0,4) has standard deviation 2 and beta N(0,0.1) has std sqrt(0.1).
  * A valid length "U[a,b]" is an integer drawn uniformly from a..b inclusive, one per
    batch entry; key positions j >= L_b get an additive mask value of -inf, the rest 0.
  * Tensors beyond 4 GiB (the large-tensor tests) are drawn on the GPU by ``device_normal``,
    ``device_uniform`` and ``device_bytes`` with a seeded device generator, directly in the storage dtype; the
    oracle reads the sampled rows back from the same stored values.

Shapes follow the pages' workloads: the GPT-2 training shapes B=32, T=256, C=256, H=8 of
"FastTransformer: Breaking the Compiler Ceiling ..." (section 1), the row-length template
list {32, ..., 2048} of "CMU 11-868 HW4 ..." ("Problem structure and scoring"), and the
max_seq_len = 512 of the LightSeq layer configuration quoted on the L10 lecture page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Row-length template list for the softmax backward ("Problem structure and scoring").
SOFTMAX_TK_SWEEP = (32, 64, 128, 256, 384, 512, 768, 1024, 2048)
LAYERNORM_C_SWEEP = (256, 768, 1024, 4096, 8192)
LN_EPS = 1e-8
# RMSNorm: the FastTransformer page's module (section 5.4) uses eps = 1e-6 and d_model = 256
# with the GPT-2 batch of section 1 (B = 32, T = 256, so 8192 rows).
RMS_EPS = 1e-6

K_SCORES, K_LENGTHS, K_SDY, K_X, K_OFFSET, K_GAMMA, K_BETA, K_LNDY = range(8)


def seed_of(workload: int, k: int, variant: int = 0) -> int:
    return 1000 * workload + 10 * variant + k


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, mean: float = 0.0, var: float = 1.0) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(seed), dtype=torch.float32)
    if var != 1.0:
        t.mul_(math.sqrt(var))
    if mean != 0.0:
        t.add_(mean)
    return t


def device_normal(shape, seed: int, dtype, device, std: float = 1.0) -> torch.Tensor:
    """Seeded N(0, std^2) drawn on `device` in `dtype` (tensors too large to draw on the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=dtype)
    return t.mul_(std) if std != 1.0 else t


def device_uniform(shape, seed: int, lo: float, hi: float, dtype, device) -> torch.Tensor:
    """Seeded U[lo, hi) drawn on `device` in `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, device=device, dtype=dtype).mul_(hi - lo).add_(lo)


def device_bytes(shape, seed: int, device) -> torch.Tensor:
    """Seeded uniform bytes drawn on `device` (keep-bit masks of the large-tensor tests)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.uint8)


def uniform(shape, seed: int, lo: float, hi: float) -> torch.Tensor:
    t = torch.rand(shape, generator=_gen(seed), dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def valid_lengths(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Integer lengths drawn uniformly from lo..hi inclusive, one per batch entry."""
    return torch.randint(lo, hi + 1, (B,), generator=_gen(seed), dtype=torch.int64)


def padding_mask(lengths: torch.Tensor, Tk: int, dtype: torch.dtype) -> torch.Tensor:
    """Additive key-padding mask [B, Tk]: 0 where j < L_b, -inf where j >= L_b."""
    j = torch.arange(Tk, dtype=torch.int64).unsqueeze(0)
    m = torch.zeros((lengths.numel(), Tk), dtype=torch.float32)
    m[j >= lengths.unsqueeze(1)] = float("-inf")
    return m.to(dtype)


@dataclass
class SoftmaxCase:
    name: str
    B: int
    H: int
    Tq: int
    Tk: int
    causal: bool
    dtype: torch.dtype
    x: torch.Tensor            # [B, H, Tq, Tk] storage dtype, CPU
    dy: torch.Tensor           # [B, H, Tq, Tk] storage dtype, CPU
    mask: torch.Tensor | None  # [B, Tk] storage dtype, CPU, or None
    lengths: torch.Tensor | None = None

    @property
    def rows(self) -> int:
        return self.B * self.H * self.Tq


@dataclass
class LayerNormCase:
    name: str
    N: int
    C: int
    dtype: torch.dtype
    x: torch.Tensor
    gamma: torch.Tensor
    beta: torch.Tensor
    dy: torch.Tensor
    eps: float = LN_EPS


def softmax_case(name, B, H, Tq, Tk, *, causal, dtype, seed_base, score_scale=1.0,
                 len_range=None) -> SoftmaxCase:
    """Seeded scores ~N(0,1)*score_scale, dy ~N(0,1), optional key-padding mask."""
    x = normal((B, H, Tq, Tk), seed_base + K_SCORES)
    if score_scale != 1.0:
        x.mul_(score_scale)
    dy = normal((B, H, Tq, Tk), seed_base + K_SDY)
    mask = lengths = None
    if len_range is not None:
        lengths = valid_lengths(B, len_range[0], len_range[1], seed_base + K_LENGTHS)
        mask = padding_mask(lengths, Tk, dtype)
    return SoftmaxCase(name, B, H, Tq, Tk, causal, dtype, x.to(dtype), dy.to(dtype), mask, lengths)


def layernorm_case(name, N, C, *, dtype, seed_base, row_offset_var=None, gamma_uniform=True,
                   beta_var=0.1, eps=LN_EPS) -> LayerNormCase:
    x = normal((N, C), seed_base + K_X)
    if row_offset_var is not None:
        x.add_(normal((N, 1), seed_base + K_OFFSET, var=row_offset_var))
    if gamma_uniform:
        gamma = uniform((C,), seed_base + K_GAMMA, 0.5, 1.5)
    else:
        gamma = normal((C,), seed_base + K_GAMMA)
    beta = normal((C,), seed_base + K_BETA, var=beta_var)
    dy = normal((N, C), seed_base + K_LNDY)
    return LayerNormCase(name, N, C, dtype, x.to(dtype), gamma.to(dtype), beta.to(dtype),
                         dy.to(dtype), eps)


# ------------------------------------------------------------------------------------------
# The five workloads.
# ------------------------------------------------------------------------------------------

def workload1():
    """Tiny fp32: softmax [2,2,16,16] (padding U[8,16], causal), LayerNorm [64,64]."""
    s = softmax_case("w1-softmax-2x2x16x16-causal-padded-f32", 2, 2, 16, 16, causal=True,
                     dtype=torch.float32, seed_base=seed_of(1, 0), len_range=(8, 16))
    ln = layernorm_case("w1-layernorm-64x64-f32", 64, 64, dtype=torch.float32,
                        seed_base=seed_of(1, 0))
    return [s], [ln]


def workload2():
    """GPT-2 training shapes B=32, T=256, C=256, H=8, fp16 storage."""
    s = softmax_case("w2-softmax-32x8x256x256-causal-f16", 32, 8, 256, 256, causal=True,
                     dtype=torch.float16, seed_base=seed_of(2, 0),
                     score_scale=1.0 / math.sqrt(32.0))
    ln = layernorm_case("w2-layernorm-8192x256-f16", 8192, 256, dtype=torch.float16,
                        seed_base=seed_of(2, 0))
    return [s], [ln]


def workload3_batch(Tk: int) -> int:
    """B chosen so each fp16 score tensor holds about 2^27 elements (256 MiB), H = 8."""
    return max(1, round(2 ** 27 / (8 * Tk * Tk)))


def workload3_case(Tk: int, causal: bool) -> SoftmaxCase:
    v = SOFTMAX_TK_SWEEP.index(Tk)
    B = workload3_batch(Tk)
    return softmax_case(f"w3-softmax-{B}x8x{Tk}x{Tk}-{'causal' if causal else 'full'}-padded-f16",
                        B, 8, Tk, Tk, causal=causal, dtype=torch.float16,
                        seed_base=seed_of(3, 0, v), len_range=(Tk // 2, Tk))


def workload4_case(C: int) -> LayerNormCase:
    v = LAYERNORM_C_SWEEP.index(C)
    return layernorm_case(f"w4-layernorm-16384x{C}-offset-f16", 16384, C, dtype=torch.float16,
                          seed_base=seed_of(4, 0, v), row_offset_var=4.0)


def workload5_softmax(dtype=torch.float16) -> SoftmaxCase:
    tag = "f16" if dtype == torch.float16 else "f32"
    return softmax_case(f"w5-softmax-64x16x512x512-padded-{tag}", 64, 16, 512, 512, causal=False,
                        dtype=dtype, seed_base=seed_of(5, 0), len_range=(256, 512))


def workload5_layernorm(C: int, dtype=torch.float16) -> LayerNormCase:
    tag = "f16" if dtype == torch.float16 else "f32"
    v = {1024: 0, 4096: 1}[C]
    return layernorm_case(f"w5-layernorm-32768x{C}-{tag}", 32768, C, dtype=dtype,
                          seed_base=seed_of(5, 0, v), gamma_uniform=False, beta_var=1.0)


def rmsnorm_gpt2_case(dtype=torch.float16) -> LayerNormCase:
    """RMSNorm [8192, 256]: the FastTransformer page's Pre-RMSNorm at its own model width and
    batch. x, dy ~ N(0,1); weight ~ U(0.5,1.5) (the page initialises it to ones; a random
    weight exercises the product); no bias."""
    tag = "f16" if dtype == torch.float16 else "f32"
    return layernorm_case(f"rms-8192x256-{tag}", 8192, 256, dtype=dtype,
                          seed_base=seed_of(6, 0), eps=RMS_EPS)


def rmsnorm_sweep_case(N: int, C: int, dtype=torch.float16) -> LayerNormCase:
    """RMSNorm at the LayerNorm sweep's shapes, x with a per-row N(0,4) offset (so mean(x^2)
    is dominated by the offset in some rows), dy ~ N(0,1)."""
    tag = "f16" if dtype == torch.float16 else "f32"
    return layernorm_case(f"rms-{N}x{C}-offset-{tag}", N, C, dtype=dtype,
                          seed_base=seed_of(6, 0, 1 + (LAYERNORM_C_SWEEP.index(C) if C in LAYERNORM_C_SWEEP else 9)),
                          row_offset_var=4.0, eps=RMS_EPS)


# ------------------------------------------------------------------------------------------
# Bias + dropout + residual feeding LayerNorm (the L10 page's elementwise kernel before the
# LayerNorm reduce kernel). The page gives no dropout rate; p = 0.1 is the workload rate,
# with 0 and 0.5 as edge cases. The keep mask is drawn here (keep iff a uniform draw >= p)
# and packed one bit per element, least significant bit first (numpy's packbits, bitorder
# "little"): the kernels and the oracle both read the same bits.
# ------------------------------------------------------------------------------------------
BDR_P = 0.1


@dataclass
class BdrCase:
    name: str
    N: int
    C: int
    dtype: torch.dtype
    p: float
    x: torch.Tensor
    residual: torch.Tensor
    bias: torch.Tensor
    gamma: torch.Tensor
    beta: torch.Tensor
    keep: torch.Tensor       # bool [N, C]
    mask: torch.Tensor       # uint8 [N, ceil(C/8)]
    dy: torch.Tensor
    ds_extra: torch.Tensor
    eps: float = LN_EPS


def pack_keep_bits(keep: torch.Tensor) -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.packbits(keep.numpy(), axis=1, bitorder="little"))


def bdr_case(name, N, C, *, dtype, seed_base, p=BDR_P) -> BdrCase:
    """x ~ N(0,1) (the GEMM output before its bias), residual ~ N(0,1) plus a per-row N(0,1)
    offset, bias ~ N(0, 0.1), gamma ~ U(0.5,1.5), beta ~ N(0,0.1), dy and ds_extra ~ N(0,1)."""
    x = normal((N, C), seed_base + K_X)
    residual = normal((N, C), seed_base + K_SCORES).add_(normal((N, 1), seed_base + K_OFFSET))
    bias = normal((C,), seed_base + K_LENGTHS, var=0.1)
    gamma = uniform((C,), seed_base + K_GAMMA, 0.5, 1.5)
    beta = normal((C,), seed_base + K_BETA, var=0.1)
    keep = torch.rand((N, C), generator=_gen(seed_base + K_SDY)) >= p
    dy = normal((N, C), seed_base + K_LNDY)
    ds_extra = normal((N, C), seed_base + K_LNDY + 100)
    return BdrCase(name, N, C, dtype, p, x.to(dtype), residual.to(dtype), bias.to(dtype),
                   gamma.to(dtype), beta.to(dtype), keep, pack_keep_bits(keep), dy.to(dtype),
                   ds_extra.to(dtype))


def bdr_fw_bytes(N, C, s) -> int:
    """Read x, residual, mask bits; write s, y, fp32 mean and rstd; read bias, gamma, beta."""
    return 4 * N * C * s + N * ((C + 7) // 8) + 8 * N + 3 * C * s


def bdr_bw_bytes(N, C, s, extra=False) -> int:
    """Read dy, s, mask bits (and ds_extra), fp32 mean and rstd, gamma; write dresidual, dx,
    dgamma, dbeta, dbias."""
    return (5 if extra else 4) * N * C * s + N * ((C + 7) // 8) + 8 * N + 4 * C * s


# ------------------------------------------------------------------------------------------
# Softmax cross-entropy over a vocabulary (the L10 page's third reduce kernel). The pages give
# no shapes; these stand in for a language-model head: the GPT-2 batch of [FT] section 1
# (B = 32, T = 256: 8192 tokens) over vocabularies of 10^4 - 10^5 entries, one a multiple of
# 8 (every fp16 row 16-byte aligned) and one odd (rows start at every 16-byte phase).
# ------------------------------------------------------------------------------------------
XENT_VOCABS = (32000, 50001)
XENT_IGNORE = -100


@dataclass
class XentCase:
    name: str
    N: int
    V: int
    dtype: torch.dtype
    logits: torch.Tensor
    target: torch.Tensor
    dloss: torch.Tensor
    ignore_index: int = XENT_IGNORE


def xent_case(name, N, V, *, dtype, seed_base, logit_std=2.0, ignore_frac=0.05) -> XentCase:
    """logits ~ N(0, logit_std^2); targets uniform over [0, V) with about ignore_frac of the
    rows set to the ignore index (padding tokens); dloss ~ N(0, 1) per row."""
    logits = normal((N, V), seed_base + K_SCORES, var=logit_std * logit_std)
    target = torch.randint(0, V, (N,), generator=_gen(seed_base + K_LENGTHS), dtype=torch.int64)
    pad = torch.rand(N, generator=_gen(seed_base + K_OFFSET)) < ignore_frac
    target[pad] = XENT_IGNORE
    dloss = normal((N,), seed_base + K_SDY)
    return XentCase(name, N, V, dtype, logits.to(dtype), target, dloss)


def xent_tokens_case(V: int, dtype=torch.float16, N: int = 8192) -> XentCase:
    tag = "f16" if dtype == torch.float16 else "f32"
    v = XENT_VOCABS.index(V) if V in XENT_VOCABS else 9
    return xent_case(f"xent-{N}x{V}-{tag}", N, V, dtype=dtype, seed_base=seed_of(7, 0, v))


def xent_fw_bytes(N, V, s) -> int:
    """Read logits and int64 targets; write fp32 loss and lse."""
    return N * V * s + 8 * N + 8 * N


def xent_bw_bytes(N, V, s) -> int:
    """Read logits, int64 targets, fp32 lse and dloss; write dlogits."""
    return 2 * N * V * s + 8 * N + 8 * N


# ------------------------------------------------------------------------------------------
# Algorithmic bytes: each tensor read or written once, dense (masked positions included).
# ------------------------------------------------------------------------------------------

def dtype_size(dtype: torch.dtype) -> int:
    return {torch.float16: 2, torch.float32: 4}[dtype]


def softmax_fw_bytes(B, H, Tq, Tk, s, has_mask=True) -> int:
    """Read scores, write probabilities, read the [B, Tk] mask."""
    E = B * H * Tq * Tk
    return 2 * E * s + (B * Tk * s if has_mask else 0)


def softmax_bw_bytes(B, H, Tq, Tk, s) -> int:
    """Read y and dy, write dx."""
    return 3 * B * H * Tq * Tk * s


def softmax_open_runs(mask, causal, B, H, Tq, Tk, V) -> int:
    """Number of 16-byte runs (V elements) of a [B, H, Tq, Tk] score tensor that hold at least
    one key the row may attend to: not after the query when causal, not under a -inf entry of
    the [B, Tk] mask (a CPU tensor or None). The skipping kernels read exactly these runs."""
    import numpy as np
    nr = Tk // V
    if mask is None:
        per_q = np.minimum(np.arange(Tq) // V + 1, nr) if causal else np.full(Tq, nr)
        return int(per_q.sum()) * H * B
    openk = (mask.float().numpy() != -np.inf)[:, : nr * V].reshape(B, nr, V).any(axis=2)
    if not causal:
        return int(openk.sum()) * Tq * H
    # runs 0 .. q // V lie before or at query q
    cum = np.concatenate([np.zeros((B, 1), np.int64), np.cumsum(openk, axis=1)], axis=1)
    lim = np.minimum(np.arange(Tq) // V + 1, nr)
    return int(cum[:, lim].sum()) * H


def softmax_skip_bytes(mask, causal, B, H, Tq, Tk, s) -> tuple[int, int]:
    """(fw, bw) bytes the skipping kernels move: the open runs read (once forward, y and dy
    backward), every output element written, and the mask once when given."""
    runs = softmax_open_runs(mask, causal, B, H, Tq, Tk, 16 // s)
    E = B * H * Tq * Tk
    mb = B * Tk * s if mask is not None else 0
    return runs * 16 + E * s + mb, 2 * runs * 16 + E * s + mb


def layernorm_fw_bytes(N, C, s) -> int:
    """Read x, write y, write fp32 mean and rstd, read gamma and beta."""
    return 2 * N * C * s + 8 * N + 2 * C * s


def rmsnorm_fw_bytes(N, C, s) -> int:
    """Read x, write y, write rstd (fp32), read gamma."""
    return 2 * N * C * s + 4 * N + C * s


def rmsnorm_bw_bytes(N, C, s) -> int:
    """Read x, dy, rstd (fp32) and gamma; write dx and dgamma."""
    return 3 * N * C * s + 4 * N + 2 * C * s


def layernorm_bw_bytes(N, C, s) -> int:
    """Read x, dy, gamma, mean, rstd; write dx, dgamma, dbeta."""
    return 3 * N * C * s + 8 * N + 3 * C * s


def attention_probability_traffic(B, H, T, s, layers, passes=2) -> int:
    """Bytes of the materialised [B,H,T,T] probability tensor per training step: the forward
    softmax writes it once and the backward reads it once, per layer."""
    return B * H * T * T * s * layers * passes
