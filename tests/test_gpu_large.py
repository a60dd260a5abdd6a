"""GPU parity on tensors beyond 4 GiB (through the C ABI): the softmax (dense and read-skipping),
LayerNorm, bias-dropout-residual LayerNorm and cross-entropy kernels address rows past 2^31
elements and past 2^32 bytes.

Inputs are drawn on the GPU with seeded device generators (workloads.device_normal /
device_uniform, in the storage dtype); the oracle runs on sampled rows read back from the
same stored values: rows on both sides of the 2^31-element (fp16) or 2^32-byte (fp32)
boundary, the batch boundary of the mask, the ragged last rows and seeded random rows. Each
backward takes seeded inputs of its own (y for the softmax backward, mean/rstd for LayerNorm,
lse for cross-entropy; the formulas are definitions for any such input), so no oracle input
comes from a GPU output. dgamma/dbeta (sums over every row) are checked on sampled columns.
"""
import numpy as np
import pytest
import torch

import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import assert_close, say, to_host64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SEED = 9700


def sample_rows(n_rows, boundaries, seed, n_random=8):
    """Rows 0, 1, each boundary row and its neighbours, the last two rows, and seeded random
    rows, sorted and unique."""
    rows = {0, 1, n_rows - 2, n_rows - 1}
    for b in boundaries:
        rows |= {b - 1, b, b + 1}
    g = torch.Generator().manual_seed(seed)
    rows |= set(torch.randint(0, n_rows, (n_random,), generator=g).tolist())
    return torch.tensor(sorted(r for r in rows if 0 <= r < n_rows), dtype=torch.int64)


def rows_of(t, idx, width):
    """Rows idx of t viewed as [-1, width], as a host float64 array."""
    return to_host64(t.reshape(-1, width).index_select(0, idx.to(t.device)))


@pytest.mark.parametrize("dtype,B,H,T,causal", [
    (torch.float16, 2, 260, 2048, True),    # 2.18e9 elements: past 2^31 elements and 2^32 bytes
    (torch.float32, 2, 132, 2048, False),   # 1.11e9 elements, 4.4 GB: past 2^32 bytes
])
def test_softmax_beyond_4gib(dtype, B, H, T, causal):
    rows, es = B * H * T, torch.finfo(dtype).bits // 8
    assert rows * T * es > 2 ** 32
    boundary = (2 ** 31 if es == 2 else 2 ** 30) // T        # first row at 2^31 elements / 2^32 bytes
    idx = sample_rows(rows, [boundary, H * T], SEED + es)
    say(f"softmax [{B},{H},{T},{T}] {dtype}", "draw on device")
    # scores ~N(0, 16): peaked rows, so a row read from the wrong place cannot pass the bound
    x = W.device_normal((B, H, T, T), SEED + 10 + es, dtype, DEV, std=4.0)
    lengths = W.valid_lengths(B, T // 2, T, SEED + 20 + es)
    mask = W.padding_mask(lengths, T, dtype)
    say("GPU forward")
    y = lnr.attn_softmax_fw(x, mask.to(DEV), causal)
    torch.cuda.synchronize()
    x_rows = rows_of(x, idx, T)
    y_rows = rows_of(y, idx, T)
    del x, y
    m_rows = mask.double().numpy()[(idx // (H * T)).numpy()]
    say("oracle forward on", idx.numel(), "rows")
    ref = oracle.softmax_fw_rows(x_rows, m_rows, (idx % T).numpy(), causal)
    assert_close(y_rows, ref, dtype, f"softmax fw beyond 4 GiB {dtype}")

    say("GPU backward")
    # y ~U[0, 1) (the backward's formula holds for any y): gradients of order 10, far above atol
    yb = W.device_uniform((B, H, T, T), SEED + 30 + es, 0.0, 1.0, dtype, DEV)
    dy = W.device_normal((B, H, T, T), SEED + 40 + es, dtype, DEV)
    dx = lnr.attn_softmax_bw(dy, yb)
    torch.cuda.synchronize()
    yb_rows, dy_rows, dx_rows = rows_of(yb, idx, T), rows_of(dy, idx, T), rows_of(dx, idx, T)
    del yb, dy, dx
    torch.cuda.empty_cache()
    assert_close(dx_rows, oracle.softmax_bw(yb_rows, dy_rows), dtype, f"softmax bw beyond 4 GiB {dtype}")


def test_layernorm_beyond_2_31_elements():
    dtype, N, C = torch.float16, 262147, 8192                 # 2^31 elements end at row 262144
    assert N * C > 2 ** 31
    idx = sample_rows(N, [2 ** 31 // C, N // 2], SEED + 50)
    say(f"layernorm [{N},{C}]", "draw on device")
    x = W.device_normal((N, C), SEED + 51, dtype, DEV)
    x.add_(W.device_normal((N, 1), SEED + 52, dtype, DEV, std=2.0))   # distinct row means
    gamma = W.uniform((C,), SEED + 53, 0.5, 1.5).to(dtype)
    beta = W.normal((C,), SEED + 54, var=0.1).to(dtype)
    g64, b64 = gamma.double().numpy(), beta.double().numpy()
    say("GPU forward")
    y, mean, rstd = lnr.layernorm_fw(x, gamma.to(DEV), beta.to(DEV), W.LN_EPS)
    torch.cuda.synchronize()
    x_rows = rows_of(x, idx, C)
    y_ref, mean_ref, rstd_ref = oracle.layernorm_fw(x_rows, g64, b64, W.LN_EPS)
    assert_close(rows_of(y, idx, C), y_ref, dtype, "layernorm y beyond 2^31")
    assert_close(to_host64(mean[idx.to(DEV)]), mean_ref, dtype, "layernorm mean beyond 2^31")
    assert_close(to_host64(rstd[idx.to(DEV)]), rstd_ref, dtype, "layernorm rstd beyond 2^31")
    del y, mean, rstd

    say("GPU backward on seeded statistics")
    ms = W.device_normal((N,), SEED + 55, torch.float32, DEV, std=2.0)
    rs = W.device_uniform((N,), SEED + 56, 0.5, 1.5, torch.float32, DEV)
    dy = W.device_normal((N, C), SEED + 57, dtype, DEV)
    dx, dg, db = lnr.layernorm_bw(dy, x, gamma.to(DEV), ms, rs)
    torch.cuda.synchronize()
    ms64, rs64 = to_host64(ms), to_host64(rs)
    dx_ref, _, _ = oracle.layernorm_bw_given_stats(x_rows, rows_of(dy, idx, C), g64,
                                                   ms64[idx.numpy()], rs64[idx.numpy()])
    assert_close(rows_of(dx, idx, C), dx_ref, dtype, "layernorm dx beyond 2^31")
    # column sums over all rows, on sampled columns: the oracle's dgamma/dbeta of the [N, k]
    # problem made of those columns are the same column sums
    cols = torch.tensor([0, 1, 4095, 4096, 8190, 8191, 1234, 5678], dtype=torch.int64)
    xc = to_host64(x.index_select(1, cols.to(DEV)))
    dyc = to_host64(dy.index_select(1, cols.to(DEV)))
    del x, dy, dx
    torch.cuda.empty_cache()
    _, dg_ref, db_ref = oracle.layernorm_bw_given_stats(xc, dyc, g64[cols.numpy()], ms64, rs64)
    assert_close(to_host64(dg)[cols.numpy()], dg_ref, dtype, "layernorm dgamma beyond 2^31")
    assert_close(to_host64(db)[cols.numpy()], db_ref, dtype, "layernorm dbeta beyond 2^31")


def test_cross_entropy_beyond_2_31_elements():
    dtype, N, V = torch.float16, 32771, 65536                 # 2^31 elements end at row 32768
    assert N * V > 2 ** 31
    idx = sample_rows(N, [2 ** 31 // V], SEED + 60)
    say(f"cross-entropy [{N},{V}]", "draw on device")
    z = W.device_normal((N, V), SEED + 61, dtype, DEV)
    t = torch.randint(0, V, (N,), generator=torch.Generator().manual_seed(SEED + 62), dtype=torch.int64)
    td = t.to(DEV)
    say("GPU forward")
    loss, lse = lnr.cross_entropy_fw(z, td)
    torch.cuda.synchronize()
    z_rows, t_rows = rows_of(z, idx, V), t[idx].numpy()
    loss_ref, lse_ref = oracle.xent_fw(z_rows, t_rows)
    assert_close(to_host64(loss[idx.to(DEV)]), loss_ref, torch.float32, "xent loss beyond 2^31",
                 atol=1e-5, rtol=1e-5)
    assert_close(to_host64(lse[idx.to(DEV)]), lse_ref, torch.float32, "xent lse beyond 2^31",
                 atol=1e-5, rtol=1e-5)

    say("GPU backward on a seeded lse")
    ls = W.device_uniform((N,), SEED + 63, 11.0, 12.0, torch.float32, DEV)
    dl = W.device_normal((N,), SEED + 64, torch.float32, DEV)
    dz = lnr.cross_entropy_bw(z, td, ls, dl, 1.0)
    torch.cuda.synchronize()
    ref = oracle.xent_bw_given_lse(z_rows, t_rows, to_host64(ls)[idx.numpy()], to_host64(dl)[idx.numpy()])
    assert_close(rows_of(dz, idx, V), ref, dtype, "xent dz beyond 2^31")
    del z, dz
    torch.cuda.empty_cache()


def test_softmax_skip_beyond_4gib():
    """The read-skipping forward and backward on the fp16 causal, padded case past 2^31
    elements. The backward's y is zero wherever the forward's would be (masked keys and
    future positions), the condition under which it equals the dense backward."""
    dtype, B, H, T = torch.float16, 2, 260, 2048
    rows = B * H * T
    idx = sample_rows(rows, [2 ** 31 // T, H * T], SEED + 70)
    say(f"skip softmax [{B},{H},{T},{T}]", "draw on device")
    x = W.device_normal((B, H, T, T), SEED + 71, dtype, DEV, std=4.0)
    lengths = W.valid_lengths(B, T // 2, T, SEED + 72)
    mask = W.padding_mask(lengths, T, dtype)
    y = lnr.attn_softmax_fw_skip(x, mask.to(DEV), True)
    torch.cuda.synchronize()
    x_rows, y_rows = rows_of(x, idx, T), rows_of(y, idx, T)
    del x, y
    m_rows = mask.double().numpy()[(idx // (H * T)).numpy()]
    ref = oracle.softmax_fw_rows(x_rows, m_rows, (idx % T).numpy(), True)
    assert_close(y_rows, ref, dtype, "skip softmax fw beyond 4 GiB")

    say("GPU backward (skipping)")
    yb = W.device_uniform((B, H, T, T), SEED + 73, 0.0, 1.0, dtype, DEV)
    j = torch.arange(T, device=DEV)
    yb.masked_fill_(j.view(1, 1, 1, T) >= lengths.to(DEV).view(B, 1, 1, 1), 0.0)
    yb.masked_fill_(j.view(1, 1, 1, T) > j.view(1, 1, T, 1), 0.0)
    dy = W.device_normal((B, H, T, T), SEED + 74, dtype, DEV)
    dx = lnr.attn_softmax_bw_skip(dy, yb, mask.to(DEV), True)
    torch.cuda.synchronize()
    yb_rows, dy_rows, dx_rows = rows_of(yb, idx, T), rows_of(dy, idx, T), rows_of(dx, idx, T)
    del yb, dy, dx
    torch.cuda.empty_cache()
    assert_close(dx_rows, oracle.softmax_bw(yb_rows, dy_rows), dtype, "skip softmax bw beyond 4 GiB")


def test_bdr_layernorm_beyond_2_31_elements():
    """Bias + dropout + residual LayerNorm past 2^31 elements: forward and backward rows, and
    dgamma/dbeta on sampled columns (dbias, whose rows need full-row sums, is covered at the
    smaller sizes of the bias-dropout-residual tests)."""
    dtype, N, C, p = torch.float16, 262147, 8192, 0.1
    idx = sample_rows(N, [2 ** 31 // C, N // 2], SEED + 80)
    say(f"bdr layernorm [{N},{C}]", "draw on device")
    x = W.device_normal((N, C), SEED + 81, dtype, DEV)
    r = W.device_normal((N, C), SEED + 82, dtype, DEV)
    keep = W.device_bytes((N, C // 8), SEED + 83, DEV)
    bias = W.normal((C,), SEED + 84, var=0.1).to(dtype)
    gamma = W.uniform((C,), SEED + 85, 0.5, 1.5).to(dtype)
    beta = W.normal((C,), SEED + 86, var=0.1).to(dtype)
    g64 = gamma.double().numpy()
    s, y, mean, rstd = lnr.bdr_layernorm_fw(x, r, bias.to(DEV), keep, p, gamma.to(DEV), beta.to(DEV), W.LN_EPS)
    torch.cuda.synchronize()
    k_rows = keep.index_select(0, idx.to(DEV)).cpu().numpy()
    s_ref, y_ref, mean_ref, rstd_ref = oracle.bdr_ln_fw(rows_of(x, idx, C), rows_of(r, idx, C),
                                                        bias.double().numpy(), k_rows, p, g64,
                                                        beta.double().numpy(), W.LN_EPS)
    assert_close(rows_of(s, idx, C), s_ref, dtype, "bdr s beyond 2^31")
    assert_close(rows_of(y, idx, C), y_ref, dtype, "bdr y beyond 2^31")
    assert_close(to_host64(mean[idx.to(DEV)]), mean_ref, dtype, "bdr mean beyond 2^31")
    assert_close(to_host64(rstd[idx.to(DEV)]), rstd_ref, dtype, "bdr rstd beyond 2^31")
    del x, r, s, y, mean, rstd

    say("GPU backward on a seeded s and statistics")
    sb = W.device_normal((N, C), SEED + 87, dtype, DEV)
    ms = W.device_normal((N,), SEED + 88, torch.float32, DEV, std=0.5)
    rs = W.device_uniform((N,), SEED + 89, 0.5, 1.5, torch.float32, DEV)
    dy = W.device_normal((N, C), SEED + 90, dtype, DEV)
    dres, dx, dg, db, _ = lnr.bdr_layernorm_bw(dy, sb, keep, p, gamma.to(DEV), ms, rs)
    torch.cuda.synchronize()
    ms64, rs64 = to_host64(ms), to_host64(rs)
    dres_ref, dx_ref, _, _, _ = oracle.bdr_ln_bw(rows_of(sb, idx, C), rows_of(dy, idx, C), None, k_rows, p,
                                                 g64, ms64[idx.numpy()], rs64[idx.numpy()])
    assert_close(rows_of(dres, idx, C), dres_ref, dtype, "bdr dresidual beyond 2^31")
    assert_close(rows_of(dx, idx, C), dx_ref, dtype, "bdr dx beyond 2^31")
    cols = torch.tensor([0, 1, 4095, 4096, 8190, 8191, 1234, 5678], dtype=torch.int64)
    sc = to_host64(sb.index_select(1, cols.to(DEV)))
    dyc = to_host64(dy.index_select(1, cols.to(DEV)))
    del sb, dy, dres, dx, keep
    torch.cuda.empty_cache()
    ones = np.full((N, 1), 0xFF, np.uint8)     # dgamma and dbeta do not depend on the keep bits
    _, _, dg_ref, db_ref, _ = oracle.bdr_ln_bw(sc, dyc, None, ones, p, g64[cols.numpy()], ms64, rs64)
    assert_close(to_host64(dg)[cols.numpy()], dg_ref, dtype, "bdr dgamma beyond 2^31")
    assert_close(to_host64(db)[cols.numpy()], db_ref, dtype, "bdr dbeta beyond 2^31")
