"""GPU parity of bdr_layernorm_fw / bdr_layernorm_bw (bias + dropout + residual feeding
LayerNorm) through the C ABI against the fp64 oracle.

  * forward: s, y, mean and rstd on seeded inputs, every element (s is formed and normalised
    in fp32; the stored s is rounded to the storage type);
  * backward on identical inputs: both sides receive the oracle's s rounded to the storage
    type, that s's statistics rounded to fp32, the same mask, dy and ds_extra; compared
    element by element at the plain bound (near-constant rows of the edge-case tests may add
    the LayerNorm dx formula's rounding term; parity_utils.assert_grad_close prints how many
    elements needed it);
  * chained: GPU forward outputs feeding the GPU backward against the oracle's gradient of the
    pipeline as stored: the oracle's s rounded to the storage type with the statistics of the
    exact s (what the forward saves). Against fully exact fp64 math the column sums cannot
    agree at fp16: each stored s carries ~2^-11 relative rounding, and dgamma = sum over 8192
    rows of dy * shat accumulates it to a few percent. dgamma is compared norm-wise (max |err|
    <= atol + rtol * max |ref|): the kernel forms s in fp32 and rounds that to fp16, so where
    the exact s lies within fp32 roundoff of an fp16 rounding midpoint (about 1 element in
    2000) the stored s is the neighbouring fp16 value; at |s| ~ 4-8 one such step moves
    dgamma_j by dy * 2^-8 * rstd ~ 4e-3. dbeta and dbias do not depend on s and stay
    element-wise; the element-wise dgamma check is the identical-input one above.
"""
import numpy as np
import pytest
import torch

import gpu_cases
import layernorm_reduction_amd as lnr
import oracle
from layernorm_reduction_amd import workloads as W
from parity_utils import TOL, assert_close, assert_grad_close, say, to_host64, violations

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
def gmax_of(dy64, g64):
    """Per row, max_j |gamma_j * dy_ij|: the largest term the LayerNorm dx formula subtracts."""
    return np.max(np.abs(dy64 * g64.reshape(1, -1)), axis=1)


def on_device(t, shift=False):
    """t on the GPU; with shift, at an address one element past a 16-byte boundary (the
    element-wise kernels)."""
    if not shift:
        return t.to(DEV)
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
    buf[1:].copy_(t.reshape(-1).to(DEV))
    return buf[1:].view(t.shape)


def run_bdr(case, extra=True, chain=True, edge=False, shift=False):
    dt = case.dtype
    atol, rtol = TOL[dt]
    m = case.mask.numpy()
    say(case.name, "oracle forward")
    x64, r64, b64 = (t.double().numpy() for t in (case.x, case.residual, case.bias))
    g64, be64 = case.gamma.double().numpy(), case.beta.double().numpy()
    s_ref, y_ref, mean_ref, rstd_ref = oracle.bdr_ln_fw(x64, r64, b64, m, case.p, g64, be64, case.eps)

    say(case.name, "GPU forward")
    xd, rd, bd = (on_device(t, shift) for t in (case.x, case.residual, case.bias))
    gd, bed, md = on_device(case.gamma, shift), on_device(case.beta, shift), case.mask.to(DEV)
    s, y, mean, rstd = lnr.bdr_layernorm_fw(xd, rd, bd, md, case.p, gd, bed, case.eps,
                                            s=on_device(case.x, shift), y=on_device(case.x, shift))
    torch.cuda.synchronize()
    assert_close(s, s_ref, dt, f"{case.name} s")
    assert_close(y, y_ref, dt, f"{case.name} y")
    assert_close(mean, mean_ref, dt, f"{case.name} mean")
    assert_close(rstd, rstd_ref, dt, f"{case.name} rstd")

    say(case.name, "oracle backward (identical inputs)")
    s_in = torch.from_numpy(s_ref).to(dt)                  # the stored s
    s_in64 = s_in.double().numpy()
    _, mu_in, rs_in = oracle.layernorm_fw(s_in64, g64, be64, case.eps)
    mu32 = torch.from_numpy(mu_in).float()
    rs32 = torch.from_numpy(rs_in).float()
    dy64 = case.dy.double().numpy()
    de64 = case.ds_extra.double().numpy() if extra else None
    refs = oracle.bdr_ln_bw(s_in64, dy64, de64, m, case.p, g64, mu32.numpy(), rs32.numpy())
    say(case.name, "GPU backward")
    dyd = on_device(case.dy, shift)
    ded = on_device(case.ds_extra, shift) if extra else None
    got = lnr.bdr_layernorm_bw(dyd, on_device(s_in, shift), md, case.p, gd, mu32.to(DEV), rs32.to(DEV), ded,
                               dresidual=on_device(case.dy, shift), dx=on_device(case.dy, shift))
    torch.cuda.synchronize()
    inv_keep = 1.0 / (1.0 - case.p)
    r32 = rs32.double().numpy()
    gm = gmax_of(dy64, g64)
    assert_grad_close(got[0], refs[0], dt, f"{case.name} dresidual", r32, gm, allow_near_constant=edge)
    assert_grad_close(got[1], refs[1], dt, f"{case.name} dx", r32, gm, allow_near_constant=edge,
                      factor=inv_keep)
    assert_close(got[2], refs[2], dt, f"{case.name} dgamma")
    assert_close(got[3], refs[3], dt, f"{case.name} dbeta")
    assert_close(got[4], refs[4], dt, f"{case.name} dbias")

    if chain:
        say(case.name, "chained fw -> bw against the stored-s gradient")
        ex = oracle.bdr_ln_bw(s_in64, dy64, de64, m, case.p, g64, mean_ref, rstd_ref)
        ch = lnr.bdr_layernorm_bw(dyd, s, md, case.p, gd, mean, rstd, ded)
        torch.cuda.synchronize()
        assert_grad_close(ch[0], ex[0], dt, f"{case.name} chain dresidual", rstd_ref, gm,
                          allow_near_constant=edge)
        assert_grad_close(ch[1], ex[1], dt, f"{case.name} chain dx", rstd_ref, gm,
                          allow_near_constant=edge, factor=inv_keep)
        got = to_host64(ch[2])
        bad, _ = violations(got, ex[2], atol, rtol)
        print(f"[info] {case.name} chained dgamma element-wise: {case.C - bad}/{case.C} within "
              f"atol=rtol={atol}", flush=True)
        err = float(np.max(np.abs(got - ex[2])))
        assert err <= atol + rtol * float(np.max(np.abs(ex[2]))), err
        for k, nm in ((3, "dbeta"), (4, "dbias")):
            assert_close(ch[k], ex[k], dt, f"{case.name} chain {nm}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("extra", [False, True])
def test_gpt2_shape(extra):
    run_bdr(W.bdr_case("bdr-8192x256-f16", 8192, 256, dtype=torch.float16, seed_base=9000), extra)


@pytest.mark.parametrize("C", [768, 1024, 4096])
def test_hidden_sizes_fp16(C):
    run_bdr(W.bdr_case(f"bdr-16384x{C}-f16", 16384, C, dtype=torch.float16, seed_base=9100 + C))


def test_long_ragged_launch():
    """A long launch (beyond 24576 rows, where the forward's plan at 4096 fp16 columns changes)
    with a ragged row count, at a width with idle lanes."""
    run_bdr(W.bdr_case("bdr-long-24581x4000-f16", 24581, 4000, dtype=torch.float16, seed_base=9600),
            chain=False)


@pytest.mark.parametrize("C", [1024, 8192])
def test_fp32(C):
    # C = 8192 fp32 is the plan whose backward spills part of its fp64 partials to scratch
    N = 8192 if C == 1024 else 2048
    run_bdr(W.bdr_case(f"bdr-{N}x{C}-f32", N, C, dtype=torch.float32, seed_base=9200 + C),
            chain=(C == 1024))


@pytest.mark.parametrize("p", [0.0, 0.5])
@pytest.mark.parametrize("dtype,C", [(torch.float16 if d == "fp16" else torch.float32, c)
                                     for d, c in gpu_cases.BDR_EDGE])
def test_edges(dtype, C, p):
    for N in (1, 7, 1031):
        run_bdr(W.bdr_case(f"bdr-edge-{N}x{C}-{dtype}-p{p}", N, C, dtype=dtype,
                           seed_base=9300 + C, p=p), extra=(N != 7), chain=False, edge=True)


def test_p_zero_equals_layernorm_of_the_sum():
    case = W.bdr_case("bdr-p0", 1000, 1024, dtype=torch.float32, seed_base=9400, p=0.0)
    xd, rd, bd = case.x.to(DEV), case.residual.to(DEV), case.bias.to(DEV)
    gd, bed = case.gamma.to(DEV), case.beta.to(DEV)
    say(case.name)
    s, y, _, _ = lnr.bdr_layernorm_fw(xd, rd, bd, case.mask.to(DEV), 0.0, gd, bed, case.eps)
    y2, _, _ = lnr.layernorm_fw(s, gd, bed, case.eps)
    torch.cuda.synchronize()
    assert torch.all(case.keep)
    assert_close(y, to_host64(y2), torch.float32, "bdr(p=0) vs layernorm(s)")


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_in_place_and_determinism(dtype):
    case = W.bdr_case("bdr-inplace", 3000, 1024, dtype=dtype, seed_base=9500)
    xd, rd, bd = case.x.to(DEV), case.residual.to(DEV), case.bias.to(DEV)
    gd, bed, md = case.gamma.to(DEV), case.beta.to(DEV), case.mask.to(DEV)
    say(case.name, dtype)
    s1, y1, m1, r1 = lnr.bdr_layernorm_fw(xd, rd, bd, md, case.p, gd, bed)
    ri = rd.clone()
    si, yi, _, _ = lnr.bdr_layernorm_fw(xd, ri, bd, md, case.p, gd, bed, s=ri)   # s over residual
    dyd, ded = case.dy.to(DEV), case.ds_extra.to(DEV)
    a = lnr.bdr_layernorm_bw(dyd, s1, md, case.p, gd, m1, r1, ded)
    b = lnr.bdr_layernorm_bw(dyd, s1, md, case.p, gd, m1, r1, ded)
    dyi = dyd.clone()
    c = lnr.bdr_layernorm_bw(dyi, s1, md, case.p, gd, m1, r1, ded, dresidual=dyi)  # over dy
    torch.cuda.synchronize()
    assert torch.equal(s1, ri) and torch.equal(y1, yi)
    for u, v, w in zip(a, b, c):
        assert torch.equal(u, v) and torch.equal(u, w)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("C", [1, 7, 100, 1000])
def test_element_wise_fallback(C, dtype):
    """Widths whose rows are not whole 16-byte vectors, and buffers one element past a 16-byte
    boundary, take the element-wise kernels: parity with the oracle, forward and backward,
    with and without the second gradient of s. No chained comparison at C = 1: a one-element
    row has variance 0, so rstd = 1/sqrt(eps) = 1e4 multiplies the storage rounding of s,
    which the chained reference pairs with the exact statistics, by 1e4."""
    for N in (7, 1031):
        for shift in (False, True):
            case = W.bdr_case(f"bdr-generic-{N}x{C}-{dtype}-{'unaligned' if shift else 'aligned'}", N, C,
                              dtype=dtype, seed_base=9900 + C)
            run_bdr(case, extra=(N == 1031), chain=(N == 1031 and C > 1), edge=True, shift=shift)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_element_wise_fallback_in_place(dtype):
    """s over residual and dresidual over dy on the element-wise kernels (C = 100): bitwise
    equal to the out-of-place results."""
    case = W.bdr_case("bdr-generic-inplace", 513, 100, dtype=dtype, seed_base=9950)
    xd, rd, bd = case.x.to(DEV), case.residual.to(DEV), case.bias.to(DEV)
    gd, bed, md = case.gamma.to(DEV), case.beta.to(DEV), case.mask.to(DEV)
    say(case.name, dtype)
    s1, y1, m1, r1 = lnr.bdr_layernorm_fw(xd, rd, bd, md, case.p, gd, bed)
    ri = rd.clone()
    si, yi, mi, rri = lnr.bdr_layernorm_fw(xd, ri, bd, md, case.p, gd, bed, s=ri)
    dyd, ded = case.dy.to(DEV), case.ds_extra.to(DEV)
    a = lnr.bdr_layernorm_bw(dyd, s1, md, case.p, gd, m1, r1, ded)
    dyi = dyd.clone()
    c = lnr.bdr_layernorm_bw(dyi, s1, md, case.p, gd, m1, r1, ded, dresidual=dyi)
    dei = ded.clone()
    d = lnr.bdr_layernorm_bw(dyd, s1, md, case.p, gd, m1, r1, dei, dresidual=dei)
    torch.cuda.synchronize()
    assert torch.equal(s1, ri) and torch.equal(y1, yi) and torch.equal(m1, mi) and torch.equal(r1, rri)
    for u, v, w in zip(a, c, d):
        assert torch.equal(u, v) and torch.equal(u, w)


def test_invalid_p_is_rejected():
    N, C = 16, 64
    z = torch.zeros(N, C, dtype=torch.float16, device=DEV)
    c = torch.zeros(C, dtype=torch.float16, device=DEV)
    mk = torch.zeros(N, C // 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(lnr.LnrError) as e:
        lnr.bdr_layernorm_fw(z, z.clone(), c, mk, 1.0, c, c)   # p must be < 1
    assert e.value.status == 2


def test_zero_rows_give_zero_parameter_gradients():
    C = 512
    s = torch.empty(0, C, dtype=torch.float16, device=DEV)
    g = torch.ones(C, dtype=torch.float16, device=DEV)
    st = torch.empty(0, dtype=torch.float32, device=DEV)
    mk = torch.empty(0, C // 8, dtype=torch.uint8, device=DEV)
    outs = [torch.full((C,), 7.0, dtype=torch.float16, device=DEV) for _ in range(3)]
    say("N=0 bdr backward")
    lnr.bdr_layernorm_bw(s, s, mk, 0.1, g, st, st, None, dgamma=outs[0], dbeta=outs[1], dbias=outs[2])
    torch.cuda.synchronize()
    for o in outs:
        assert torch.all(o == 0)
