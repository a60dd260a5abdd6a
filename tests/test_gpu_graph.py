"""Every entry point of the library inside a captured HIP graph.

The library allocates nothing, never synchronises and issues only kernel launches on the
caller's stream, so one call of each operation can be captured into a graph (torch's
CUDAGraph on a default-priority stream) and replayed. Checked here: three replays, each after
the outputs were overwritten with NaN by eager work and a synchronisation, reproduce the eager
results bit for bit (every kernel is deterministic); after the inputs are changed in place, a
replay reproduces the new eager results. Cross-entropy runs 64 rows, so its forward splits
rows over workgroups and its finish kernel reads the workspace inside the graph.
"""
import pytest
import torch

import layernorm_reduction_amd as lnr
from layernorm_reduction_amd import workloads as W
from parity_utils import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _d(t):
    return t.to(DEV)


def test_every_entry_point_replays_in_a_graph():
    sc = W.softmax_case("graph-softmax", 4, 4, 128, 128, causal=True, dtype=torch.float16,
                        seed_base=9990, len_range=(64, 128))
    lc = W.layernorm_case("graph-ln", 1000, 1024, dtype=torch.float16, seed_base=9991)
    # Rows of 280 KB: the forward splits them and combines the chunks in a second kernel.
    xc = W.xent_case("graph-xent", 4, 70001, dtype=torch.float32, seed_base=9992)
    bc = W.bdr_case("graph-bdr", 1000, 768, dtype=torch.float16, seed_base=9993)
    f16 = torch.float16

    sx, sm, sdy = _d(sc.x), _d(sc.mask), _d(sc.dy)
    lx, lg, lb, ldy = _d(lc.x), _d(lc.gamma), _d(lc.beta), _d(lc.dy)
    xz, xt, xdl = _d(xc.logits), _d(xc.target), _d(xc.dloss)
    bx, br, bb, bm = _d(bc.x), _d(bc.residual), _d(bc.bias), _d(bc.mask)
    bg, bbe, bdy, bde = _d(bc.gamma), _d(bc.beta), _d(bc.dy), _d(bc.ds_extra)
    N, C = lc.N, lc.C
    empty = lambda *shape, dtype=f16: torch.empty(*shape, dtype=dtype, device=DEV)
    o = {
        "sy": torch.empty_like(sx), "sdx": torch.empty_like(sx),
        "ky": torch.empty_like(sx), "kdx": torch.empty_like(sx),
        "ly": torch.empty_like(lx), "lm": empty(N, dtype=torch.float32), "lr": empty(N, dtype=torch.float32),
        "ldx": torch.empty_like(lx), "ldg": empty(C), "ldb": empty(C),
        "ry": torch.empty_like(lx), "rr": empty(N, dtype=torch.float32), "rdx": torch.empty_like(lx),
        "rdg": empty(C),
        "xl": empty(xc.N, dtype=torch.float32), "xs": empty(xc.N, dtype=torch.float32),
        "xdz": torch.empty_like(xz),
        "bs": torch.empty_like(bx), "by": torch.empty_like(bx), "bmu": empty(bc.N, dtype=torch.float32),
        "brs": empty(bc.N, dtype=torch.float32), "bdr": torch.empty_like(bx), "bdx": torch.empty_like(bx),
        "bdg": empty(bc.C), "bdb": empty(bc.C), "bdbi": empty(bc.C),
    }
    ws = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)
    lws = ws(lnr.layernorm_bw_workspace_bytes(N, C, f16))
    rws = ws(lnr.rmsnorm_bw_workspace_bytes(N, C, f16))
    xws = ws(lnr.cross_entropy_fw_workspace_bytes(xc.N, xc.V, torch.float32))
    bws = ws(lnr.bdr_layernorm_bw_workspace_bytes(bc.N, bc.C, f16))
    assert lnr.cross_entropy_fw_workspace_bytes(xc.N, xc.V, torch.float32) > 0

    def step():
        lnr.attn_softmax_fw(sx, sm, True, out=o["sy"])
        lnr.attn_softmax_bw(sdy, o["sy"], dinp=o["sdx"])
        lnr.attn_softmax_fw_skip(sx, sm, True, out=o["ky"])
        lnr.attn_softmax_bw_skip(sdy, o["ky"], sm, True, dinp=o["kdx"])
        lnr.layernorm_fw(lx, lg, lb, lc.eps, y=o["ly"], mean=o["lm"], rstd=o["lr"])
        lnr.layernorm_bw(ldy, lx, lg, o["lm"], o["lr"], dx=o["ldx"], dgamma=o["ldg"], dbeta=o["ldb"],
                         workspace=lws)
        lnr.rmsnorm_fw(lx, lg, W.RMS_EPS, y=o["ry"], rstd=o["rr"])
        lnr.rmsnorm_bw(ldy, lx, lg, o["rr"], dx=o["rdx"], dgamma=o["rdg"], workspace=rws)
        lnr.cross_entropy_fw(xz, xt, xc.ignore_index, loss=o["xl"], lse=o["xs"], workspace=xws)
        lnr.cross_entropy_bw(xz, xt, o["xs"], xdl, 0.5, xc.ignore_index, dlogits=o["xdz"])
        lnr.bdr_layernorm_fw(bx, br, bb, bm, bc.p, bg, bbe, bc.eps, s=o["bs"], y=o["by"],
                             mean=o["bmu"], rstd=o["brs"])
        lnr.bdr_layernorm_bw(bdy, o["bs"], bm, bc.p, bg, o["bmu"], o["brs"], bde, dresidual=o["bdr"],
                             dx=o["bdx"], dgamma=o["bdg"], dbeta=o["bdb"], dbias=o["bdbi"],
                             workspace=bws)

    def eager_reference():
        step()
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in o.items()}
        for k, v in ref.items():
            assert bool(torch.isfinite(v).all()), k
        return ref

    def replay_and_compare(g, ref, what):
        for rep in range(3):
            for v in o.values():
                v.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k, v in o.items():
                assert torch.equal(v, ref[k]), f"{what}, replay {rep}: {k} differs from the eager result"

    say("graph", "eager reference")
    ref1 = eager_reference()
    g = torch.cuda.CUDAGraph()
    say("graph", "capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    say("graph", "replays")
    replay_and_compare(g, ref1, "same inputs")

    say("graph", "new inputs in place")
    for t in (sx, sdy, lx, ldy, xz, bx, br, bdy, bde):
        t.mul_(0.75).add_(0.125)
    lg.mul_(1.25)
    ref2 = eager_reference()
    assert not torch.equal(ref2["sy"], ref1["sy"]) and not torch.equal(ref2["bdx"], ref1["bdx"])
    replay_and_compare(g, ref2, "changed inputs")
