"""Every compiled instantiation of the row-length dispatch is reached by at least one GPU
parity case (no GPU needed: the plan queries touch no device).

The dispatch picks the smallest bucket of the HW4 page's template list at or above the row
length (LayerNorm: the same list up to 8192 columns); every bucket is a template instantiation
of its own. The row lengths the GPU tests run are the workload shapes (workloads.py) plus the
edge-case lists in gpu_cases.py."""
import gpu_cases
import layernorm_reduction_amd as lnr
from layernorm_reduction_amd import workloads as W

F32, F16 = lnr.LNR_F32, lnr.LNR_F16
ES = {F32: 4, F16: 2}


def softmax_buckets(dtype, backward):
    return {lnr.softmax_plan(t, dtype, backward=backward)[0] for t in range(1, lnr.SOFTMAX_MAX_TK + 1)} - {0}


def norm_buckets(dtype, backward):
    return {lnr.layernorm_plan(64, c, dtype, backward=backward)[0]
            for c in range(1, lnr.LAYERNORM_MAX_C + 1)} - {0}


def reached_softmax(lengths, dtype, backward):
    return {lnr.softmax_plan(t, dtype, backward=backward)[0] for t in lengths} - {0}


def reached_norm(widths, dtype, backward):
    return {lnr.layernorm_plan(64, c, dtype, backward=backward)[0] for c in widths} - {0}


def test_plan_tables_have_the_template_buckets():
    tl = {32, 64, 128, 256, 384, 512, 768, 1024, 2048}
    for dt in (F16, F32):
        for bw in (False, True):
            assert softmax_buckets(dt, bw) == tl
            assert norm_buckets(dt, bw) == {64, 128, 256, 512, 768, 1024, 2048, 4096, 8192}


def test_softmax_gpu_cases_reach_every_bucket():
    # dense: workload 1 (fp32, Tk 16), 2 (fp16, 256), 3 (fp16, the sweep), 5 (both, 512)
    lengths = {F16: set(gpu_cases.SOFTMAX_EDGE_TK) | {256, 512} | set(W.SOFTMAX_TK_SWEEP),
               F32: set(gpu_cases.SOFTMAX_EDGE_TK) | {16, 512}}
    skip = {F16: set(gpu_cases.SKIP_EDGE_TK) | {256, 512} | set(W.SOFTMAX_TK_SWEEP),
            F32: set(gpu_cases.SKIP_EDGE_TK) | {16, 512}}
    for dt in (F16, F32):
        for bw in (False, True):
            missing = softmax_buckets(dt, bw) - reached_softmax(lengths[dt], dt, bw)
            assert not missing, ("dense", dt, bw, sorted(missing))
            missing = softmax_buckets(dt, bw) - reached_softmax(skip[dt], dt, bw)
            assert not missing, ("skip", dt, bw, sorted(missing))


def test_norm_gpu_cases_reach_every_bucket():
    edge = set(gpu_cases.NORM_EDGE_C)
    # LayerNorm: workloads 1 (fp32, 64), 2 (fp16, 256), 4 (fp16 sweep), 5 (both, 1024, 4096)
    ln = {F16: edge | {256, 1024, 4096} | set(W.LAYERNORM_C_SWEEP), F32: edge | {64, 1024, 4096}}
    # RMSNorm: the page's model shape (256, both), the sweep (fp16), [32768, 1024] fp32
    rms = {F16: edge | {256} | set(W.LAYERNORM_C_SWEEP), F32: edge | {256, 1024}}
    # bias + dropout + residual: [8192, 256] and [16384, 768/1024/4096] fp16, 1024/8192 fp32
    bdr = {F16: {256, 768, 1024, 4096} | {c for d, c in gpu_cases.BDR_EDGE if d == "fp16"},
           F32: {1024, 8192} | {c for d, c in gpu_cases.BDR_EDGE if d == "fp32"}}
    for name, table in (("layernorm", ln), ("rmsnorm", rms), ("bdr", bdr)):
        for dt in (F16, F32):
            for bw in (False, True):
                missing = norm_buckets(dt, bw) - reached_norm(table[dt], dt, bw)
                assert not missing, (name, dt, bw, sorted(missing))


def test_bdr_edge_widths_take_its_vector_path():
    for d, c in gpu_cases.BDR_EDGE:
        assert (c * (2 if d == "fp16" else 4)) % 16 == 0, (d, c)
