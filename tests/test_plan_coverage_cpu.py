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


def softmax_buckets(dtype, backward, skip=False):
    return {lnr.softmax_plan(t, dtype, backward=backward, skip=skip)[0]
            for t in range(1, lnr.SOFTMAX_MAX_TK + 1)} - {0}


def norm_buckets(dtype, backward):
    return {lnr.layernorm_plan(64, c, dtype, backward=backward)[0]
            for c in range(1, lnr.LAYERNORM_MAX_C + 1)} - {0}


# Row counts at which a bucket's plan may change (a plan table may list plans taken only from
# some launch length on); every (bucket, lanes, vectors, workgroup) instantiation a launch can
# take.
PLAN_ROWS = (64, 16384, 24576, 32768, 65536)


def norm_plans(dtype, backward):
    return {lnr.layernorm_plan(n, c, dtype, backward=backward)[:4]
            for n in PLAN_ROWS for c in range(1, lnr.LAYERNORM_MAX_C + 1)} - {(0, 256, 0, 256)}


def reached_softmax(lengths, dtype, backward, skip=False):
    return {lnr.softmax_plan(t, dtype, backward=backward, skip=skip)[0] for t in lengths} - {0}


def reached_norm(cases, dtype, backward):
    """cases: (rows, width) pairs."""
    return {lnr.layernorm_plan(n, c, dtype, backward=backward)[:4] for n, c in cases} - {(0, 256, 0, 256)}


def test_plan_tables_have_the_template_buckets():
    tl = {32, 64, 128, 256, 384, 512, 768, 1024, 2048}
    for dt in (F16, F32):
        for bw in (False, True):
            assert softmax_buckets(dt, bw) == tl
            assert softmax_buckets(dt, bw, skip=True) == tl
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
            missing = softmax_buckets(dt, bw, skip=True) - reached_softmax(skip[dt], dt, bw, skip=True)
            assert not missing, ("skip", dt, bw, sorted(missing))


def test_norm_gpu_cases_reach_every_plan():
    # edge widths run at 1, 7 and 1031 rows
    edge = {(n, c) for c in gpu_cases.NORM_EDGE_C for n in (1, 7, 1031)}
    sweep = {(16384, c) for c in W.LAYERNORM_C_SWEEP}
    long16 = set(gpu_cases.NORM_LONG_F16)
    # LayerNorm: workloads 1 (fp32 [64,64]), 2 (fp16 [8192,256]), 4 (fp16 sweep), 5 (both,
    # [32768, 1024/4096])
    w5 = {(32768, 1024), (32768, 4096)}
    ln = {F16: edge | {(8192, 256)} | sweep | w5 | long16, F32: edge | {(64, 64)} | w5}
    # RMSNorm: the page's model shape [8192,256] (both), the sweep (fp16), [32768,1024] fp32
    rms = {F16: edge | {(8192, 256)} | sweep | long16, F32: edge | {(8192, 256), (32768, 1024)}}
    # bias + dropout + residual: [8192,256], [16384, 768/1024/4096] and the long [24581,4000]
    # fp16, [8192,1024] and [2048,8192] fp32, its edge widths at 1, 7 and 1031 rows
    bdr = {F16: {(8192, 256), (16384, 768), (16384, 1024), (16384, 4096), (24581, 4000)}
           | {(n, c) for d, c in gpu_cases.BDR_EDGE if d == "fp16" for n in (1, 7, 1031)},
           F32: {(8192, 1024), (2048, 8192)}
           | {(n, c) for d, c in gpu_cases.BDR_EDGE if d == "fp32" for n in (1, 7, 1031)}}
    for name, table in (("layernorm", ln), ("rmsnorm", rms), ("bdr", bdr)):
        for dt in (F16, F32):
            for bw in (False, True):
                if name == "bdr" and bw:
                    # its backward has a plan table of its own over the same buckets, with
                    # no long-launch plans: every bucket reached
                    got = {p[0] for p in reached_norm(table[dt], dt, bw)}
                    missing = norm_buckets(dt, bw) - got
                else:
                    missing = norm_plans(dt, bw) - reached_norm(table[dt], dt, bw)
                assert not missing, (name, dt, bw, sorted(missing))


def test_row_count_dependent_plans_are_reached_by_long_cases():
    """Where a bucket's forward or backward plan changes with the row count (between
    PLAN_ROWS), the GPU's long-launch cases reach the plan of the longest launches in that
    bucket."""
    for bw in (False, True):
        long_reached = reached_norm(gpu_cases.NORM_LONG_F16, F16, bw)
        for c in sorted(norm_buckets(F16, bw)):
            plans = [lnr.layernorm_plan(n, c, F16, backward=bw)[:4] for n in PLAN_ROWS[1:]]
            if len(set(plans)) > 1:
                assert plans[-1] in long_reached, (bw, c, plans)
    for n, _ in gpu_cases.NORM_LONG_F16:
        assert n > PLAN_ROWS[2], n


def test_bdr_edge_widths_take_its_vector_path():
    for d, c in gpu_cases.BDR_EDGE:
        assert (c * (2 if d == "fp16" else 4)) % 16 == 0, (d, c)
