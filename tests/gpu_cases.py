"""Row lengths the GPU edge-case tests run, one list per op family. The GPU tests parametrize
over these lists, and tests/test_plan_coverage_cpu.py checks on the CPU that, together with the
workload shapes, they reach every instantiation of the row-length dispatch."""

# LayerNorm and RMSNorm widths: bucket boundaries and their neighbours, odd widths (element-wise
# kernel), and a width in every bucket of the plan tables at both storage types.
NORM_EDGE_C = [1, 2, 8, 24, 64, 100, 128, 200, 264, 768, 1000, 1024, 1536, 2048, 2056, 4095,
               4096, 8191, 8192]

# Long launches (fp16, beyond 24576 rows, the row count from which a plan table may list
# row-count-dependent plans): ragged row counts (not whole row groups, a partial last band) at
# widths with idle lanes and at a bucket's full width.
NORM_LONG_F16 = [(24577, 1000), (24579, 1024), (24581, 4000)]

# Softmax row lengths: every bucket of the template list at fp16 and fp32, its neighbours,
# and odd lengths (element-wise kernel).
SOFTMAX_EDGE_TK = [1, 2, 8, 16, 24, 31, 32, 33, 40, 100, 200, 256, 264, 520, 1000, 2047, 2048]

# The read-skipping softmax: the same buckets, whole-vector lengths first.
SKIP_EDGE_TK = [8, 16, 24, 32, 40, 200, 256, 264, 520, 1000, 2048, 1, 31, 33, 100, 2047]

# Bias + dropout + residual feeding LayerNorm: (storage, width) pairs on its vector path, at
# least one in every backward bucket together with the workload widths.
BDR_EDGE = [("fp16", 8), ("fp16", 24), ("fp16", 128), ("fp16", 264), ("fp16", 1000),
            ("fp16", 1536), ("fp16", 2056), ("fp16", 8192),
            ("fp32", 4), ("fp32", 12), ("fp32", 100), ("fp32", 200), ("fp32", 500),
            ("fp32", 768), ("fp32", 1536), ("fp32", 4092)]
