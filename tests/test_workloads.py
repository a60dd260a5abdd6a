"""Seeded generators: reproducible bits, the stated shapes, and masks that match the lengths."""
import math

import torch

from layernorm_reduction_amd import workloads as W


def test_generators_are_bit_reproducible():
    a, _ = W.workload1()
    b, _ = W.workload1()
    assert torch.equal(a[0].x, b[0].x) and torch.equal(a[0].dy, b[0].dy)
    assert torch.equal(a[0].mask, b[0].mask)


def test_workload1_mask_matches_lengths_and_dtypes():
    [s], [ln] = W.workload1()
    assert s.x.dtype == torch.float32 and ln.x.dtype == torch.float32
    assert s.lengths.min() >= 8 and s.lengths.max() <= 16
    for b, L in enumerate(s.lengths.tolist()):
        assert torch.all(s.mask[b, :L] == 0) and torch.all(torch.isinf(s.mask[b, L:]))
    assert ln.gamma.min() >= 0.5 and ln.gamma.max() <= 1.5


def test_workload3_batches_give_about_2_pow_27_elements():
    for Tk in W.SOFTMAX_TK_SWEEP:
        B = W.workload3_batch(Tk)
        E = B * 8 * Tk * Tk
        assert abs(E - 2 ** 27) / 2 ** 27 < 0.02, (Tk, B)


def test_distinct_tensors_use_distinct_seeds():
    seeds = {W.seed_of(w, k, v) for w in range(1, 6) for v in range(9) for k in range(8)}
    assert len(seeds) == 5 * 9 * 8


def test_row_offset_reading_is_variance():
    off = W.normal((200000, 1), 123, var=4.0)
    assert abs(off.std().item() - 2.0) < 0.02


def test_byte_formulas():
    s = 2
    assert W.layernorm_fw_bytes(8192, 256, s) == 2 * 8192 * 256 * s + 8 * 8192 + 2 * 256 * s
    assert W.layernorm_bw_bytes(8192, 256, s) == 3 * 8192 * 256 * s + 8 * 8192 + 3 * 256 * s
    assert W.softmax_fw_bytes(64, 16, 512, 512, s) == 2 * 64 * 16 * 512 * 512 * s + 64 * 512 * s
    assert math.isclose(W.softmax_bw_bytes(32, 8, 256, 256, 2) / 1e6, 100.663296)


def test_softmax_open_runs_counts_like_brute_force():
    """The skipping kernels' byte count: runs of V keys with at least one key that is neither
    after the query (causal) nor under a -inf mask entry, counted one by one on small cases."""
    import numpy as np

    def brute(mask, causal, B, H, Tq, Tk, V):
        n = 0
        for b in range(B):
            for q in range(Tq):
                for r in range(Tk // V):
                    n += any((not causal or k <= q) and (mask is None or mask[b, k] != -np.inf)
                             for k in range(r * V, r * V + V))
        return n * H

    for causal in (False, True):
        for Tk, V in ((64, 8), (48, 4), (72, 8)):
            B, H = 3, 2
            m = torch.zeros(B, Tk)
            m[0, 20:] = -float("inf")
            m[2, :] = -float("inf")
            m[1, 5] = -float("inf")
            assert W.softmax_open_runs(m, causal, B, H, Tk, Tk, V) == brute(m.numpy(), causal, B, H, Tk, Tk, V)
            assert W.softmax_open_runs(None, causal, B, H, Tk, Tk, V) == brute(None, causal, B, H, Tk, Tk, V)
    fw, bw = W.softmax_skip_bytes(None, False, 2, 3, 16, 64, 2)
    assert fw == W.softmax_fw_bytes(2, 3, 16, 64, 2, has_mask=False)     # nothing to skip
    assert bw == W.softmax_bw_bytes(2, 3, 16, 64, 2)
