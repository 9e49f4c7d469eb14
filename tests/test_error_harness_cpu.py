"""FLOP accounting of the error harness (CPU only): the FLOPs-matched static
rank k' is the largest multiple of 8 whose static flops stay within DyRA's,
correction overhead included (paperlayer.ai E.4: the baseline's rank is
raised until its exact FLOPs match DyRA's total)."""
import pytest

from input_adaptive_rank_amd import error_harness as H
from input_adaptive_rank_amd import synth


@pytest.mark.parametrize("name", ["tiny_fp32", "vitb_fc1", "vitl_fc1", "vitl_fc2"])
def test_flops_matched_rank_brackets_dyra_flops(name):
    w = synth.WORKLOADS[name]
    kp = H.flops_matched_rank(w.s, w.c1, w.c2, w.k, w.r)
    fd = H.dyra_flops_per_segment(w.s, w.c1, w.c2, w.k, w.r)
    assert kp % 8 == 0 and kp > w.k
    assert H.static_flops_per_segment(w.s, w.c1, w.c2, kp) <= fd < H.static_flops_per_segment(w.s, w.c1, w.c2, kp + 8)


def test_dyra_flops_count_each_term_once():
    """Term by term on a shape where each is easy to count by hand."""
    s, c1, c2, k, r = 10, 6, 4, 2, 1
    want = (2 * s * c1 * (k + r)       # [T | L] = X [U | P]
            + 2 * s * r * r            # G = L^T L
            + 2 * s * r * c1           # M = L^T X
            + 2 * r * c1 * c2          # R = M' W_res
            + r ** 3 / 3 + 2 * r * r * 4   # Cholesky and the solve against M (min(c1, c2) = 4)
            + 2 * s * (k + r) * c2)    # Y = [T | L] [V; R]
    assert H.dyra_flops_per_segment(s, c1, c2, k, r) == pytest.approx(want)
    assert H.static_flops_per_segment(s, c1, c2, 3) == 2 * 10 * 3 * 10
