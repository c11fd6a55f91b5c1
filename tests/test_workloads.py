"""Host-side accounting of the workloads: the visible-pair counts behind the
FLOP figures the benchmark reports, checked against a brute-force count of
the mask (no GPU)."""
import numpy as np
import pytest

from flashattention_attention_amd import inputs


def _brute_pairs(sq, skv, causal, window):
    pos = np.arange(sq)[:, None] + (skv - sq)
    keys = np.arange(skv)[None, :]
    vis = np.ones((sq, skv), dtype=bool)
    if causal:
        vis &= keys <= pos
    if window > 0:
        vis &= keys > pos - window
    return int(vis.sum())


@pytest.mark.parametrize("sq,skv,causal,window", [
    (128, 128, True, 0), (100, 300, True, 0), (64, 200, False, 0), (300, 300, True, 1),
    (300, 300, True, 77), (90, 500, True, 640), (64, 200, False, 100), (3314, 3314, True, 1024),
])
def test_visible_pairs_match_the_mask(sq, skv, causal, window):
    cfg = inputs.PrefillConfig("t", 1, 1, 1, 64, sq, skv, "f16", causal, seed=0, window=window)
    assert cfg.visible_pairs() == _brute_pairs(sq, skv, causal, window)


def test_flops_of_named_workloads():
    g = inputs.GQA_PREFILL
    assert g.visible_pairs() == 3314 * 3315 // 2
    assert g.flops() == 4 * 128 * (3314 * 3315 // 2) * 28
    w = inputs.WINDOW_PREFILL
    # rows 0..1023 see i + 1 keys, the rest see 1024
    assert w.visible_pairs() == 1024 * 1025 // 2 + (3314 - 1024) * 1024
