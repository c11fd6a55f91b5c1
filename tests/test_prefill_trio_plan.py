"""Host side of the choice between two and three prefill work-groups per
compute unit (CPU only).

The rule is re-derived here from the shape: head_dim 128, an odd number of
query heads per KV head (one head per work-group), 128-row blocks whose key
tile counts (64-key tiles, from the mask definitions: causal bound with
bottom-right alignment, sliding window) are about equal (longest <= 1.25 x
mean), and more blocks than 512 (two per compute unit of 256) but at most 768
(three). The query must be pure and reject bad sizes.
"""
import os

import pytest

from flashattention_attention_amd import fa

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa.so not built")


def _tiles(sq, skv, causal, window, bm=128, bn=64):
    off = skv - sq
    out = []
    for qb in range(-(-sq // bm)):
        first, last = qb * bm + off, min((qb + 1) * bm, sq) - 1 + off
        hi = min(skv - 1, last) if causal else skv - 1
        lo = max(0, first - window + 1) if window > 0 else 0
        out.append(hi // bn - lo // bn + 1 if hi >= lo else 0)
    return out


def _expected(b, sq, skv, hq, hkv, d, causal, window):
    if d != 128 or (hq // hkv) % 2 == 0:
        return False
    t = _tiles(sq, skv, causal, window)
    wgs = b * hq * len(t)
    if not 512 < wgs <= 768 or sum(t) == 0:
        return False
    return max(t) <= 1.25 * sum(t) / len(t)


SHAPES = [
    # batch, Sq, Skv, Hq, Hkv, D, causal, window
    (1, 3314, 3314, 28, 4, 128, True, 1024),   # the windowed GQA prompt: three per CU
    (1, 3314, 3314, 28, 4, 128, True, 0),      # the causal GQA prompt: two
    (1, 3314, 3314, 28, 4, 64, True, 1024),    # head_dim 64: two
    (1, 3314, 3314, 32, 4, 128, True, 1024),   # even group (paired heads): two
    (1, 2048, 2048, 28, 4, 128, False, 0),     # 448 equal blocks: one round of two
    (1, 2600, 2600, 28, 4, 128, False, 0),     # 588 equal blocks: three
    (1, 3500, 3500, 28, 4, 128, False, 0),     # 784 blocks: more than three hold
    (1, 129, 129, 280, 40, 128, False, 0),     # 560 blocks of 3 tiles
    (1, 1024, 1024, 70, 10, 128, True, 256),   # windowed: tiles 2, 4, 6 x 6
    (2, 1024, 1024, 42, 6, 128, True, 256),
    (1, 1024, 1024, 70, 10, 128, True, 0),     # causal: unequal
    (3, 77, 5000, 189, 27, 128, True, 0),      # queries at the end of a long cache
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_trio_choice_matches_rule(shape):
    b, sq, skv, hq, hkv, d, causal, win = shape
    got = fa.prefill_trio(b, sq, skv, hq, hkv, d, causal, win)
    assert got == _expected(b, sq, skv, hq, hkv, d, causal, win)
    assert got == fa.prefill_trio(b, sq, skv, hq, hkv, d, causal, win)   # pure


def test_trio_choice_for_the_workloads():
    assert fa.prefill_trio(1, 3314, 3314, 28, 4, 128, True, 1024)
    assert not fa.prefill_trio(1, 3314, 3314, 28, 4, 128, True, 0)


@pytest.mark.parametrize("bad", [(0, 10, 10, 1, 1, 128, 1, 0), (1, 10, 10, 3, 2, 128, 1, 0),
                                 (1, 10, 10, 1, 1, 128, 1, -1), (1, -5, 10, 1, 1, 128, 1, 0)])
def test_trio_rejects_bad_sizes(bad):
    assert fa.load_library().fa_prefill_trio(*bad) == -1
