"""Host side of the key-split prefill (CPU only): the work order the library
plans for a shape, the scratch size, and argument checks of the split entry
point before any HIP call.

The plan is checked against an independent reading of what it must be: each
128-row query block is handed out either whole or as both halves of its key
tiles, units come longest first, and the plan's end time under the list-
scheduling model (two work-groups per compute unit of 256, units handed to the
earliest free slot in order, a half costing 6 tile times beyond its tiles)
beats the unsplit order by at least 5 %, and that only launches whose
longest blocks far outlast the average slot's work are split. Tile
counts are recomputed here from the mask definitions (causal bound with
bottom-right alignment, sliding window).
"""
import ctypes
import heapq
import os

import pytest

from flashattention_attention_amd import fa

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa.so not built")

ALIGNED = 0x10000          # never dereferenced: every call below fails validation first
SLOTS = 256 * 2


def _tiles(sq, skv, causal, window, bm=128, bn=64):
    """Key tiles of 64 keys touched by each query block (keys any of its rows sees)."""
    off = skv - sq
    out = []
    for qb in range(-(-sq // bm)):
        first, last = qb * bm + off, min((qb + 1) * bm, sq) - 1 + off   # key positions of rows
        hi = min(skv - 1, last) if causal else skv - 1
        lo = max(0, first - window + 1) if window > 0 else 0
        out.append(hi // bn - lo // bn + 1 if hi >= lo else 0)
    return out


def _makespan(sizes, copies, slots):
    heap = [0.0] * slots
    end = 0.0
    for s in sizes:
        for _ in range(copies):
            t = heapq.heappop(heap) + s
            heapq.heappush(heap, t)
            end = max(end, t)
    return end


SHAPES = [
    # batch, Sq, Skv, Hq, Hkv, D, causal, window
    (1, 3314, 3314, 28, 4, 128, True, 0),      # the GQA prompt
    (1, 3314, 3314, 28, 4, 128, True, 1024),   # ... under a 1024-position window
    (1, 1000, 1000, 8, 8, 64, True, 0),
    (2, 777, 1500, 16, 2, 128, True, 0),        # queries at the end of a longer cache
    (1, 4096, 4096, 32, 8, 128, False, 0),      # unmasked: equal blocks
    (1, 8192, 8192, 8, 8, 128, True, 0),        # few heads, a long prompt
    (1, 6000, 6000, 4, 2, 64, True, 2048),      # ... under a window
]


@pytest.mark.parametrize("shape", SHAPES)
def test_plan_covers_blocks_longest_first_and_gains(shape):
    B, sq, skv, hq, hkv, d, causal, win = shape
    units = fa.prefill_split_units(B, sq, skv, hq, hkv, d, causal, win)
    assert units == fa.prefill_split_units(B, sq, skv, hq, hkv, d, causal, win)   # pure
    tiles = _tiles(sq, skv, causal, win)
    nqb = len(tiles)
    hp = 2 if (hq // hkv) % 2 == 0 else 1
    copies, slots = B * hkv * (hq // hkv) // hp, SLOTS // hp
    none = _makespan(sorted(tiles, reverse=True), copies, slots)
    if not units:
        return
    # split only where the longest blocks far outlast the average slot's work
    assert none >= 1.5 * sum(tiles) * copies / slots
    seen = {}
    for qb, kind in units:
        assert 0 <= qb < nqb and kind in (0, 1, 2)
        seen.setdefault(qb, []).append(kind)
    assert sorted(seen) == list(range(nqb))
    for qb, kinds in seen.items():
        assert sorted(kinds) in ([0], [1, 2]), (qb, kinds)
        if kinds != [0]:
            assert tiles[qb] >= 2
    # a half costs 6 tile times beyond its tiles (prologue, partial, merge)
    sizes = [tiles[qb] if k == 0 else
             (tiles[qb] // 2 if k == 1 else tiles[qb] - tiles[qb] // 2) + 6.0
             for qb, k in units]
    assert sizes == sorted(sizes, reverse=True)
    modeled = _makespan(sizes, copies, slots)
    assert modeled <= 0.95 * none, (modeled, none)


def test_plan_examples():
    # 28 heads x 26 blocks over 512 slots: the tail costs too little to split
    assert fa.prefill_split_units(1, 3314, 3314, 28, 4, 128, True, 0) == []
    assert fa.prefill_split_units(1, 3314, 3314, 28, 4, 128, True, 1024) == []
    # few heads, a long prompt: nearly every block splits, the longest first
    u = fa.prefill_split_units(1, 8192, 8192, 8, 8, 128, True, 0)
    assert sum(1 for _, k in u if k == 1) >= 60
    assert u[:2] == [(63, 1), (63, 2)]
    assert (0, 0) in u                          # the shortest runs whole
    # four prompts already fill the slots evenly enough: no split
    assert fa.prefill_split_units(4, 3314, 3314, 28, 4, 128, True, 0) == []
    # head dims the split kernel is not built for
    assert fa.prefill_split_units(1, 3314, 3314, 28, 4, 256, True, 0) == []
    assert fa.prefill_split_units(1, 3314, 3314, 28, 4, 512, True, 0) == []
    with pytest.raises(fa.FAError):
        fa.prefill_split_units(1, 3314, 3314, 28, 3, 128, True, 0)
    with pytest.raises(fa.FAError):
        fa.prefill_split_units(1, 3314, 3314, 28, 4, 128, True, -1)


def test_split_workspace_size():
    # 64 KiB of arrival counters at offset 0 for every shape, then the partial
    # LSEs and outputs of the two halves of every query block
    lib = fa.load_library()
    blocks = 1 * 28 * 26
    up = lambda x: (x + 255) // 256 * 256
    want = 65536 + up(blocks * 2 * 128 * 4) + blocks * 2 * 128 * 128 * 4
    assert lib.fa_prefill_split_workspace_size(1, 3314, 28, 128) == want
    assert lib.fa_prefill_split_workspace_size(0, 3314, 28, 128) == 0
    assert lib.fa_prefill_split_workspace_size(1, 1, 1, 64) == 65536 + 1024 + 2 * 128 * 64 * 4


def test_split_counter_capacity():
    # one counter per 128-row query block of every (batch entry, query head):
    # 16384 fit in the fixed region; a shape with more runs unsplit
    few = fa.prefill_split_units(1, 8192, 8192, 8, 8, 128, True, 0)
    assert few, "a long prompt over few heads splits"
    assert fa.prefill_split_units(1, 16384, 16384, 129, 129, 64, True, 0) == []


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(Hkv=3), 1), (dict(D=1024), 2), (dict(ws=None), 1),
    (dict(sws=None), 1), (dict(swsb=1000), 1), (dict(sws=ALIGNED + 16), 1),
])
def test_prefill_fwd_packed_split_validation(kw, status):
    b = dict(q=ALIGNED, k=ALIGNED, o=ALIGNED, lse=ALIGNED, row_sum=None, B=1, Sq=128, Skv=128,
             Hq=4, Hkv=2, D=128, dtype=0, causal=1, scale=0.125, unnorm=0,
             qs=(128 * 4 * 128, 4 * 128, 128), ks=(128 * 2 * 128, 2 * 128, 128),
             os=(128 * 4 * 128, 4 * 128, 128), ws=ALIGNED, wsb=1 << 40, lens=None, win=0,
             sink=None, sws=ALIGNED, swsb=1 << 40)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_prefill_fwd_packed_split(
        b["q"], *b["qs"], b["k"], *b["ks"], b["o"], *b["os"], b["lse"], b["row_sum"], b["B"],
        b["Sq"], b["Skv"], b["Hq"], b["Hkv"], b["D"], b["dtype"], b["causal"], b["scale"],
        b["unnorm"], b["lens"], b["win"], b["sink"], b["ws"], b["wsb"], b["sws"], b["swsb"],
        None)
    assert st == status, lib.fa_last_error()
