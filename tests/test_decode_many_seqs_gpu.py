"""Decode over batches of many sequences (70, 80, 130 and 300) against the fp64
oracle (needs an MI355X).

Source: "66 · D2: explicit K+V register staging ...", section 1 (split-KV
partials merged by their LSE) and "STAGE_D.md — FMHA Kernel Development",
"Kernel Output" (O and the natural-log LSE). The decode kernels number the (sequence, split) units
with work densely: each work-group scans the lengths, 64 sequences per step
and four steps per round of loads, to find its unit. These batches cross one,
two and more than four such steps, and mix in sequences with no key and
sequences longer than max_splits * split_len (reported as NaN), so every
branch of that scan and both launch forms meet the oracle:

* two launches: every split's partial O and LSE (up to max_splits for the
  long sequences), untouched NaN canaries past a sequence's last split, the
  merged O and LSE of the well-formed sequences, NaN for the others;
* one launch (fa_decode_fused): the same merged results, repeated bitwise,
  with its arrival counters back at zero.

Gate: |O| error <= 2e-3, LSE error <= 1e-4. The oracle's extra time is under
a second per case (one fp64 attention per sequence, head and split).
"""
import numpy as np
import pytest

import oracle
from flashattention_attention_amd import inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-4


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from flashattention_attention_amd import fa
    fa.load_library()
    return torch


def _say(*a):
    print("[case]", *a, flush=True)


def _dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


# (batch, Hq, Hkv, D, dtype, split_len, max_splits)
CASES = [
    (300, 8, 2, 128, "f16", 32, 5),
    (80, 28, 4, 128, "bf16", 16, 6),
    (130, 4, 4, 64, "f16", 16, 4),
    (70, 16, 2, 256, "bf16", 32, 4),     # head_dim 256: the VALU split form
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_many_sequences_match_oracle(torch_gpu, case):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, Hq, Hkv, D, dtype, sl, ms = case
    _say("many sequences", case)
    rng = np.random.default_rng(B * 7 + Hq + D)
    lens = rng.integers(1, sl * (ms + 2), B).astype(np.int32)
    lens[::37] = 0                                   # sequences with no key
    lens[5] = sl * ms                                # exactly max_splits full splits
    lens[6] = sl * ms + 1                            # one key too many
    good = (lens >= 1) & (lens <= sl * ms)
    assert good.sum() > B // 2 and (~good & (lens > 0)).any() and (lens == 0).any()
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    T = int(lens.sum())
    q = inputs.draw_half(rng, (B, Hq, D), dtype)
    kc = inputs.draw_half(rng, (T, Hkv, D), dtype)
    vc = inputs.draw_half(rng, (T, Hkv, D), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    dx = (_dev(torch, q, dtype), _dev(torch, kc, dtype), _dev(torch, vc, dtype),
          torch.from_numpy(offs).cuda(), torch.from_numpy(lens).cuda())

    # two launches
    po = torch.full((B, Hq, ms, D), float("nan"), device="cuda")
    pl = torch.full((B, Hq, ms), float("nan"), device="cuda")
    fa.decode_split_partial(*dx, split_len=sl, max_splits=ms, softmax_scale=scale,
                            part_o=po, part_lse=pl)
    o2, lse2 = fa.decode_merge_lse(po, pl, dx[4], split_len=sl)
    torch.cuda.synchronize()
    po, pl, o2, lse2 = (t.cpu().numpy() for t in (po, pl, o2, lse2))

    # the partials the kernel computes: the first max_splits splits of every sequence
    trunc = np.minimum(lens, sl * ms).astype(np.int32)
    parts = oracle.decode_split_partials(q, kc, vc, offs, trunc, scale=scale, split_len=sl,
                                         max_splits=ms, dtype=dtype)
    ns = np.array([-(-int(L) // sl) for L in trunc])
    for b in range(B):
        assert np.isnan(pl[b, :, ns[b]:]).all() and np.isnan(po[b, :, ns[b]:]).all()
        if ns[b]:
            assert np.abs(po[b, :, :ns[b]] - parts["part_o"][b, :, :ns[b]]).max() <= O_TOL
            assert np.abs(pl[b, :, :ns[b]] - parts["part_lse"][b, :, :ns[b]]).max() <= LSE_TOL

    ref = oracle.decode(q[good], kc, vc, offs[good], lens[good], scale=scale, dtype=dtype)
    assert np.abs(o2[good] - ref["o"]).max() <= O_TOL
    assert np.abs(lse2[good] - ref["lse"]).max() <= LSE_TOL
    assert np.isnan(o2[~good]).all() and np.isnan(lse2[~good]).all()

    # one launch
    ws = torch.zeros(fa.decode_fused_workspace_size(B, Hq, Hkv, D, ms), dtype=torch.uint8,
                     device="cuda")
    runs = []
    for _ in range(2):
        o1 = torch.full((B, Hq, D), float("nan"), device="cuda")
        l1 = torch.full((B, Hq), float("nan"), device="cuda")
        fa.decode_fused(*dx, split_len=sl, max_splits=ms, softmax_scale=scale, out=o1, lse=l1,
                        workspace=ws)
        torch.cuda.synchronize()
        runs.append((o1.cpu().numpy(), l1.cpu().numpy()))
    assert runs[0][0].tobytes() == runs[1][0].tobytes()
    assert runs[0][1].tobytes() == runs[1][1].tobytes()
    g = max(d for d in range(1, 9) if (Hq // Hkv) % d == 0)
    assert not ws[:B * (Hq // g) * 4].cpu().numpy().any()     # arrival counters back at zero
    o1, l1 = runs[0]
    assert np.abs(o1[good] - ref["o"]).max() <= O_TOL
    assert np.abs(l1[good] - ref["lse"]).max() <= LSE_TOL
    assert np.isnan(o1[~good]).all() and np.isnan(l1[~good]).all()
