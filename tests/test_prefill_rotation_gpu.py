"""Prefill launches whose first two rounds of work-groups are re-paired
(grids of at least 512 work-groups at two per compute unit) against the fp64
oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O and the
natural-log LSE) and "60 · r57 — FA KV staging double buffering (REVERTED)",
section 1 (grid over query blocks and heads). The launcher permutes the
work-group ids of the second round of first-dispatched work-groups; every
query block of every head must still be computed exactly once. The shapes
reach each branch of the work-group numbering with the permutation on: a
number of (batch, KV head) groups that is neither a divisor nor a multiple
of 8 (3 groups), a multiple of 8 (16 groups), and a divisor of 8 with the
one-launch fp16 form at head_dim 64 (4 groups). The causal GQA prompt (4
groups, bf16, head_dim 128) is compared in full by the full-size parity
test. Gate: |O| error <= 2e-3, LSE error <= 1e-4 on the first, last and one
inner row of every 128-row block of every head, plus byte-identical repeats.
The oracle's extra time is under a second per case.
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


def _rows(S):
    rows = set()
    for qb in range(-(-S // 128)):
        rows |= {qb * 128, qb * 128 + 45, min(qb * 128 + 127, S - 1)}
    return sorted(rows)


def _grid(B, S, Hq, Hkv):
    """Work-groups of the one-head-per-work-group launch (odd or unit groups)."""
    groups, per_group, nqb = B * Hkv, Hq // Hkv, -(-S // 128)
    m = per_group * nqb
    if groups % 8 == 0 or 8 % groups != 0:
        return groups * m
    s = 8 // groups
    return 8 * (-(-m // s))


# (B, S, Hq, Hkv, D, dtype)
CASES = [
    (1, 3200, 21, 3, 128, "bf16"),    # 3 groups of 7 heads: 525 work-groups
    (1, 4096, 16, 16, 128, "bf16"),   # 16 groups of 1 head: 512 work-groups
    (2, 4096, 14, 2, 64, "f16"),      # 4 groups of 7 heads, one launch: 896 work-groups
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_repaired_first_rounds_match_oracle(torch_gpu, case):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype = case
    assert (Hq // Hkv) % 2 == 1 and _grid(B, S, Hq, Hkv) >= 512
    assert not fa.prefill_trio(B, S, S, Hq, Hkv, D, True, 0)
    _say("re-paired first rounds", case)
    rng = np.random.default_rng(S + Hq * 11 + D)
    q = inputs.draw_half(rng, (B, S, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
    v = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    outs = []
    for _ in range(2):
        o, lse = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    assert outs[0][0].tobytes() == outs[1][0].tobytes()
    assert outs[0][1].tobytes() == outs[1][1].tobytes()
    rows = _rows(S)
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, rows=rows)
    o, lse = outs[0][0][:, rows], outs[0][1][:, :, rows]
    err_o = np.abs(o - ref["o"]).max()
    err_l = np.abs(lse - ref["lse"]).max()
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
