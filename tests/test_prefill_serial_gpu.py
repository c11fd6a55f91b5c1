"""head_dim 256 prefill in the serial work-group order (each XCD takes its
query-head groups one after the other; every second group walks its key tiles
from the last to the first) against the fp64 oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O, row sum,
LSE), D2 (query heads of a KV head packed on one K/V stream), D3/D4 (length
and causal masks on the windowed branch). The order applies when the launch
has a multiple of 8 (batch, KV head) groups, more than 8, and each group has at
least 64 work-groups (an XCD's slots); the shapes here are sized for that
(16 groups of 4 query heads x 16 blocks). The online softmax may take the
tiles in any order, so the gate is the usual one: |O| error <= 2e-3, LSE error
<= 1e-4, on rows sampled from every 128-row block (first, last and one inside)
of every head, plus byte-identical repeats.
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
        rows |= {qb * 128, qb * 128 + 61, min(qb * 128 + 127, S - 1)}
    return sorted(rows)


# (B, S, Hq, Hkv, dtype, unnorm, kv_lens, window, k_mult)
CASES = [
    (1, 2048, 64, 16, "bf16", False, None, 0, 1.0),
    (2, 2048, 32, 8, "bf16", True, None, 0, 4.0),          # un-normalized, peaked rows
    (2, 2000, 32, 8, "f16", False, [2000, 1377], 700, 1.0),  # ragged, lengths, window
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:6])))
def test_serial_order_matches_oracle(torch_gpu, case):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv, dtype, unnorm, lens, window, kmul = case
    D = 256
    nqb = -(-S // 128)
    assert (B * Hkv) % 8 == 0 and B * Hkv > 8 and (Hq // Hkv) * nqb >= 64
    _say("serial order", case)
    rng = np.random.default_rng(S + Hq + B)
    q = inputs.draw_half(rng, (B, S, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, S, Hkv, D), dtype, mult=kmul)
    v = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        r = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale, out_unnormalized=unnorm,
                       want_row_sum=True, kv_lens=ld, window=window)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in r])
    for a, b in zip(*outs):
        assert a.tobytes() == b.tobytes()
    o, lse, rs = outs[0]
    rows = _rows(S)
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, rows=rows,
                         kv_lens=lens, window=window)
    got_o = o[:, rows]
    got_l = lse[:, :, rows]
    if unnorm:
        got_o = got_o / np.transpose(rs[:, :, rows], (0, 2, 1))[..., None]
        err_rs = np.abs(np.log(rs[:, :, rows].astype(np.float64)) - np.log(ref["row_sum"]))
        assert err_rs.max() <= LSE_TOL
    seen = np.isfinite(ref["lse"])
    seen_o = np.transpose(seen, (0, 2, 1))
    err_o = np.abs(got_o[seen_o] - ref["o"][seen_o]).max()
    err_l = np.abs(got_l[seen] - ref["lse"][seen]).max()
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
    assert (got_o[~seen_o] == 0).all() and np.isneginf(got_l[~seen]).all()
