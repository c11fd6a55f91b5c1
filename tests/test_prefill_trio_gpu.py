"""The three-per-CU prefill form (head_dim 128, one query head per work-group,
32-key tiles read as halves of the pre-pass's 64-key V^T tiles) against the
fp64 oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O, row sum,
LSE), D3/D4 (length and window masks) and D5 (per-head sinks); "60 · r57 — FA
KV staging double buffering (REVERTED)", section 1 (grid over query blocks and
heads). Every shape here is one the library runs in this form
(fa.prefill_trio is asserted first): grids of about equal blocks with more
than 512 and at most 768 of them. The gate is the prefill one: |O| error <=
2e-3, LSE error <= 1e-4, plus byte-identical repeats. The oracle's extra time
is under two seconds per case (sampled rows for the long ones).
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


def _block_rows(S):
    rows = set()
    for qb in range(-(-S // 128)):
        rows |= {qb * 128, qb * 128 + 61, min(qb * 128 + 127, S - 1)}
    return sorted(rows)


# (B, Sq, Skv, Hq, Hkv, dtype, causal, unnorm, kv_lens, window, sinks, k_mult, rows)
CASES = [
    (1, 129, 129, 280, 40, "bf16", False, False, None, 0, False, 1.0, None),   # ragged block
    (1, 129, 129, 280, 40, "f16", False, False, None, 0, False, 1.0, None),
    (1, 129, 129, 280, 40, "bf16", False, True, None, 0, False, 4.0, None),    # un-normalized
    (1, 1024, 1024, 70, 10, "bf16", True, False, None, 256, True, 1.0, None),  # window + sinks
    (2, 1024, 1024, 42, 6, "f16", True, False, [1024, 700], 256, False, 4.0, None),
    (3, 77, 5000, 189, 27, "bf16", True, False, None, 0, False, 1.0, [0, 38, 76]),
    (2, 129, 129, 140, 20, "bf16", False, False, [0, 77], 0, False, 1.0, None),  # empty sequence
    (2, 200, 300, 140, 20, "f16", True, False, [300, 150], 5000, True, 2.0, None),  # window > S
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:11])))
def test_trio_prefill_matches_oracle(torch_gpu, case):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, Sq, Skv, Hq, Hkv, dtype, causal, unnorm, lens, window, with_sinks, kmul, rows = case
    D = 128
    assert fa.prefill_trio(B, Sq, Skv, Hq, Hkv, D, causal, window)
    _say("trio", case[:11])
    rng = np.random.default_rng(Sq * 3 + Skv + Hq)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype, mult=kmul)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    sinks = np.linspace(-1.0, 3.0, Hq).astype(np.float32) if with_sinks else None
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    sd = None if sinks is None else torch.from_numpy(sinks).cuda()
    vt = fa.prefill_pack_v(vd)
    outs = []
    for _ in range(2):
        r = fa.prefill_packed(qd, kd, vt, causal=causal, softmax_scale=scale,
                              out_unnormalized=unnorm, want_row_sum=unnorm, kv_lens=ld,
                              window=window, sink_logits=sd)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in r])
    for a, b in zip(*outs):
        assert a.tobytes() == b.tobytes()
    o, lse = outs[0][0], outs[0][1]
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype=dtype, rows=rows,
                         kv_lens=lens, window=window, sink_logits=sinks)
    if rows is not None:
        o, lse = o[:, rows], lse[:, :, rows]
    seen = np.isfinite(ref["lse"])
    seen_o = np.transpose(seen, (0, 2, 1))
    if unnorm:
        rs = outs[0][2] if rows is None else outs[0][2][:, :, rows]
        o = o / np.transpose(rs, (0, 2, 1))[..., None]
        err_rs = np.abs(np.log(rs[seen].astype(np.float64)) - np.log(ref["row_sum"][seen]))
        assert err_rs.max() <= LSE_TOL
    err_o = np.abs(o[seen_o] - ref["o"][seen_o]).max()
    err_l = np.abs(lse[seen] - ref["lse"][seen]).max()
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
    if not with_sinks:
        assert (o[~seen_o] == 0).all() and np.isneginf(lse[~seen]).all()


def test_trio_windowed_gqa_prompt(torch_gpu):
    """The 3314-token GQA prompt under a 1024-position window (28 query / 4 KV
    heads, bf16): rows sampled from every 128-row block of every head (first,
    last and one inside) meet the gate, through the two-launch call the
    benchmark times."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    cfg = inputs.WINDOW_PREFILL
    B, S, Hq, Hkv, D = cfg.batch, cfg.seqlen_q, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim
    assert fa.prefill_trio(B, S, S, Hq, Hkv, D, True, cfg.window)
    _say("trio windowed prompt", cfg.name)
    x = inputs.make_prefill_inputs(cfg)
    q, k, v = x["q"], x["k"], x["v"]
    scale = cfg.scale
    o, lse = fa.prefill(_dev(torch, q, "bf16"), _dev(torch, k, "bf16"), _dev(torch, v, "bf16"),
                        causal=True, softmax_scale=scale, window=cfg.window)
    torch.cuda.synchronize()
    rows = _block_rows(S)
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="bf16", rows=rows,
                         window=cfg.window)
    o, lse = o.cpu().numpy()[:, rows], lse.cpu().numpy()[:, :, rows]
    assert np.abs(o - ref["o"]).max() <= O_TOL
    assert np.abs(lse - ref["lse"]).max() <= LSE_TOL
