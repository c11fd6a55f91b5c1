"""The one-launch fp16 prefill (head_dim 64 and 128), which takes V's rows
straight from HBM into LDS and transposes them on the way into the P.V
contraction, against the fp64 oracle and against the two-launch form (V
repacked, then the attention kernel) (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O and the
natural-log LSE), D3/D4 (length and causal masks) and D5 (per-head sinks).
The two forms feed the same fp16 values of V into the same products in the
same order, so their outputs must agree bit for bit; the oracle gate is the
prefill one: |O| error <= 2e-3, LSE error <= 1e-4.
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


def _dev(torch, bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16).cuda()


def _both(torch, qd, kd, vd, scale, causal, unnorm, lens, window, sinks):
    """(direct, packed) outputs as numpy: o, lse, row_sum."""
    from flashattention_attention_amd import fa
    kw = dict(causal=causal, softmax_scale=scale, out_unnormalized=unnorm, want_row_sum=True,
              kv_lens=lens, window=window, sink_logits=sinks)
    d = fa.prefill(qd, kd, vd, **kw)
    p = fa.prefill_packed(qd, kd, fa.prefill_pack_v(vd), **kw)
    torch.cuda.synchronize()
    return [tuple(x.cpu().numpy() for x in r) for r in (d, p)]


# (B, Sq, Skv, Hq, Hkv, D, causal, unnorm, kv_lens, window, sinks)
CASES = [
    (1, 128, 128, 1, 1, 64, True, False, None, 0, False),         # the tiny prompt
    (1, 200, 200, 7, 1, 128, True, False, None, 0, False),        # odd group: one head per wave
    (2, 190, 190, 8, 2, 128, True, False, None, 0, False),        # even group: paired heads
    (1, 77, 333, 4, 4, 64, False, False, None, 0, False),         # unmasked, Sq < Skv, ragged
    (2, 300, 300, 6, 3, 128, True, True, None, 0, False),         # un-normalized + row sums
    (2, 250, 250, 8, 4, 64, True, True, None, 0, False),          # ... paired, head_dim 64
    (3, 160, 260, 4, 2, 128, True, False, [260, 131, 1], 70, False),   # lengths + window
    (2, 129, 129, 6, 2, 64, True, False, None, 33, True),         # window + sinks
    (1, 1, 777, 28, 4, 128, True, False, None, 0, False),         # one query row, long KV
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:8])))
def test_vrow_prefill_matches_oracle_and_packed(torch_gpu, case):
    torch = torch_gpu
    B, Sq, Skv, Hq, Hkv, D, causal, unnorm, lens, window, with_sinks = case
    _say("vrow", case)
    rng = np.random.default_rng(Sq * 13 + Skv * 3 + D + Hq)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), "f16")
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), "f16", mult=4.0 if unnorm else 1.0)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), "f16")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    sinks = (np.linspace(-1.0, 3.0, Hq).astype(np.float32) if with_sinks else None)
    ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    sd = None if sinks is None else torch.from_numpy(sinks).cuda()
    (o, lse, rs), packed = _both(torch, _dev(torch, q), _dev(torch, k), _dev(torch, v), scale,
                                 causal, unnorm, ld, window, sd)
    for a, b in zip((o, lse, rs), packed):
        assert a.tobytes() == b.tobytes()
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16", kv_lens=lens,
                         window=window, sink_logits=sinks)
    seen = np.isfinite(ref["lse"])
    seen_o = np.transpose(seen, (0, 2, 1))
    got = o / np.transpose(rs, (0, 2, 1))[..., None] if unnorm else o
    err_o = np.abs(got[seen_o] - ref["o"][seen_o]).max(initial=0.0)
    err_l = np.abs(lse[seen] - ref["lse"][seen]).max(initial=0.0)
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
    if not with_sinks:
        assert (o[~seen_o] == 0).all() and np.isneginf(lse[~seen]).all()


@pytest.mark.parametrize("D", [64, 128])
def test_vrow_reads_strided_v(torch_gpu, D):
    """V as a view into a fused [B, S, 2, Hkv, D] KV tensor (row stride
    2 * Hkv * D, batch stride with padding): same bytes as a contiguous V."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv = 2, 230, 8, 2
    _say("vrow-strided", D)
    rng = np.random.default_rng(D + 1)
    q = inputs.draw_half(rng, (B, S, Hq, D), "f16")
    kv = inputs.draw_half(rng, (B, S + 3, 2, Hkv, D), "f16")
    kvd = _dev(torch, kv)[:, :S]
    kd, vd = kvd[:, :, 0], kvd[:, :, 1]
    assert vd.stride(1) == 2 * Hkv * D
    qd = _dev(torch, q)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o1, l1 = fa.prefill(qd, kd, vd, softmax_scale=scale)
    o2, l2 = fa.prefill(qd, kd.contiguous(), vd.contiguous(), softmax_scale=scale)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()


def test_vrow_full_gqa_prompt_matches_packed(torch_gpu):
    """The 3314-token prompt, 28 query / 4 KV heads, head_dim 128, in fp16:
    the one-launch form equals the two-launch form bit for bit on every row,
    and sampled rows of every head meet the oracle gate."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv, D = 1, 3314, 28, 4, 128
    _say("vrow-gqa-full", B, S, Hq, Hkv, D)
    rng = np.random.default_rng(3314)
    q = inputs.draw_half(rng, (B, S, Hq, D), "f16")
    k, v = (inputs.draw_half(rng, (B, S, Hkv, D), "f16") for _ in range(2))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q), _dev(torch, k), _dev(torch, v)
    o1, l1 = fa.prefill(qd, kd, vd, softmax_scale=scale)
    o2, l2 = fa.prefill_packed(qd, kd, fa.prefill_pack_v(vd), softmax_scale=scale)
    torch.cuda.synchronize()
    o1, l1 = o1.cpu().numpy(), l1.cpu().numpy()
    assert o1.tobytes() == o2.cpu().numpy().tobytes()
    assert l1.tobytes() == l2.cpu().numpy().tobytes()
    rows = [0, 1, 63, 64, 127, 128, 1000, 2047, 3200, 3263, 3264, 3313]
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16", rows=rows)
    assert np.abs(o1[:, rows] - ref["o"]).max() <= O_TOL
    assert np.abs(l1[:, :, rows] - ref["lse"]).max() <= LSE_TOL
