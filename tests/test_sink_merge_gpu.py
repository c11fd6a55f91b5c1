"""Parity of the sink logit (folded into the prefill epilogue) and of the LSE
merge of two passes (fa_attn_merge) against the fp64 oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", D5 (a sliding-window pass and
a sink merged through their LSEs; D5b merges after the kernels, D5d folds the
sink merge into the epilogue). Gate as for the prefill: |O| error <= 2e-3,
natural-log LSE error <= 1e-4 (row sums: |ln| error <= 1e-4), rows without
keys exact.
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


def _f32(torch, x):
    return torch.tensor(np.asarray(x, np.float32), device="cuda")


def _prefill(torch, q, k, v, dtype, *, causal, scale, lens=None, window=0, sinks=None,
             unnorm=False):
    from flashattention_attention_amd import fa
    B, Sq, Hq, D = q.shape
    out = torch.full((B, Sq, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    rs = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    fa.prefill(_dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype),
               causal=causal, softmax_scale=scale, out_unnormalized=unnorm, out=out, lse=lse,
               row_sum=rs,
               kv_lens=None if lens is None else torch.tensor(lens, dtype=torch.int32,
                                                              device="cuda"),
               window=window, sink_logits=None if sinks is None else _f32(torch, sinks))
    torch.cuda.synchronize()
    return out, lse, rs


def _check(o, lse, ref, rs=None, unnorm=False):
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(o).all() and not np.isnan(lse).any()
    if unnorm:
        rs = rs.cpu().numpy()
        err_rs = np.abs(np.log(rs.astype(np.float64)) - np.log(ref["row_sum"])).max()
        assert err_rs <= LSE_TOL, err_rs
        o = o / np.transpose(rs, (0, 2, 1))[..., None]
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lse) == ~fin).all()
    err_o = np.abs(o - ref["o"]).max()
    err_l = np.abs(lse[fin] - ref["lse"][fin]).max(initial=0.0)
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"


# (B, Sq, Skv, Hq, Hkv, D, dtype, causal, kv_lens, window, sinks, unnorm)
SINK_CASES = [
    (2, 200, 200, 8, 2, 128, "bf16", True, None, 0, [0.5, -1.0, 3.0, 0.0, 1.5, -2.0, 20.0, 0.25],
     False),
    (1, 300, 300, 7, 1, 128, "f16", True, None, 64, [1.0, 2.0, -3.0, 0.0, 4.0, -0.5, 8.0], False),
    (2, 150, 150, 4, 2, 64, "bf16", True, [150, 40], 30, [0.0, 1.0, -1.0, 30.0], False),
    (1, 260, 260, 4, 4, 256, "bf16", True, None, 100, [2.0, -2.0, 0.5, 12.0], False),
    (2, 129, 300, 4, 2, 128, "f16", True, [300, 0], 0, [-0.75, 0.75, 1.0, 5.0], False),
    (2, 200, 200, 4, 2, 128, "bf16", True, [200, 77], 50, [0.5, 3.0, -4.0, 25.0], True),
    (1, 190, 190, 4, 4, 256, "f16", False, None, 0, [1.0, 0.0, -1.0, 40.0], True),
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,dtype,causal,lens,window,sinks,unnorm", SINK_CASES)
def test_prefill_sink_epilogue(torch_gpu, B, Sq, Skv, Hq, Hkv, D, dtype, causal, lens, window,
                               sinks, unnorm):
    torch = torch_gpu
    _say("sink", B, Sq, Skv, Hq, Hkv, D, dtype, causal, lens, window, unnorm)
    rng = np.random.default_rng(Sq + Skv + D + window)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype, mult=4.0 if unnorm else 1.0)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    sinks32 = np.asarray(sinks, np.float32)
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype=dtype, kv_lens=lens,
                         window=window, sink_logits=sinks32.astype(np.float64))
    o, lse, rs = _prefill(torch, q, k, v, dtype, causal=causal, scale=scale, lens=lens,
                          window=window, sinks=sinks32, unnorm=unnorm)
    _check(o, lse, ref, rs, unnorm)


def test_sink_at_minus_inf_is_no_sink(torch_gpu):
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype = 2, 300, 8, 2, 128, "bf16"
    _say("sink -inf identity")
    rng = np.random.default_rng(21)
    q, k, v = (inputs.draw_half(rng, (B, S, h, D), dtype) for h in (Hq, Hkv, Hkv))
    scale = float(np.float32(1 / np.sqrt(D)))
    a = _prefill(torch, q, k, v, dtype, causal=True, scale=scale, lens=[300, 120], window=70)
    b = _prefill(torch, q, k, v, dtype, causal=True, scale=scale, lens=[300, 120], window=70,
                 sinks=[-np.inf] * Hq)
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, kv_lens=[300, 120],
                         window=70)
    _check(b[0], b[1], ref)
    # the sink path normalizes through exp2/log2 instead of 1/l: a few ulp apart
    np.testing.assert_allclose(a[0].cpu().numpy(), b[0].cpu().numpy(), rtol=2e-6, atol=1e-6)
    np.testing.assert_allclose(a[1].cpu().numpy(), b[1].cpu().numpy(), rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("D,Hq,Hkv,dtype,L,Sq", [(128, 28, 4, "bf16", 700, 300),
                                                (64, 8, 8, "f16", 129, 64),
                                                (256, 4, 2, "bf16", 333, 129)])
def test_merge_prefix_and_new_tokens(torch_gpu, D, Hq, Hkv, dtype, L, Sq):
    """A cached prefix of L keys (every query sees all of it) and Sq new tokens
    (causal among themselves): the LSE merge of the two passes is causal
    attention over the whole L + Sq keys; with a sink, it is that attention with
    the sink. Also in place (out = pass A)."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    _say("merge prefix+new", D, Hq, Hkv, dtype, L, Sq)
    B = 2
    rng = np.random.default_rng(D + L)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, L + Sq, Hkv, D), dtype)
    v = inputs.draw_half(rng, (B, L + Sq, Hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    oa, la, _ = _prefill(torch, q, k[:, :L], v[:, :L], dtype, causal=False, scale=scale)
    ob, lb, _ = _prefill(torch, q, k[:, L:], v[:, L:], dtype, causal=True, scale=scale)
    sinks = np.linspace(-2.0, 6.0, Hq).astype(np.float32)
    o, lse = fa.attn_merge(oa, la, ob, lb)
    o_s, lse_s = fa.attn_merge(oa, la, ob, lb, sink_logits=_f32(torch, sinks))
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype)
    _check(o, lse, ref)
    ref_s = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype,
                           sink_logits=sinks.astype(np.float64))
    _check(o_s, lse_s, ref_s)
    # in place: the result replaces pass A and matches the out-of-place one bitwise
    fa.attn_merge(oa, la, ob, lb, sink_logits=_f32(torch, sinks), out=oa, lse=la)
    torch.cuda.synchronize()
    assert oa.cpu().numpy().tobytes() == o_s.cpu().numpy().tobytes()
    assert la.cpu().numpy().tobytes() == lse_s.cpu().numpy().tobytes()


def test_merge_sink_matches_epilogue_sink(torch_gpu):
    """The sink folded into the epilogue and the sink merged afterwards agree."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype = 1, 500, 28, 4, 128, "bf16"
    _say("sink epilogue vs merge")
    rng = np.random.default_rng(31)
    q, k, v = (inputs.draw_half(rng, (B, S, h, D), dtype) for h in (Hq, Hkv, Hkv))
    scale = float(np.float32(1 / np.sqrt(D)))
    sinks = np.linspace(-3.0, 9.0, Hq).astype(np.float32)
    fused = _prefill(torch, q, k, v, dtype, causal=True, scale=scale, window=128, sinks=sinks)
    plain = _prefill(torch, q, k, v, dtype, causal=True, scale=scale, window=128)
    o, lse = fa.attn_merge(plain[0], plain[1], sink_logits=_f32(torch, sinks))
    torch.cuda.synchronize()
    assert np.abs(o.cpu().numpy() - fused[0].cpu().numpy()).max() <= 1e-5
    assert np.abs(lse.cpu().numpy() - fused[1].cpu().numpy()).max() <= 1e-5


def test_merge_decode_layout_and_empty_rows(torch_gpu):
    """Decode outputs ([B,H,D], [B,H]) of two caches merged, one sequence with an
    empty second pass (LSE -inf) and all-empty rows (both -inf, no sink)."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    _say("merge decode layout")
    rng = np.random.default_rng(41)
    B, H, D = 3, 6, 128
    oa = rng.standard_normal((B, H, D)).astype(np.float32)
    ob = rng.standard_normal((B, H, D)).astype(np.float32)
    la = (rng.standard_normal((B, H)) * 3).astype(np.float32)
    lb = (rng.standard_normal((B, H)) * 3).astype(np.float32)
    lb[1] = -np.inf                        # second pass saw no key
    la[2, :2] = lb[2, :2] = -np.inf        # neither did
    o, lse = fa.attn_merge(_f32(torch, oa), _f32(torch, la), _f32(torch, ob), _f32(torch, lb))
    torch.cuda.synchronize()
    ref = oracle.merge_branches([oa.astype(np.float64), ob.astype(np.float64)],
                                [la.astype(np.float64), lb.astype(np.float64)])
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    np.testing.assert_allclose(o, ref["o"], rtol=0, atol=1e-5)
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lse) == ~fin).all()
    np.testing.assert_allclose(lse[fin], ref["lse"][fin], rtol=0, atol=1e-5)
    assert (o[2, :2] == 0).all()
