"""Parity of the key-split prefill (fa_prefill_fwd_packed_split) against the
fp64 oracle (needs an MI355X).

Source: "66 · D2 ...", section 1 (the KV range of a query split into parts
merged afterwards, with the partition fixed by the shape) and "STAGE_D.md —
FMHA Kernel Development", D5 / D5c (partials merged through their LSE inside
the one launch). Same gate as every prefill test: |O| error <= 2e-3,
natural-log LSE error <= 1e-4, byte-identical repeats (which half of a split
block finishes last varies from run to run; the merge must not depend on it),
and the arrival counters back at zero after every call. Every case asserts
that the planner does split it.
"""
import zlib

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


def _split_runs(torch, q, k, v, dtype, *, causal, scale, window=0, lens=None, sinks=None,
                repeats=2):
    """Runs the split call `repeats` times and the unsplit call once; returns
    ([(o, lse) per split run], (o, lse) unsplit)."""
    from flashattention_attention_amd import fa
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    units = fa.prefill_split_units(B, Sq, Skv, Hq, Hkv, D, causal, window)
    assert units, "the planner does not split this shape"
    assert any(kind for _, kind in units)
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    kl = torch.from_numpy(np.asarray(lens, np.int32)).cuda() if lens is not None else None
    sk = torch.from_numpy(np.asarray(sinks, np.float32)).cuda() if sinks is not None else None
    packed = fa.prefill_pack_v(vd)
    sws = torch.zeros(fa.prefill_split_workspace_size(B, Sq, Hq, D), dtype=torch.uint8,
                      device="cuda")
    n_cnt = B * Hq * (-(-Sq // 128))
    assert n_cnt * 4 <= 65536
    runs = []
    for _ in range(repeats):
        out = torch.full((B, Sq, Hq, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
        fa.prefill_packed(qd, kd, packed, causal=causal, softmax_scale=scale, out=out, lse=lse,
                          kv_lens=kl, window=window, sink_logits=sk, split_workspace=sws)
        torch.cuda.synchronize()
        runs.append((out.cpu().numpy(), lse.cpu().numpy()))
        counters = sws[:4 * n_cnt].view(torch.int32)
        assert int(counters.abs().sum().item()) == 0, "arrival counters not reset"
    o1, l1 = fa.prefill_packed(qd, kd, packed, causal=causal, softmax_scale=scale, kv_lens=kl,
                               window=window, sink_logits=sk)
    torch.cuda.synchronize()
    return runs, (o1.cpu().numpy(), l1.cpu().numpy())


def _check(o, lse, ref, rows=None):
    if rows is not None:
        o, lse = o[:, rows], lse[:, :, rows]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    err_o = np.abs(o - ref["o"]).max()
    err_l = np.abs(lse - ref["lse"]).max()
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"


# name, B, Sq, Skv, Hq, Hkv, D, dtype, causal, window, kv_lens, sinks, k_mult
CASES = [
    ("gqa_causal_bf16", 1, 1000, 1000, 28, 4, 128, "bf16", True, 0, None, False, 1.0),
    ("mha_causal_f16_d64", 1, 1000, 1000, 8, 8, 64, "f16", True, 0, None, False, 4.0),
    # even group: two query heads per work-group; queries at the end of a longer cache
    ("paired_heads_cache_tail", 2, 777, 1500, 16, 2, 128, "bf16", True, 0, None, False, 1.0),
    ("window_1000", 1, 3000, 3000, 4, 2, 128, "bf16", True, 1000, None, False, 1.0),
    # a one-key sequence: the first half of every split block of it sees no key
    ("lens_and_sinks_f16", 3, 900, 900, 8, 4, 128, "f16", True, 0, [900, 451, 1], True, 4.0),
    ("window_sinks_d64", 1, 2500, 2500, 4, 4, 64, "bf16", True, 800, None, True, 1.0),
    # paired heads, fp16, a sequence shorter than the prompt's blocks reach
    ("paired_heads_lens_f16", 2, 1400, 1400, 8, 4, 128, "f16", True, 0, [1400, 650], False, 4.0),
]


@pytest.mark.parametrize("name,B,Sq,Skv,Hq,Hkv,D,dtype,causal,window,lens,sinks,k_mult", CASES,
                         ids=[c[0] for c in CASES])
def test_split_prefill_matches_oracle(torch_gpu, name, B, Sq, Skv, Hq, Hkv, D, dtype, causal,
                                      window, lens, sinks, k_mult):
    _say("split prefill", name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype, mult=k_mult)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    sk = rng.normal(size=Hq).astype(np.float32) * 2 if sinks else None
    runs, (o1, l1) = _split_runs(torch_gpu, q, k, v, dtype, causal=causal, scale=scale,
                                 window=window, lens=lens, sinks=sk)
    for a, b in zip(runs[0], runs[1]):
        assert a.tobytes() == b.tobytes()
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype=dtype,
                         kv_lens=None if lens is None else np.asarray(lens),
                         window=window, sink_logits=sk)
    _check(*runs[0], ref)
    _check(o1, l1, ref)


@pytest.mark.parametrize("cfg", [inputs.FEW_HEADS_PREFILL], ids=lambda c: c.name)
def test_split_prefill_full_size(torch_gpu, cfg):
    """The benchmark's split prompt in the benchmark's launch: byte-identical
    repeats, and against the oracle the first, the last and one drawn row of
    every 128-row query block (split and whole blocks alike) plus boundary
    rows, over all 8 heads (~200 rows; ~2 s of oracle time on 8 host cores)."""
    _say("split prefill full size", cfg.name)
    x = inputs.make_prefill_inputs(cfg)
    runs, _ = _split_runs(torch_gpu, x["q"], x["k"], x["v"], cfg.dtype, causal=cfg.causal,
                          scale=cfg.scale, window=cfg.window)
    for a, b in zip(runs[0], runs[1]):
        assert a.tobytes() == b.tobytes()
    S = cfg.seqlen_q
    rng = np.random.default_rng(cfg.seed)
    rows = {0, 1, 127, 128, S // 2, S - 129, S - 128, S - 65, S - 64, S - 2, S - 1}
    for b0 in range(0, S, 128):
        b1 = min(S, b0 + 128) - 1
        rows |= {b0, b1, int(rng.integers(b0, b1 + 1))}
    rows = sorted(rows)
    ref = oracle.prefill(x["q"], x["k"], x["v"], scale=cfg.scale, causal=cfg.causal,
                         dtype=cfg.dtype, rows=rows, window=cfg.window)
    _check(*runs[0], ref, rows=rows)


def test_one_call_prefill_with_split_workspace(torch_gpu):
    """fa.prefill(..., split_workspace=...) runs the V repack and the split
    attention: the same bytes as the two calls made separately."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    _say("one-call prefill with split workspace")
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D, dtype = 1, 1000, 8, 8, 64, "f16"
    q = _dev(torch, inputs.draw_half(rng, (B, S, Hq, D), dtype), dtype)
    k = _dev(torch, inputs.draw_half(rng, (B, S, Hkv, D), dtype), dtype)
    v = _dev(torch, inputs.draw_half(rng, (B, S, Hkv, D), dtype), dtype)
    assert fa.prefill_split_units(B, S, S, Hq, Hkv, D, True, 0)
    sws = torch.zeros(fa.prefill_split_workspace_size(B, S, Hq, D), dtype=torch.uint8,
                      device="cuda")
    o1, l1 = fa.prefill(q, k, v, split_workspace=sws)
    o2, l2 = fa.prefill_packed(q, k, fa.prefill_pack_v(v), split_workspace=sws)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()


def test_split_workspace_reused_across_shapes(torch_gpu):
    """One split workspace, zero-filled once, serves calls of different shapes
    and inputs: a small shape, a larger one, then the small one again with new
    inputs. The counters live in a fixed region at the start of the buffer, so
    no call's partial results land on another shape's counters; every call is
    checked against the oracle (none is the first call on a fresh buffer) and
    all counters are zero after each call."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    _say("split workspace reused across shapes")
    shapes = [  # B, S, Hq, Hkv, D, dtype
        (1, 1000, 8, 8, 64, "f16"),
        (1, 4096, 8, 4, 128, "bf16"),
        (1, 1000, 8, 8, 64, "f16"),
    ]
    size = max(fa.prefill_split_workspace_size(B, S, Hq, D) for B, S, Hq, _, D, _ in shapes)
    assert size >= 65536
    sws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for i, (B, S, Hq, Hkv, D, dtype) in enumerate(shapes):
        assert fa.prefill_split_units(B, S, S, Hq, Hkv, D, True, 0), "planner must split"
        rng = np.random.default_rng(100 + i)
        q = inputs.draw_half(rng, (B, S, Hq, D), dtype)
        k = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
        v = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
        scale = float(np.float32(1 / np.sqrt(D)))
        o, lse = fa.prefill_packed(_dev(torch, q, dtype), _dev(torch, k, dtype),
                                   fa.prefill_pack_v(_dev(torch, v, dtype)), causal=True,
                                   softmax_scale=scale, split_workspace=sws)
        torch.cuda.synchronize()
        assert int(sws[:65536].view(torch.int32).abs().sum().item()) == 0, \
            f"arrival counters not back at zero after call {i}"
        # every row of the small shape; the last two blocks (split) and samples of the large one
        rows = None if S <= 1000 else sorted({0, 1, 127, 128, S // 2} | set(range(S - 256, S)))
        ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, rows=rows)
        _check(o.cpu().numpy(), lse.cpu().numpy(), ref, rows=rows)
