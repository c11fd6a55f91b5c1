"""Parity of the head_dim 512 prefill (the two waves of a pair split the head
dimension) against the fp64 oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", D1.4 (a 512-wide head does not
fit the on-chip budget of the narrower kernels; the contraction dimension is
split). Same gate as every prefill: |O| error <= 2e-3, natural-log LSE error
<= 1e-4, byte-identical repeats.
"""
import numpy as np
import pytest

import oracle
from flashattention_attention_amd import inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-4
D = 512


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


def _run(torch, q, k, v, dtype, *, causal, scale, unnorm=False, lens=None, window=0,
         sinks=None):
    from flashattention_attention_amd import fa
    B, Sq, Hq, _ = q.shape
    out = torch.full((B, Sq, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    rs = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    fa.prefill(_dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype),
               causal=causal, softmax_scale=scale, out_unnormalized=unnorm, out=out, lse=lse,
               row_sum=rs,
               kv_lens=None if lens is None else torch.tensor(lens, dtype=torch.int32,
                                                              device="cuda"),
               window=window,
               sink_logits=None if sinks is None else torch.tensor(
                   np.asarray(sinks, np.float32), device="cuda"))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), rs.cpu().numpy()


def _check(o, lse, rs, ref, unnorm=False, rows=None):
    if rows is not None:
        o, lse, rs = o[:, rows], lse[:, :, rows], rs[:, :, rows]
    assert np.isfinite(o).all() and not np.isnan(lse).any()
    if unnorm:
        err_rs = np.abs(np.log(rs.astype(np.float64)) - np.log(ref["row_sum"])).max()
        assert err_rs <= LSE_TOL, err_rs
        o = o / np.transpose(rs, (0, 2, 1))[..., None]
    fin = np.isfinite(ref["lse"])
    assert (np.isneginf(lse) == ~fin).all()
    err_o = np.abs(o - ref["o"]).max()
    err_l = np.abs(lse[fin] - ref["lse"][fin]).max(initial=0.0)
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"


# (B, Sq, Skv, Hq, Hkv, dtype, causal, unnorm)
SWEEP = [
    (1, 1, 1, 2, 1, "bf16", True, False),
    (1, 31, 31, 2, 2, "f16", True, False),
    (1, 33, 33, 3, 1, "bf16", True, False),
    (1, 129, 129, 4, 1, "f16", True, False),
    (2, 100, 300, 4, 2, "bf16", True, False),     # Sq < Skv: bottom-right alignment
    (1, 200, 200, 2, 2, "bf16", False, False),    # unmasked
    (1, 1, 777, 8, 1, "f16", True, False),        # one query row, long KV
    (1, 300, 300, 4, 4, "bf16", True, True),      # un-normalized
    (2, 257, 257, 8, 1, "f16", True, False),      # multi-query, group 8
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,dtype,causal,unnorm", SWEEP)
def test_hd512_sweep(torch_gpu, B, Sq, Skv, Hq, Hkv, dtype, causal, unnorm):
    _say("hd512", B, Sq, Skv, Hq, Hkv, dtype, causal, unnorm)
    rng = np.random.default_rng(Sq * 31 + Skv + Hq)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype, mult=4.0 if unnorm else 1.0)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype=dtype)
    o, lse, rs = _run(torch_gpu, q, k, v, dtype, causal=causal, scale=scale, unnorm=unnorm)
    _check(o, lse, rs, ref, unnorm)


def test_hd512_masks_and_sinks(torch_gpu):
    _say("hd512 masks+sinks")
    B, S, Hq, Hkv, dtype = 2, 230, 4, 1, "bf16"
    rng = np.random.default_rng(512)
    q = inputs.draw_half(rng, (B, S, Hq, D), dtype)
    k, v = (inputs.draw_half(rng, (B, S, Hkv, D), dtype) for _ in range(2))
    scale = float(np.float32(1 / np.sqrt(D)))
    lens, window, sinks = [230, 90], 70, [0.5, -1.0, 4.0, 0.0]
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, kv_lens=lens,
                         window=window)
    o, lse, rs = _run(torch_gpu, q, k, v, dtype, causal=True, scale=scale, lens=lens,
                      window=window)
    _check(o, lse, rs, ref)
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, kv_lens=lens,
                         window=window, sink_logits=np.asarray(sinks, np.float32))
    o, lse, rs = _run(torch_gpu, q, k, v, dtype, causal=True, scale=scale, lens=lens,
                      window=window, sinks=sinks)
    _check(o, lse, rs, ref)


def test_hd512_packed_matches_fused(torch_gpu):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    _say("hd512 packed")
    B, Sq, Skv, Hq, Hkv, dtype = 1, 150, 333, 4, 2, "f16"
    rng = np.random.default_rng(77)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k, v = (inputs.draw_half(rng, (B, Skv, Hkv, D), dtype) for _ in range(2))
    scale = float(np.float32(1 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    ws = fa.prefill_pack_v(vd)
    o1, l1 = fa.prefill_packed(qd, kd, ws, causal=True, softmax_scale=scale)
    o2, l2 = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()


def test_hd512_full_size(torch_gpu):
    """The 4096-token multi-query workload at head_dim 512, in the configuration
    the benchmark times: sampled rows against the oracle (one inside every
    128-row block, so every work-group of the serial order, half of which
    walk their key tiles backwards, is checked), repeat identity."""
    cfg = inputs.HD512_PREFILL
    _say(cfg.name)
    x = inputs.make_prefill_inputs(cfg)
    runs = [_run(torch_gpu, x["q"], x["k"], x["v"], cfg.dtype, causal=True, scale=cfg.scale)
            for _ in range(2)]
    for a, b in zip(runs[0], runs[1]):
        assert a.tobytes() == b.tobytes()
    rng = np.random.default_rng(cfg.seed)
    S = cfg.seqlen_q
    rows = sorted({0, 1, 31, 32, 127, 128, 129, S // 2, S - 129, S - 128, S - 2, S - 1}
                  | set(rng.integers(0, S, 6).tolist())
                  | {qb * 128 + 61 for qb in range(-(-S // 128))})
    ref = oracle.prefill(x["q"], x["k"], x["v"], scale=cfg.scale, causal=True, dtype=cfg.dtype,
                         rows=rows)
    o, lse, rs = runs[0]
    _check(o, lse, rs, ref, rows=rows)
