"""Parity of the prefill masks (per-sequence KV length, sliding window) against
the fp64 oracle (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", D3 (a per-sequence valid
length hides the keys past it) and D4 (the causal comparison applied on the
windowed branch). Same gate as the unmasked prefill: |O| error <= 2e-3 and
natural-log LSE error <= 1e-4 on every row that sees at least one key; rows
that see none must come back exactly as O = 0, row_sum = 0, LSE = -inf.
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


def _lens_dev(torch, lens):
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")


def _run(torch, q, k, v, dtype, causal, scale, lens, window, unnorm=False):
    from flashattention_attention_amd import fa
    B, Sq, Hq, D = q.shape
    out = torch.full((B, Sq, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    rs = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    fa.prefill(_dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype),
               causal=causal, softmax_scale=scale, out_unnormalized=unnorm, out=out, lse=lse,
               row_sum=rs, kv_lens=_lens_dev(torch, lens), window=window)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), rs.cpu().numpy()


def _check(o, lse, rs, ref, unnorm=False):
    """Tolerance on rows with a visible key; exact zeros / -inf on the others.
    rs may be None when the row sums were not asked for."""
    empty = np.isneginf(ref["lse"])                       # [B, Hq, R]
    empty_o = np.transpose(empty, (0, 2, 1))              # [B, R, Hq]
    assert (o[empty_o] == 0).all() and np.isneginf(lse[empty]).all()
    full = ~empty
    assert np.isfinite(lse[full]).all() and np.isfinite(o).all()
    if rs is not None:
        assert (rs[empty] == 0).all() and np.isfinite(rs).all()
    got_o = o[~empty_o]
    if unnorm:
        got_o = got_o / np.transpose(rs, (0, 2, 1))[~empty_o][:, None]
        err_rs = np.abs(np.log(rs[full].astype(np.float64)) - np.log(ref["row_sum"][full]))
        assert err_rs.max(initial=0.0) <= LSE_TOL
    err_o = np.abs(got_o - ref["o"][~empty_o]).max(initial=0.0)
    err_l = np.abs(lse[full] - ref["lse"][full]).max(initial=0.0)
    assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
    return int(empty.sum())


# (B, Sq, Skv, Hq, Hkv, D, dtype, causal, kv_lens, window, unnorm)
CASES = [
    (3, 200, 200, 8, 2, 128, "bf16", True, [200, 137, 64], 0, False),   # lengths, paired heads
    (2, 150, 150, 7, 1, 128, "f16", True, None, 50, False),             # window, odd group
    (2, 100, 300, 4, 4, 64, "bf16", True, [250, 300], 64, False),       # both, Sq < Skv
    (1, 260, 260, 4, 2, 256, "bf16", True, None, 33, False),            # window, large head
    (2, 129, 129, 6, 2, 64, "f16", False, [1, 70], 0, False),           # lengths, unmasked
    (2, 64, 200, 4, 2, 128, "bf16", False, None, 100, False),           # window, unmasked
    (1, 200, 200, 4, 2, 128, "bf16", True, [120], 30, False),           # rows with no key
    (2, 100, 200, 4, 2, 128, "f16", True, [0, 50], 0, False),           # an empty sequence
    (2, 90, 100, 4, 2, 64, "bf16", True, [500, -3], 0, False),          # clamped lengths
    (2, 300, 300, 4, 2, 256, "bf16", True, [300, 211], 77, True),       # un-normalized
    (1, 333, 333, 8, 4, 128, "f16", True, [301], 129, True),            # un-normalized, pairs
    (1, 70, 70, 8, 2, 128, "f16", True, None, 1, False),                # window of one key
    (2, 1000, 1000, 4, 1, 128, "bf16", True, [1000, 777], 256, False),  # many tiles skipped
]


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,dtype,causal,lens,window,unnorm", CASES)
def test_prefill_masks(torch_gpu, B, Sq, Skv, Hq, Hkv, D, dtype, causal, lens, window, unnorm):
    _say("masks", B, Sq, Skv, Hq, Hkv, D, dtype, causal, lens, window, unnorm)
    rng = np.random.default_rng(Sq * 7 + Skv + D + window)
    q = inputs.draw_half(rng, (B, Sq, Hq, D), dtype)
    k = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype, mult=4.0 if unnorm else 1.0)
    v = inputs.draw_half(rng, (B, Skv, Hkv, D), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    clamped = None if lens is None else [min(max(x, 0), Skv) for x in lens]
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype=dtype, kv_lens=clamped,
                         window=window)
    o, lse, rs = _run(torch_gpu, q, k, v, dtype, causal, scale, lens, window, unnorm)
    _check(o, lse, rs, ref, unnorm)
    if window == 1 and causal and lens is None:
        # each row sees only its own position: O is that key's V row (up to
        # the fp32 rounding of the one weight against the row sum)
        pos = np.arange(Sq) + Skv - Sq
        vv = inputs.half_bits_to_f32(v, dtype)[:, pos]               # [B, Sq, Hkv, D]
        np.testing.assert_allclose(o, np.repeat(vv, Hq // Hkv, axis=2), rtol=1e-6, atol=1e-6)


def test_prefill_masks_reduce_to_unmasked(torch_gpu):
    """kv_lens = seqlen_kv everywhere and a window wider than the cache change
    nothing: the outputs are byte-identical to the unmasked call."""
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype = 2, 300, 8, 2, 128, "bf16"
    _say("masks-identity", B, S, Hq, Hkv, D)
    rng = np.random.default_rng(5)
    q, k, v = (inputs.draw_half(rng, (B, S, h, D), dtype) for h in (Hq, Hkv, Hkv))
    scale = float(np.float32(1 / np.sqrt(D)))
    base = _run(torch, q, k, v, dtype, True, scale, None, 0)
    for lens, window in (([S, S], 0), (None, S), ([S + 9, S], S + 100)):
        got = _run(torch, q, k, v, dtype, True, scale, lens, window)
        for a, b in zip(base, got):
            assert a.tobytes() == b.tobytes(), (lens, window)


def test_prefill_padding_is_ignored(torch_gpu):
    """Keys past kv_lens[b] and outside the window may hold any finite values:
    changing them leaves the outputs byte-identical."""
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype = 2, 260, 4, 2, 128, "f16"
    lens, window = [200, 131], 90
    _say("masks-padding", B, S, lens, window)
    rng = np.random.default_rng(11)
    q, k, v = (inputs.draw_half(rng, (B, S, h, D), dtype) for h in (Hq, Hkv, Hkv))
    scale = float(np.float32(1 / np.sqrt(D)))
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(lens):
        k2[b, L:] = inputs.draw_half(rng, k2[b, L:].shape, dtype, mult=4.0)
        v2[b, L:] = inputs.draw_half(rng, v2[b, L:].shape, dtype, mult=4.0)
    a = _run(torch, q, k, v, dtype, True, scale, lens, window)
    b_ = _run(torch, q, k2, v2, dtype, True, scale, lens, window)
    for x, y in zip(a, b_):
        assert x.tobytes() == y.tobytes()


@pytest.mark.parametrize("D,hq,hkv,dtype", [(128, 28, 4, "bf16"), (64, 6, 3, "f16")])
def test_prefill_packed_masks_match_fused(torch_gpu, D, hq, hkv, dtype):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, Sq, Skv, lens, window = 2, 150, 400, [400, 233], 120
    _say("masks-packed", D, hq, hkv, dtype)
    rng = np.random.default_rng(D * 3 + hq)
    q = inputs.draw_half(rng, (B, Sq, hq, D), dtype)
    k, v = (inputs.draw_half(rng, (B, Skv, hkv, D), dtype) for _ in range(2))
    scale = float(np.float32(1 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    ld = _lens_dev(torch, lens)
    ws = fa.prefill_pack_v(vd)
    o1, l1 = fa.prefill_packed(qd, kd, ws, causal=True, softmax_scale=scale, kv_lens=ld,
                               window=window)
    o2, l2 = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale, kv_lens=ld, window=window)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, kv_lens=lens,
                         window=window)
    _check(o1.cpu().numpy(), l1.cpu().numpy(), None, ref)
