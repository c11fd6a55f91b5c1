"""Parity of the decode form that runs on the matrix cores (two or more query
heads per wave, head_dim <= 128) against the fp64 oracle (needs an MI355X):
Q.K^T and P.V on 16x16x32 MFMAs, K and V rows through LDS, V^T by transposing
LDS reads (bf16 V converted to fp16 for the P.V after them).

Source: "66 · D2: explicit K+V register staging ...", section 3.2 (per-block
online update) and "STAGE_D.md — FMHA Kernel Development", section D2 (several
query heads packed on one K/V stream). Same gate as every decode test: |O|
error <= 2e-3, natural-log LSE error <= 1e-4, byte-identical repeats.

The shapes of the matrix-core cases are sized so that the heads-per-wave rule
takes the whole GQA group (the call spans more than one round of resident
waves at any smaller divisor): 8 sequences x ceil(max_len / split_len) splits
x (Hq / g) waves > 2048 for every divisor g below the group. The last test
checks that head-major caches (any kv_stride_head / kv_stride_tok) give the
same bytes as token-major ones, in both decode forms.
"""
import numpy as np
import pytest

import oracle
from flashattention_attention_amd import inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-4
SLOTS = 256 * 8          # resident decode waves at head_dim <= 128


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


def _heads_per_wave(group, batch, hq, max_splits):
    """The library's rule (a pure function of the shape), restated."""
    gmax = max(g for g in range(1, 9) if group % g == 0)
    for g in range(1, gmax):
        if group % g == 0 and batch * (hq // g) * max_splits <= SLOTS:
            return g
    return gmax


# (dtype, D, Hq, Hkv, split_len, k_mult)
CASES = [
    ("f16", 128, 32, 4, 32, 1.0),     # 8 heads per wave
    ("bf16", 128, 28, 4, 32, 4.0),    # 7, large scores (the running max moves)
    ("f16", 64, 24, 4, 32, 1.0),      # 6
    ("bf16", 64, 40, 8, 16, 4.0),     # 5
    ("bf16", 128, 40, 8, 48, 1.0),    # 5
    ("f16", 128, 64, 8, 32, 4.0),     # 8 (a group of 8 out of 64 heads)
    ("f16", 128, 32, 8, 16, 1.0),     # 4: fp16 takes P.V on the matrix cores from 4
    ("f16", 64, 16, 4, 32, 4.0),      # 4
    ("bf16", 128, 24, 8, 16, 4.0),    # 3
    ("f16", 128, 16, 8, 16, 1.0),     # 2
    ("f16", 64, 16, 8, 16, 1.0),      # 2
]


@pytest.mark.parametrize("dtype,D,hq,hkv,split_len,k_mult", CASES)
def test_decode_matrix_core_form(torch_gpu, dtype, D, hq, hkv, split_len, k_mult):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    rng = np.random.default_rng(D * 7 + hq + split_len)
    # ragged lengths, a single-key sequence and one of exactly one block
    lens = np.array([1, 17, 32, 333, 700, 1000, 1231, 1300], np.int32)
    B = len(lens)
    max_splits = -(-int(lens.max()) // split_len)
    g = _heads_per_wave(hq // hkv, B, hq, max_splits)
    assert g >= 2, g
    _say("mfma decode", dtype, D, hq, hkv, split_len, k_mult, "heads/wave", g)
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    T = int(lens.sum())
    q = inputs.draw_half(rng, (B, hq, D), dtype)
    kc = inputs.draw_half(rng, (T, hkv, D), dtype, mult=k_mult)
    vc = inputs.draw_half(rng, (T, hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    dx = (_dev(torch, q, dtype), _dev(torch, kc, dtype), _dev(torch, vc, dtype),
          torch.from_numpy(offs).cuda(), torch.from_numpy(lens).cuda())
    ref = oracle.decode(q, kc, vc, offs, lens, scale=scale, dtype=dtype)

    runs = []
    for _ in range(2):
        o, lse = fa.decode(*dx, split_len=split_len, max_splits=max_splits, softmax_scale=scale)
        of, lsef = fa.decode_fused(*dx, split_len=split_len, max_splits=max_splits,
                                   softmax_scale=scale)
        torch.cuda.synchronize()
        runs.append(tuple(t.cpu().numpy() for t in (o, lse, of, lsef)))
    for a, b in zip(runs[0], runs[1]):
        assert a.tobytes() == b.tobytes()
    o, lse, of, lsef = runs[0]
    for got_o, got_l in ((o, lse), (of, lsef)):
        assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
        err_o = np.abs(got_o - ref["o"]).max()
        err_l = np.abs(got_l - ref["lse"]).max()
        assert err_o <= O_TOL and err_l <= LSE_TOL, f"O err {err_o:.3e}, LSE err {err_l:.3e}"
    # the single-key sequence returns its one V row for every head of the group,
    # up to rounding: with P.V on the matrix cores the weight enters as fp16
    # while the row sum keeps the fp32 weight 2^(x + 6), x the rounded
    # difference between the score and the base (|x| <= 2^-20 for scores
    # below 32 in log2 units), so the two differ by < 1.5e-6 relative
    hk_of = np.arange(hq) // (hq // hkv)
    v0 = inputs.half_bits_to_f32(vc[0], dtype)[hk_of]
    np.testing.assert_allclose(o[0], v0, atol=1e-6, rtol=4e-6)


@pytest.mark.parametrize("dtype,D,hq,hkv,split_len,want_g", [
    ("f16", 128, 28, 4, 32, 7),     # matrix-core form
    ("f16", 128, 32, 8, 32, 4),     # matrix-core form, 4 heads per wave
    ("bf16", 128, 32, 8, 32, 4),    # matrix-core form, bf16, 4 heads per wave
    ("bf16", 64, 8, 8, 48, 1),      # VALU form, bf16, one head per wave
    ("f16", 64, 8, 8, 48, 1),       # VALU form, one head per wave
])
def test_decode_head_major_caches(torch_gpu, dtype, D, hq, hkv, split_len, want_g):
    """Caches stored head-major ([Hkv, T, D], passed through kv_stride_head = T*D
    and kv_stride_tok = D) give byte-identical results to the token-major ones:
    the kernels read the same values in the same order."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    rng = np.random.default_rng(D + hq * 3 + split_len)
    lens = np.array([1, 17, 32, 333, 700, 1000, 1231, 1300], np.int32)
    B = len(lens)
    max_splits = -(-int(lens.max()) // split_len)
    assert _heads_per_wave(hq // hkv, B, hq, max_splits) == want_g
    _say("head-major caches", dtype, D, hq, hkv, split_len)
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    T = int(lens.sum())
    q = inputs.draw_half(rng, (B, hq, D), dtype)
    kc = inputs.draw_half(rng, (T, hkv, D), dtype)
    vc = inputs.draw_half(rng, (T, hkv, D), dtype)
    scale = float(np.float32(1 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, kc, dtype), _dev(torch, vc, dtype)
    khm, vhm = (t.permute(1, 0, 2).contiguous().permute(1, 0, 2) for t in (kd, vd))
    assert khm.stride() == (D, T * D, 1)
    od, ld = torch.from_numpy(offs).cuda(), torch.from_numpy(lens).cuda()
    outs = []
    for k, v in ((kd, vd), (khm, vhm)):
        o, lse = fa.decode(qd, k, v, od, ld, split_len=split_len, max_splits=max_splits,
                           softmax_scale=scale)
        of, lsef = fa.decode_fused(qd, k, v, od, ld, split_len=split_len,
                                   max_splits=max_splits, softmax_scale=scale)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (o, lse, of, lsef)])
    for a, b in zip(*outs):
        assert a.tobytes() == b.tobytes()
    ref = oracle.decode(q, kc, vc, offs, lens, scale=scale, dtype=dtype)
    assert np.abs(outs[1][0] - ref["o"]).max() <= O_TOL
    assert np.abs(outs[1][1] - ref["lse"]).max() <= LSE_TOL
