"""Pins that tie the fp64 oracle to facts other than itself (CPU only).

Each test names the property it checks and the passage that fixes it. The
oracle is the parity authority for the HIP path, so a plausible mistake in it
(dropped scale, wrong mask direction or offset, wrong GQA head map, transposed
operand, missing normalization, log base, merge weights) must fail one of them.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from flashattention_attention_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_half(rng, shape, dtype="f16", mult=1.0):
    return inputs.draw_half(rng, shape, dtype, mult=mult)


def _f(bits, dtype="f16"):
    """Independent half decoding for the tests (struct-free, via numpy)."""
    return inputs.half_bits_to_f32(bits, dtype).astype(np.float64)


# --------------------------------------------------------------------------
# Half decoding: known bit patterns (IEEE binary16; bfloat16 = top half of fp32)
# --------------------------------------------------------------------------

def test_half_decoding_known_patterns():
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x7BFF: 65504.0,
           0x3555: 0.333251953125, 0x0400: 2.0 ** -14}
    bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0080: 2.0 ** -126,
            0x3EAB: 0.333984375}
    for bits, val in f16.items():
        assert oracle.half_to_f64(np.array([bits], np.uint16), "f16")[0] == val
    for bits, val in bf16.items():
        assert oracle.half_to_f64(np.array([bits], np.uint16), "bf16")[0] == val


def test_bf16_rounding_is_nearest_even():
    one_half_ulp = np.float32(1.0 + 2.0 ** -8)            # tie between 1 and 1+2^-7
    three_half_ulp = np.float32(1.0 + 3 * 2.0 ** -8)      # tie between 1+2^-7 and 1+2^-6
    above = np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20)
    bits = inputs.round_f32_to_half_bits(np.array([one_half_ulp, three_half_ulp, above]), "bf16")
    assert list(bits) == [0x3F80, 0x3F82, 0x3F81]


# --------------------------------------------------------------------------
# Worked example (hand-derived closed forms; tests/golden)
# --------------------------------------------------------------------------

def _closed(expr):
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log1p": math.log1p}))


def test_worked_example_two_keys():
    with open(os.path.join(GOLDEN, "worked_example_two_keys.json")) as fh:
        ex = json.load(fh)
    to_bits = lambda a: inputs.round_f32_to_half_bits(np.array(a, np.float32), "f16")
    q = to_bits(ex["q"]).reshape(1, 2, 1, 2)
    k = to_bits(ex["k"]).reshape(1, 2, 1, 2)
    v = to_bits(ex["v"]).reshape(1, 2, 1, 2)
    for mode, causal in (("causal", True), ("unmasked", False)):
        r = oracle.prefill(q, k, v, scale=ex["scale"], causal=causal, dtype="f16")
        want = ex[mode]
        for i in range(2):
            assert r["lse"][0, 0, i] == pytest.approx(_closed(want["lse"][i]), abs=1e-15)
            for d in range(2):
                assert r["o"][0, i, 0, d] == pytest.approx(_closed(want["o"][i][d]), abs=1e-15)
            if "row_sum" in want:
                assert r["row_sum"][0, 0, i] == pytest.approx(_closed(want["row_sum"][i]),
                                                              abs=1e-15)


# --------------------------------------------------------------------------
# P-1: online softmax over key tiles equals the two-pass definition
# ("60 · r57 ...", §2.3 tile-end rescale; "66 · D2 ...", §3.2 per-row update)
# --------------------------------------------------------------------------

def _online_attention(qf, kf, vf, scale, q_pos, boundaries):
    """Online softmax over consecutive key tiles; written here independently."""
    R, D = qf.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, D))
    for lo, hi in zip(boundaries[:-1], boundaries[1:]):
        s = np.einsum("rd,jd->rj", qf, kf[lo:hi]) * scale
        if q_pos is not None:
            s[np.arange(lo, hi)[None, :] > q_pos[:, None]] = -np.inf
        tile_max = s.max(axis=1)
        m_new = np.maximum(m, tile_max)
        live = np.isfinite(m_new)
        corr = np.where(live, np.exp(np.where(live, m - m_new, 0.0)), 1.0)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = l * corr + p.sum(axis=1)
        acc = acc * corr[:, None] + p @ vf[lo:hi]
        m = m_new
    return acc / l[:, None], m + np.log(l)


@pytest.mark.parametrize("tile", [1, 7, 32, 64, 128, "random"])
@pytest.mark.parametrize("sq,skv,causal", [(150, 150, True), (37, 150, True), (20, 97, False)])
def test_online_equals_two_pass(tile, sq, skv, causal):
    rng = np.random.default_rng(11)
    D = 24
    q, k, v = (_rand_half(rng, (1, s, 1, D)) for s in (sq, skv, skv))
    scale = float(np.float32(1 / math.sqrt(D)))
    ref = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16")
    if tile == "random":
        cuts = sorted(set(rng.integers(1, skv, 9).tolist()))
        bounds = [0] + cuts + [skv]
    else:
        bounds = list(range(0, skv, tile)) + [skv]
    q_pos = np.arange(sq) + (skv - sq) if causal else None
    o, lse = _online_attention(_f(q[0, :, 0]), _f(k[0, :, 0]), _f(v[0, :, 0]), scale, q_pos,
                               bounds)
    np.testing.assert_allclose(ref["o"][0, :, 0], o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["lse"][0, 0], lse, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# P-2: all scores tie (Q = 0): LSE_i = ln(n_i) exactly; O_i = mean of visible V
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sq,skv,hq,hkv", [(64, 64, 4, 2), (10, 50, 3, 1), (1, 33, 2, 2)])
def test_tied_scores_closed_form(sq, skv, hq, hkv):
    rng = np.random.default_rng(5)
    D = 16
    q = np.zeros((2, sq, hq, D), np.uint16)           # +0.0 bit pattern
    k = _rand_half(rng, (2, skv, hkv, D))
    v = _rand_half(rng, (2, skv, hkv, D))
    r = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="f16")
    n = np.arange(sq) + (skv - sq) + 1                # visible keys per row (bottom-right)
    vf = _f(v)
    running_sum = np.zeros((2, hkv, D))
    means = np.zeros((2, skv, hkv, D))
    for j in range(skv):                              # independent prefix means
        running_sum += vf[:, j]
        means[:, j] = running_sum / (j + 1)
    for h in range(hq):
        hk = h // (hq // hkv)
        np.testing.assert_allclose(r["lse"][:, h, :], np.broadcast_to(np.log(n), (2, sq)),
                                   rtol=0, atol=1e-15)
        np.testing.assert_array_equal(r["row_sum"][:, h, :],
                                      np.broadcast_to(n.astype(float), (2, sq)))
        np.testing.assert_allclose(r["o"][:, :, h, :], means[:, n - 1, hk, :], rtol=1e-13,
                                   atol=1e-14)


def test_tied_scores_constant_v_is_exact():
    D = 8
    q = np.zeros((1, 40, 1, D), np.uint16)
    rng = np.random.default_rng(3)
    k = _rand_half(rng, (1, 40, 1, D))
    row = _rand_half(rng, (D,))
    v = np.broadcast_to(row, (1, 40, 1, D)).copy()
    r = oracle.prefill(q, k, v, scale=1.0, causal=True, dtype="f16")
    # equal weights summing to one on identical rows give that row up to the
    # rounding of 1/n weights; the exact definition is the row itself
    np.testing.assert_allclose(r["o"][0, :, 0, :], np.broadcast_to(_f(row), (40, D)),
                               rtol=1e-15, atol=0)


# --------------------------------------------------------------------------
# P-3: one visible key returns that key's V row; LSE is its exact score
# (sections D3/D4 mask comparator; decode at KV length 1)
# --------------------------------------------------------------------------

def _exact_score(qrow, krow, scale):
    s = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qrow, krow))
    return float(Fraction(scale) * s)


def test_single_visible_key_prefill_row0():
    rng = np.random.default_rng(7)
    for dtype in ("f16", "bf16"):
        q = _rand_half(rng, (2, 16, 4, 32), dtype)
        k = _rand_half(rng, (2, 16, 2, 32), dtype)
        v = _rand_half(rng, (2, 16, 2, 32), dtype)
        scale = float(np.float32(0.1767767))
        r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype)
        for b in range(2):
            for h in range(4):
                hk = h // 2
                assert np.array_equal(r["o"][b, 0, h], _f(v[b, 0, hk], dtype))
                exact = _exact_score(_f(q[b, 0, h], dtype), _f(k[b, 0, hk], dtype), scale)
                assert r["lse"][b, h, 0] == pytest.approx(exact, rel=1e-14, abs=1e-14)
                assert r["row_sum"][b, h, 0] == 1.0


def test_single_key_decode():
    rng = np.random.default_rng(8)
    q = _rand_half(rng, (3, 6, 16))
    kc = _rand_half(rng, (3, 2, 16))
    vc = _rand_half(rng, (3, 2, 16))
    lens = np.array([1, 1, 1], np.int32)
    offs = np.array([0, 1, 2], np.int64)
    r = oracle.decode(q, kc, vc, offs, lens, scale=0.25, dtype="f16")
    for b in range(3):
        for h in range(6):
            hk = h // 3
            assert np.array_equal(r["o"][b, h], _f(vc[b, hk]))
            exact = _exact_score(_f(q[b, h]), _f(kc[b, hk]), 0.25)
            assert r["lse"][b, h] == pytest.approx(exact, rel=1e-14, abs=1e-14)


# --------------------------------------------------------------------------
# P-4: merging split partials by LSE equals the unsplit result
# ("66 · D2 ...", §1 split ranges; "STAGE_D.md ...", D5 merge by LSE)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("split_len", [1, 29, 52, 512, 1641])
def test_merge_equals_unsplit(split_len):
    rng = np.random.default_rng(100 + split_len)
    lens = np.array([1, 29, 52, 512, 1641], np.int32)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    hq, hkv, D = 2, 1, 8
    q = _rand_half(rng, (5, hq, D))
    kc = _rand_half(rng, (total, hkv, D), mult=4.0)   # peaked rows stress the weights
    vc = _rand_half(rng, (total, hkv, D))
    max_splits = int(oracle.num_splits(lens.max(), split_len)) + 2   # room for empty splits
    parts = oracle.decode_split_partials(q, kc, vc, offs, lens, scale=0.35, split_len=split_len,
                                         max_splits=max_splits, dtype="f16")
    assert np.all(np.isneginf(parts["part_lse"][:, :, -1]))      # empty splits
    merged = oracle.merge_partials(parts["part_o"], parts["part_lse"], parts["n_splits"])
    full = oracle.decode(q, kc, vc, offs, lens, scale=0.35, dtype="f16")
    np.testing.assert_allclose(merged["o"], full["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(merged["lse"], full["lse"], rtol=1e-12, atol=1e-12)


def test_merge_of_one_split_is_identity():
    rng = np.random.default_rng(9)
    po = rng.standard_normal((2, 3, 4, 5))
    pl = rng.standard_normal((2, 3, 4)) * 50
    r = oracle.merge_partials(po, pl, np.array([1, 1]))
    np.testing.assert_array_equal(r["o"], po[:, :, 0])
    np.testing.assert_array_equal(r["lse"], pl[:, :, 0])


def test_merge_large_lse_no_overflow():
    po = np.stack([np.full((1, 1, 4), 1.0), np.full((1, 1, 4), 3.0)], axis=2)
    pl = np.array([[[1000.0, 1000.0 + math.log(3.0)]]])
    r = oracle.merge_partials(po, pl, np.array([2]))
    np.testing.assert_allclose(r["o"][0, 0], np.full(4, (1 * 1 + 3 * 3) / 4), rtol=1e-13)
    assert r["lse"][0, 0] == pytest.approx(1000.0 + math.log(4.0), rel=1e-15)


# --------------------------------------------------------------------------
# P-5: causal invariance -- keys past the query position cannot matter
# --------------------------------------------------------------------------

def test_causal_invariance_bitwise():
    rng = np.random.default_rng(12)
    q = _rand_half(rng, (1, 48, 2, 16))
    k = _rand_half(rng, (1, 48, 2, 16))
    v = _rand_half(rng, (1, 48, 2, 16))
    base = oracle.prefill(q, k, v, scale=0.25, causal=True, dtype="f16")
    for i in (0, 5, 31, 46):
        k2, v2 = k.copy(), v.copy()
        k2[0, i + 1:] = _rand_half(rng, k2[0, i + 1:].shape, mult=8.0)
        v2[0, i + 1:] = _rand_half(rng, v2[0, i + 1:].shape, mult=8.0)
        pert = oracle.prefill(q, k2, v2, scale=0.25, causal=True, dtype="f16")
        assert np.array_equal(base["o"][0, : i + 1], pert["o"][0, : i + 1])
        assert np.array_equal(base["lse"][0, :, : i + 1], pert["lse"][0, :, : i + 1])
        if i + 1 < 48:
            assert not np.array_equal(base["o"][0, i + 1], pert["o"][0, i + 1])


# --------------------------------------------------------------------------
# P-6: GQA equals MHA with every KV head repeated for its group of query heads
# ("60 · r57 ...", §2.2 KV-head addressing)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv", [(28, 4), (8, 8), (6, 1), (32, 8)])
def test_gqa_equals_repeated_mha(hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv)
    q = _rand_half(rng, (1, 12, hq, 8), "bf16")
    k = _rand_half(rng, (1, 12, hkv, 8), "bf16")
    v = _rand_half(rng, (1, 12, hkv, 8), "bf16")
    group = hq // hkv
    k_rep = np.repeat(k, group, axis=2)               # heads 0..g-1 -> kv 0, etc.
    v_rep = np.repeat(v, group, axis=2)
    a = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="bf16")
    b = oracle.prefill(q, k_rep, v_rep, scale=0.3, causal=True, dtype="bf16")
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    # the contiguous-group map, stated directly: query head h uses KV head h // group
    for h in range(hq):
        single = oracle.prefill(q[:, :, h:h + 1], k[:, :, h // group: h // group + 1],
                                v[:, :, h // group: h // group + 1], scale=0.3, causal=True,
                                dtype="bf16")
        assert np.array_equal(single["o"][:, :, 0], a["o"][:, :, h])


# --------------------------------------------------------------------------
# P-7: brute force on tiny shapes in 60-digit decimal arithmetic, using the
# unshifted form exp(s_j) / sum_k exp(s_k) and LSE = ln sum_j exp(s_j)
# --------------------------------------------------------------------------

def _decimal_attention(qf, kf, vf, scale, causal, sq, skv):
    getcontext().prec = 60
    D = qf.shape[1]
    sc = Decimal(scale)
    out_o = np.zeros((sq, vf.shape[1]))
    out_lse = np.zeros(sq)
    for i in range(sq):
        last = i + skv - sq if causal else skv - 1
        ex = []
        for j in range(last + 1):
            s = sum(Decimal(float(qf[i, d])) * Decimal(float(kf[j, d])) for d in range(D)) * sc
            ex.append(s.exp())
        tot = sum(ex)
        out_lse[i] = float(tot.ln())
        for d in range(vf.shape[1]):
            out_o[i, d] = float(sum(e * Decimal(float(vf[j, d])) for j, e in enumerate(ex)) / tot)
    return out_o, out_lse


@pytest.mark.parametrize("sq,skv,D,causal", [(1, 1, 1, True), (3, 5, 2, True), (8, 8, 8, True),
                                             (5, 7, 3, False), (6, 6, 4, False)])
def test_brute_force_decimal(sq, skv, D, causal):
    rng = np.random.default_rng(sq * 31 + skv * 7 + D)
    hq, hkv = 2, 1
    q = _rand_half(rng, (1, sq, hq, D))
    k = _rand_half(rng, (1, skv, hkv, D), mult=2.0)
    v = _rand_half(rng, (1, skv, hkv, D))
    scale = float(np.float32(0.7))
    r = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16")
    for h in range(hq):
        o, lse = _decimal_attention(_f(q[0, :, h]), _f(k[0, :, 0]), _f(v[0, :, 0]), scale,
                                    causal, sq, skv)
        np.testing.assert_allclose(r["o"][0, :, h], o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["lse"][0, h], lse, rtol=1e-13, atol=1e-14)


def test_two_key_closed_form():
    rng = np.random.default_rng(21)
    D = 16
    for _ in range(20):
        q = _rand_half(rng, (1, 1, 1, D))
        k = _rand_half(rng, (1, 2, 1, D))
        v = _rand_half(rng, (1, 2, 1, D))
        scale = float(np.float32(rng.uniform(0.05, 2.0)))
        r = oracle.prefill(q, k, v, scale=scale, causal=False, dtype="f16")
        s0 = _exact_score(_f(q[0, 0, 0]), _f(k[0, 0, 0]), scale)
        s1 = _exact_score(_f(q[0, 0, 0]), _f(k[0, 1, 0]), scale)
        sig = lambda x: 1.0 / (1.0 + math.exp(-x))
        o = sig(s0 - s1) * _f(v[0, 0, 0]) + sig(s1 - s0) * _f(v[0, 1, 0])
        lse = max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))
        np.testing.assert_allclose(r["o"][0, 0, 0], o, rtol=1e-13, atol=1e-14)
        assert r["lse"][0, 0, 0] == pytest.approx(lse, rel=1e-14, abs=1e-14)


# --------------------------------------------------------------------------
# Further invariants that catch a dropped normalization, a transposed operand
# or a wrong scale.
# --------------------------------------------------------------------------

def test_affine_in_v():
    """Weights sum to one: O(V A + 1 b^T) = O(V) A + b (fails without the 1/l)."""
    rng = np.random.default_rng(31)
    q = _rand_half(rng, (1, 20, 1, 6))
    k = _rand_half(rng, (1, 30, 1, 6))
    vr = rng.standard_normal((1, 30, 1, 5))
    A = rng.standard_normal((5, 5))
    bvec = rng.standard_normal(5)
    qf, kf = _f(q), _f(k)
    r1 = oracle.prefill(qf, kf, vr, scale=0.4, causal=True)
    r2 = oracle.prefill(qf, kf, vr @ A + bvec, scale=0.4, causal=True)
    np.testing.assert_allclose(r2["o"], r1["o"] @ A + bvec, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r2["lse"], r1["lse"], rtol=0, atol=0)


def test_key_shift_moves_lse_only():
    """Adding c to every key adds scale*q.c to each score: O fixed, LSE shifted."""
    rng = np.random.default_rng(32)
    qf = rng.standard_normal((1, 9, 1, 4))
    kf = rng.standard_normal((1, 9, 1, 4))
    vf = rng.standard_normal((1, 9, 1, 3))
    c = rng.standard_normal(4)
    r1 = oracle.prefill(qf, kf, vf, scale=0.8, causal=True)
    r2 = oracle.prefill(qf, kf + c, vf, scale=0.8, causal=True)
    np.testing.assert_allclose(r2["o"], r1["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r2["lse"][0, 0], r1["lse"][0, 0] + 0.8 * (qf[0, :, 0] @ c),
                               rtol=1e-12, atol=1e-12)


def test_large_scale_is_hardmax():
    """As scale grows the softmax picks the argmax key (non-square, unmasked)."""
    rng = np.random.default_rng(33)
    qf = rng.standard_normal((1, 5, 1, 3))
    kf = rng.standard_normal((1, 11, 1, 3))
    vf = rng.standard_normal((1, 11, 1, 7))
    r = oracle.prefill(qf, kf, vf, scale=1e6, causal=False)
    best = np.argmax(qf[0, :, 0] @ kf[0, :, 0].T, axis=1)
    np.testing.assert_allclose(r["o"][0, :, 0], vf[0, best, 0], rtol=0, atol=1e-12)


def test_permuting_keys_unmasked():
    rng = np.random.default_rng(34)
    qf = rng.standard_normal((1, 4, 2, 5))
    kf = rng.standard_normal((1, 13, 1, 5))
    vf = rng.standard_normal((1, 13, 1, 6))
    perm = rng.permutation(13)
    r1 = oracle.prefill(qf, kf, vf, scale=0.5, causal=False)
    r2 = oracle.prefill(qf, kf[:, perm], vf[:, perm], scale=0.5, causal=False)
    np.testing.assert_allclose(r2["o"], r1["o"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r2["lse"], r1["lse"], rtol=1e-13, atol=1e-14)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(35)
    q = _rand_half(rng, (2, 33, 4, 8), "bf16")
    k = _rand_half(rng, (2, 40, 2, 8), "bf16")
    v = _rand_half(rng, (2, 40, 2, 8), "bf16")
    full = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="bf16")
    rows = [0, 7, 32]
    sub = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="bf16", rows=rows)
    assert np.array_equal(sub["o"], full["o"][:, rows])
    assert np.array_equal(sub["lse"], full["lse"][:, :, rows])


# --------------------------------------------------------------------------
# P-8: generator stability (inputs are fixed by seed; chunking does not move bits)
# --------------------------------------------------------------------------

def test_generator_chunk_independent(monkeypatch):
    rng = np.random.default_rng(4)
    whole = inputs.draw_half(rng, (3, 1000), "bf16")
    monkeypatch.setattr(inputs, "_CHUNK", 77)
    rng = np.random.default_rng(4)
    chunked = inputs.draw_half(rng, (3, 1000), "bf16")
    assert np.array_equal(whole, chunked)


def test_generator_sha256_fixed():
    import hashlib
    with open(os.path.join(GOLDEN, "generator_sha256.json")) as fh:
        want = json.load(fh)
    for name in (inputs.TINY_CAUSAL.name, inputs.GQA_PREFILL.name, inputs.GQA_DECODE.name):
        cfg = inputs.WORKLOADS[name]
        data = (inputs.make_prefill_inputs(cfg) if isinstance(cfg, inputs.PrefillConfig)
                else inputs.make_decode_inputs(cfg))
        for key, arr in sorted(data.items()):
            got = hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()
            assert got == want[name][key], (name, key)
    rng = np.random.default_rng(inputs.LONG_DECODE.seed)
    lens = inputs.decode_lengths(inputs.LONG_DECODE, rng)
    assert hashlib.sha256(lens.tobytes()).hexdigest() == want[inputs.LONG_DECODE.name]["kv_lens"]
    assert lens.min() >= 512 and lens.max() <= 32768


# --------------------------------------------------------------------------
# Masks beyond causality: per-sequence KV length and sliding window
# --------------------------------------------------------------------------

def _mask_inputs(seed, B=2, sq=9, skv=13, hq=4, hkv=2, D=8):
    rng = np.random.default_rng(seed)
    return (_rand_half(rng, (B, sq, hq, D)), _rand_half(rng, (B, skv, hkv, D), mult=2.0),
            _rand_half(rng, (B, skv, hkv, D)))


@pytest.mark.parametrize("causal", [True, False])
def test_masks_that_admit_everything_change_nothing(causal):
    q, k, v = _mask_inputs(101)
    scale = float(np.float32(0.3))
    base = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16")
    full = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16",
                          kv_lens=[13, 13], window=13 + 9)
    for key in ("o", "lse", "row_sum"):
        assert base[key].tobytes() == full[key].tobytes()


def test_kv_length_equals_truncated_cache():
    """Unmasked attention with kv_lens[b] = L equals attention over the first L keys."""
    q, k, v = _mask_inputs(102)
    scale = float(np.float32(0.3))
    lens = [5, 11]
    r = oracle.prefill(q, k, v, scale=scale, causal=False, dtype="f16", kv_lens=lens)
    for b, L in enumerate(lens):
        t = oracle.prefill(q[b:b + 1], k[b:b + 1, :L], v[b:b + 1, :L], scale=scale, causal=False,
                           dtype="f16")
        np.testing.assert_allclose(r["o"][b], t["o"][0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["lse"][b], t["lse"][0], rtol=1e-13, atol=1e-15)


def test_window_of_one_is_the_diagonal_key():
    """Causal window 1: every row sees exactly key q_pos, so O = V[q_pos] exactly and
    LSE = the exact score."""
    q, k, v = _mask_inputs(103, B=1, sq=6, skv=9)
    scale = float(np.float32(0.5))
    r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16", window=1)
    off = 9 - 6
    for i in range(6):
        for h in range(4):
            hk = h // 2
            np.testing.assert_array_equal(r["o"][0, i, h], _f(v[0, i + off, hk]))
            assert r["lse"][0, h, i] == float(_exact_score(_f(q[0, i, h]), _f(k[0, i + off, hk]),
                                                           scale))


def test_window_equals_sliced_keys():
    """Causal window W: row i equals unmasked attention over keys q_pos-W+1 .. q_pos."""
    q, k, v = _mask_inputs(104, B=1, sq=10, skv=10)
    scale = float(np.float32(0.4))
    W = 4
    r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16", window=W)
    for i in range(10):
        lo = max(0, i - W + 1)
        for h in range(4):
            hk = h // 2
            t = oracle.attend_rows(_f(q[0, i:i + 1, h]), _f(k[0, lo:i + 1, hk]),
                                   _f(v[0, lo:i + 1, hk]), scale, None)
            np.testing.assert_allclose(r["o"][0, i, h], t["o"][0], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(r["lse"][0, h, i], t["lse"][0], rtol=1e-13, atol=1e-15)


def test_masked_keys_do_not_matter_bitwise():
    """Changing K/V rows outside every row's window and past each sequence's length
    leaves all outputs bit-identical."""
    q, k, v = _mask_inputs(105, B=2, sq=8, skv=12)
    scale = float(np.float32(0.3))
    lens, W = [9, 12], 3
    r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16", kv_lens=lens, window=W)
    k2, v2 = k.copy(), v.copy()
    rng = np.random.default_rng(7)
    # rows are at positions 4..11: keys 0 and 1 are below every window; keys >= len are cut
    for b, L in enumerate(lens):
        for j in list(range(0, 2)) + list(range(L, 12)):
            k2[b, j] = _rand_half(rng, k2[b, j].shape, mult=4.0)
            v2[b, j] = _rand_half(rng, v2[b, j].shape, mult=4.0)
    r2 = oracle.prefill(q, k2, v2, scale=scale, causal=True, dtype="f16", kv_lens=lens, window=W)
    for key in ("o", "lse", "row_sum"):
        assert r[key].tobytes() == r2[key].tobytes()


def test_rows_without_visible_keys():
    """A window that ends before the sequence's valid length starts leaves a row
    without keys: O = 0, row_sum = 0, LSE = -inf; the other rows are unaffected."""
    q, k, v = _mask_inputs(106, B=1, sq=8, skv=8)
    scale = float(np.float32(0.3))
    r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16", kv_lens=[3], window=2)
    # row i (q_pos = i) sees keys max(0, i-1) .. min(i, 2): empty from i = 4 on
    for i in range(8):
        if i >= 4:
            assert np.all(r["o"][0, i] == 0) and np.all(np.isneginf(r["lse"][0, :, i]))
            assert np.all(r["row_sum"][0, :, i] == 0)
        else:
            assert np.all(np.isfinite(r["lse"][0, :, i]))


def _decimal_masked(qf, kf, vf, scale, visible):
    getcontext().prec = 60
    sc = Decimal(scale)
    sq = qf.shape[0]
    out_o = np.zeros((sq, vf.shape[1]))
    out_lse = np.full(sq, -np.inf)
    for i in range(sq):
        js = [j for j in range(kf.shape[0]) if visible(i, j)]
        if not js:
            continue
        ex = [(sum(Decimal(float(qf[i, d])) * Decimal(float(kf[j, d]))
                   for d in range(qf.shape[1])) * sc).exp() for j in js]
        tot = sum(ex)
        out_lse[i] = float(tot.ln())
        for d in range(vf.shape[1]):
            out_o[i, d] = float(sum(e * Decimal(float(vf[j, d])) for j, e in zip(js, ex)) / tot)
    return out_o, out_lse


@pytest.mark.parametrize("causal,L,W", [(True, 5, 3), (False, 6, 2), (True, 7, 0)])
def test_brute_force_decimal_masks(causal, L, W):
    sq, skv, D = 5, 7, 3
    q, k, v = _mask_inputs(107 + L + W, B=1, sq=sq, skv=skv, hq=2, hkv=1, D=D)
    scale = float(np.float32(0.7))
    r = oracle.prefill(q, k, v, scale=scale, causal=causal, dtype="f16", kv_lens=[L], window=W)

    def visible(i, j):
        pos = i + skv - sq
        return (j <= pos or not causal) and j < L and (W == 0 or j > pos - W)
    for h in range(2):
        o, lse = _decimal_masked(_f(q[0, :, h]), _f(k[0, :, 0]), _f(v[0, :, 0]), scale, visible)
        np.testing.assert_allclose(r["o"][0, :, h], o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["lse"][0, h], lse, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# Sink logit and the merge of passes over disjoint key sets
# ("STAGE_D.md — FMHA Kernel Development", D5)
# --------------------------------------------------------------------------

def test_sink_at_minus_infinity_is_no_sink():
    q, k, v = _mask_inputs(301, B=2, sq=9, skv=13, hq=4, hkv=2, D=8)
    for kv_lens in (None, [13, 0]):
        a = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="f16", kv_lens=kv_lens)
        b = oracle.prefill(q, k, v, scale=0.3, causal=True, dtype="f16", kv_lens=kv_lens,
                           sink_logits=[-np.inf] * 4)
        for key in ("o", "lse", "row_sum", "row_max", "o_unnorm"):
            assert a[key].tobytes() == b[key].tobytes(), key


@pytest.mark.parametrize("sink,extra", [(0.0, 1), (math.log(3.0), 3), (math.log(0.5), 0.5)])
def test_sink_tied_scores_closed_form(sink, extra):
    """q = 0 makes every score 0: row i (causal) sees i + 1 keys of weight 1 and
    the sink adds exp(sink): LSE = ln(i + 1 + exp(sink)), O = sum of the seen
    V rows / (i + 1 + exp(sink))."""
    rng = np.random.default_rng(7)
    S, D = 6, 4
    q = np.zeros((1, S, 1, D))
    k = rng.standard_normal((1, S, 1, D))
    v = rng.standard_normal((1, S, 1, D))
    r = oracle.prefill(q, k, v, scale=1.0, causal=True, sink_logits=[sink])
    for i in range(S):
        den = i + 1 + extra
        assert abs(r["lse"][0, 0, i] - math.log(den)) < 1e-14
        np.testing.assert_allclose(r["o"][0, i, 0], v[0, :i + 1, 0].sum(axis=0) / den,
                                   rtol=1e-14, atol=1e-15)


def test_sink_only_rows():
    """Rows that see no key keep only the sink: O = 0, LSE = the sink logit,
    row_max = sink, row_sum = 1."""
    q, k, v = _mask_inputs(303, B=1, sq=5, skv=7, hq=2, hkv=1, D=4)
    sinks = [0.75, -2.5]
    r = oracle.prefill(q, k, v, scale=0.5, causal=True, dtype="f16", kv_lens=[0],
                       sink_logits=sinks)
    for h in range(2):
        assert (r["o"][0, :, h] == 0).all()
        assert (r["lse"][0, h] == sinks[h]).all() and (r["row_max"][0, h] == sinks[h]).all()
        assert (r["row_sum"][0, h] == 1.0).all()


def _decimal_with_sink(qf, kf, vf, scale, sink):
    getcontext().prec = 60
    sc = Decimal(scale)
    sq = qf.shape[0]
    out_o = np.zeros((sq, vf.shape[1]))
    out_lse = np.zeros(sq)
    off = kf.shape[0] - sq
    for i in range(sq):
        js = list(range(i + off + 1))
        ex = [(sum(Decimal(float(qf[i, d])) * Decimal(float(kf[j, d]))
                   for d in range(qf.shape[1])) * sc).exp() for j in js]
        tot = sum(ex) + Decimal(sink).exp()
        out_lse[i] = float(tot.ln())
        for d in range(vf.shape[1]):
            out_o[i, d] = float(sum(e * Decimal(float(vf[j, d])) for j, e in zip(js, ex)) / tot)
    return out_o, out_lse


@pytest.mark.parametrize("sink", [-1.25, 0.5, 3.0])
def test_sink_brute_force_decimal(sink):
    sq, skv, D = 4, 6, 3
    q, k, v = _mask_inputs(311, B=1, sq=sq, skv=skv, hq=2, hkv=1, D=D)
    scale = float(np.float32(0.6))
    r = oracle.prefill(q, k, v, scale=scale, causal=True, dtype="f16",
                       sink_logits=[sink, -sink])
    for h, sg in ((0, sink), (1, -sink)):
        o, lse = _decimal_with_sink(_f(q[0, :, h]), _f(k[0, :, 0]), _f(v[0, :, 0]), scale, sg)
        np.testing.assert_allclose(r["o"][0, :, h], o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["lse"][0, h], lse, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_a_key_partition_is_the_whole_pass(seed):
    """Attention over a key set equals the LSE merge of attention over any
    partition of it (rows whose part is empty included)."""
    rng = np.random.default_rng(400 + seed)
    R, S, D = 7, 19, 5
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((S, D)) * 2.0
    v = rng.standard_normal((S, D))
    vis = rng.random((R, S)) < 0.7
    part = rng.random((R, S)) < 0.5
    part[0] = True                           # row 0: second part empty
    part[1] = False                          # row 1: first part empty
    whole = oracle.attend_rows(q, k, v, 0.8, None, vis)
    a = oracle.attend_rows(q, k, v, 0.8, None, vis & part)
    b = oracle.attend_rows(q, k, v, 0.8, None, vis & ~part)
    m = oracle.merge_branches([a["o"], b["o"]], [a["lse"], b["lse"]])
    np.testing.assert_allclose(m["o"], whole["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m["lse"], whole["lse"], rtol=1e-12, atol=1e-13)
    # with a sink: the sink is one more branch (O = 0, LSE = sink)
    ws = oracle.attend_rows(q, k, v, 0.8, None, vis, sink=0.3)
    m2 = oracle.merge_branches([a["o"], b["o"], np.zeros_like(a["o"])],
                               [a["lse"], b["lse"], np.full(R, 0.3)])
    np.testing.assert_allclose(m2["o"], ws["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m2["lse"], ws["lse"], rtol=1e-12, atol=1e-13)


def test_merge_branches_large_and_empty():
    """Weights 1 : 3 at LSE 1000 (no overflow: the merge is max-shifted), and
    branches with LSE = -inf count for nothing; all-empty gives O = 0, -inf."""
    o1, o2 = np.array([[1.0, -2.0]]), np.array([[5.0, 2.0]])
    m = oracle.merge_branches([o1, o2], [np.array([1000.0]), np.array([1000.0 + math.log(3.0)])])
    np.testing.assert_allclose(m["o"], (o1 + 3 * o2) / 4, rtol=1e-12)  # 1000 + ln 3 rounds
    assert abs(m["lse"][0] - (1000.0 + math.log(4.0))) < 1e-12
    m = oracle.merge_branches([o1, o2], [np.array([-np.inf]), np.array([2.5])])
    assert m["o"].tobytes() == o2.tobytes() and m["lse"][0] == 2.5
    m = oracle.merge_branches([o1, o2], [np.array([-np.inf]), np.array([-np.inf])])
    assert (m["o"] == 0).all() and np.isneginf(m["lse"]).all()
