"""Parity of the single-launch decode (fa_decode_fused) against the fp64 oracle
and the two-launch form (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", D5c (the passes fused into one
launch) and "66 · D2: explicit K+V register staging ...", section 5.2 (the
combine step after the split partials). Same gate as the two-launch decode:
|O| error <= 2e-3, natural-log LSE error <= 1e-4, byte-identical repeats, and
the workspace's arrival counters back at zero after every call.
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


def _inputs(lens, hq, hkv, D, dtype, seed):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    T = max(1, int(lens.clip(min=0).sum()))
    return {"q": inputs.draw_half(rng, (len(lens), hq, D), dtype),
            "k_cache": inputs.draw_half(rng, (T, hkv, D), dtype),
            "v_cache": inputs.draw_half(rng, (T, hkv, D), dtype),
            "kv_lens": lens, "kv_offsets": offs}


def _to_dev(torch, x, dtype):
    return (_dev(torch, x["q"], dtype), _dev(torch, x["k_cache"], dtype),
            _dev(torch, x["v_cache"], dtype), torch.from_numpy(x["kv_offsets"]).cuda(),
            torch.from_numpy(x["kv_lens"]).cuda())


def _counters_bytes(B, hq, hkv):
    g = max(d for d in range(1, 9) if (hq // hkv) % d == 0)
    return B * (hq // g) * 4


def _fused(torch, dev_x, split_len, max_splits, scale, ws=None):
    from flashattention_attention_amd import fa
    q = dev_x[0]
    B, Hq, D = q.shape
    o = torch.full((B, Hq, D), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    fa.decode_fused(*dev_x, split_len=split_len, max_splits=max_splits, softmax_scale=scale,
                    out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _two_launch(torch, dev_x, split_len, max_splits, scale):
    from flashattention_attention_amd import fa
    o, lse = fa.decode(*dev_x, split_len=split_len, max_splits=max_splits, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("split_len", ["plan", 16, 32, 48, 112, 208, 1648])
def test_fused_gqa_decode_workload(torch_gpu, split_len):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    cfg = inputs.GQA_DECODE
    _say("fused", cfg.name, split_len)
    x = inputs.make_decode_inputs(cfg)
    if split_len == "plan":
        split_len, max_splits = fa.decode_plan(x["kv_lens"], cfg.n_heads_q, cfg.n_heads_kv,
                                               cfg.head_dim)
    else:
        max_splits = -(-int(x["kv_lens"].max()) // split_len)
    dx = _to_dev(torch, x, cfg.dtype)
    ws = torch.zeros(fa.decode_fused_workspace_size(cfg.batch, cfg.n_heads_q, cfg.n_heads_kv,
                                                    cfg.head_dim, max_splits),
                     dtype=torch.uint8, device="cuda")
    runs = [_fused(torch, dx, split_len, max_splits, cfg.scale, ws) for _ in range(3)]
    for r in runs[1:]:
        assert r[0].tobytes() == runs[0][0].tobytes() and r[1].tobytes() == runs[0][1].tobytes()
    nc = _counters_bytes(cfg.batch, cfg.n_heads_q, cfg.n_heads_kv)
    assert not ws[:nc].cpu().numpy().any()                    # counters back at zero
    o, lse = runs[0]
    ref = oracle.decode(x["q"], x["k_cache"], x["v_cache"], x["kv_offsets"], x["kv_lens"],
                        scale=cfg.scale, dtype=cfg.dtype)
    assert np.abs(o - ref["o"]).max() <= O_TOL
    assert np.abs(lse - ref["lse"]).max() <= LSE_TOL
    o2, lse2 = _two_launch(torch, dx, split_len, max_splits, cfg.scale)
    assert np.abs(o - o2).max() <= O_TOL and np.abs(lse - lse2).max() <= LSE_TOL


@pytest.mark.parametrize("dtype,D,hq,hkv,split_len,extra", [
    ("f16", 128, 28, 4, 48, 3), ("bf16", 128, 32, 8, 16, 20), ("f16", 64, 8, 8, 32, 0),
    ("bf16", 256, 16, 2, 48, 5), ("f16", 128, 12, 1, 112, 1), ("bf16", 64, 6, 2, 16, 9),
    ("f16", 256, 4, 4, 16, 0),
    ("f16", 128, 32, 4, 48, 0),     # 4 heads per wave, 4-wave work-groups, P.V on MFMA
])
def test_fused_lengths_and_spare_splits(torch_gpu, dtype, D, hq, hkv, split_len, extra):
    """KV lengths {1, 29, 52, 512, 1641} in one batch, with `extra` spare splits
    beyond the longest sequence (whole work-groups with nothing to do)."""
    torch = torch_gpu
    _say("fused lens", dtype, D, hq, hkv, split_len, extra)
    lens = [1, 29, 52, 512, 1641]
    x = _inputs(lens, hq, hkv, D, dtype, seed=D + hq + split_len)
    scale = float(np.float32(1 / np.sqrt(D)))
    max_splits = -(-max(lens) // split_len) + extra
    dx = _to_dev(torch, x, dtype)
    o, lse = _fused(torch, dx, split_len, max_splits, scale)
    ref = oracle.decode(x["q"], x["k_cache"], x["v_cache"], x["kv_offsets"], x["kv_lens"],
                        scale=scale, dtype=dtype)
    assert np.abs(o - ref["o"]).max() <= O_TOL
    assert np.abs(lse - ref["lse"]).max() <= LSE_TOL
    # one visible key: the output is that key's V row, up to the rounding of
    # its weight (fp16 into the matrix-core P.V against the fp32 row sum:
    # < 1.5e-6 relative, see test_decode_mfma_gpu)
    hk_of = np.arange(hq) // (hq // hkv)
    v0 = inputs.half_bits_to_f32(x["v_cache"][0], dtype)[hk_of]
    np.testing.assert_allclose(o[0], v0, atol=1e-6, rtol=4e-6)


@pytest.mark.parametrize("max_splits", [3, 20])
def test_fused_bad_lengths_give_nan(torch_gpu, max_splits):
    """Zero keys, or more splits than max_splits, give NaN; other sequences are
    unaffected (one work-group per sequence at 3 splits, several at 20)."""
    torch = torch_gpu
    _say("fused bad lengths", max_splits)
    too_long = 16 * max_splits + 1
    x = _inputs([too_long, 1, 40], 4, 2, 128, "f16", seed=5)
    x["kv_lens"] = np.array([too_long, 0, 40], np.int32)
    o, lse = _fused(torch, _to_dev(torch, x, "f16"), 16, max_splits, 0.088)
    assert np.isnan(o[0]).all() and np.isnan(lse[0]).all()
    assert np.isnan(o[1]).all() and np.isnan(lse[1]).all()
    assert np.isfinite(o[2]).all() and np.isfinite(lse[2]).all()
    ref = oracle.decode(x["q"][2:], x["k_cache"], x["v_cache"], x["kv_offsets"][2:],
                        x["kv_lens"][2:], scale=0.088, dtype="f16")
    assert np.abs(o[2:] - ref["o"]).max() <= O_TOL


def test_fused_long_decode_full_size(torch_gpu):
    """The batched long decode at full size, sampled (sequence, head) pairs against
    the oracle; one workspace reused by consecutive calls of two shapes."""
    from flashattention_attention_amd import fa
    torch = torch_gpu
    cfg = inputs.LONG_DECODE
    _say("fused", cfg.name)
    x = inputs.make_decode_inputs(cfg)
    split_len, max_splits = fa.decode_plan(x["kv_lens"], cfg.n_heads_q, cfg.n_heads_kv,
                                           cfg.head_dim)
    dx = _to_dev(torch, x, cfg.dtype)
    ws = torch.zeros(fa.decode_fused_workspace_size(cfg.batch, cfg.n_heads_q, cfg.n_heads_kv,
                                                    cfg.head_dim, max_splits),
                     dtype=torch.uint8, device="cuda")
    a = _fused(torch, dx, split_len, max_splits, cfg.scale, ws)
    small = _inputs([300, 17], 32, 8, 128, "f16", seed=9)
    s1 = _fused(torch, _to_dev(torch, small, "f16"), 32, 10, cfg.scale, ws)
    b = _fused(torch, dx, split_len, max_splits, cfg.scale, ws)
    assert a[0].tobytes() == b[0].tobytes() and a[1].tobytes() == b[1].tobytes()
    ref_s = oracle.decode(small["q"], small["k_cache"], small["v_cache"], small["kv_offsets"],
                          small["kv_lens"], scale=cfg.scale, dtype="f16")
    assert np.abs(s1[0] - ref_s["o"]).max() <= O_TOL
    o, lse = a
    rng = np.random.default_rng(4)
    picks = {(int(np.argmax(x["kv_lens"])), 0), (int(np.argmin(x["kv_lens"])), cfg.n_heads_q - 1)}
    picks |= {(int(bb), int(h)) for bb, h in zip(rng.integers(0, cfg.batch, 10),
                                                 rng.integers(0, cfg.n_heads_q, 10))}
    for bb, h in sorted(picks):
        hk = h // (cfg.n_heads_q // cfg.n_heads_kv)
        ref = oracle.decode(x["q"][bb:bb + 1, h:h + 1], x["k_cache"][:, hk:hk + 1],
                            x["v_cache"][:, hk:hk + 1], x["kv_offsets"][bb:bb + 1],
                            x["kv_lens"][bb:bb + 1], scale=cfg.scale, dtype=cfg.dtype)
        assert np.abs(o[bb, h] - ref["o"][0, 0]).max() <= O_TOL, (bb, h)
        assert abs(lse[bb, h] - ref["lse"][0, 0]) <= LSE_TOL, (bb, h)
