"""The max-free softmax of the head_dim 64/128 prefill (normalized output, no
row sums) against the fp64 oracle, on score patterns that make its exponent
base move (needs an MI355X).

Source: "STAGE_D.md — FMHA Kernel Development", "Kernel Output" (O and the
natural-log LSE) and "60 · r57 — FA KV staging double buffering (REVERTED)",
section 1 (the online softmax kept in registers). Without a per-tile row max,
the kernel moves its base only when a lane's sum of a tile's P passes 2^15.
The inputs here force that path:

* ``ramp``: scores grow along the keys (K = g * c_j, c_j increasing), so later
  tiles keep exceeding the base and the base moves again and again;
* ``step``: every key after the first 64 scores 4 log2 units above the first
  64, which trips the sum bound (32 keys x 2^11 per lane) although no single
  key is 2^8 above the base (the threshold of the max-tracking form);
* ``peaked``: K drawn 4x and 8x larger than usual (peaked rows).

Each case also runs the max-tracking kernel (the same call asking for row
sums) and both must meet the prefill gate: |O| error <= 2e-3, LSE error <=
1e-4, on every row and head.
"""
import math

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


def _structured(rng, B, S, Hq, Hkv, D, dtype, pattern):
    """q, k, v half bits. For ``ramp``/``step`` every query row of a head is
    one vector g and K row j is g * c_j / |g|^2 * sqrt(D), so that the score
    (with scale 1/sqrt(D)) is c_j before rounding to half."""
    v = inputs.draw_half(rng, (B, S, Hkv, D), dtype)
    if pattern.startswith("peaked"):
        mult = float(pattern[len("peaked"):])
        q = inputs.draw_half(rng, (B, S, Hq, D), dtype)
        k = inputs.draw_half(rng, (B, S, Hkv, D), dtype, mult=mult)
        return q, k, v
    g = rng.standard_normal((Hkv, D)).astype(np.float32)
    j = np.arange(S, dtype=np.float32)
    if pattern == "ramp":
        c = 0.02 * j                                   # +1.85 log2 units per 64 keys
    else:
        c = np.where(j < 64, 0.0, 4.0 * math.log(2.0)).astype(np.float32)
    qf = np.broadcast_to(np.repeat(g, Hq // Hkv, axis=0)[None, None], (B, S, Hq, D))
    kf = (c[None, :, None, None] * (g / (g * g).sum(axis=1, keepdims=True) * math.sqrt(D))[None, None])
    kf = np.broadcast_to(kf, (B, S, Hkv, D))
    return (inputs.round_f32_to_half_bits(np.ascontiguousarray(qf, dtype=np.float32), dtype),
            inputs.round_f32_to_half_bits(np.ascontiguousarray(kf, dtype=np.float32), dtype), v)


# (B, S, Hq, Hkv, D, dtype, pattern, window)
CASES = [
    (1, 700, 4, 2, 128, "bf16", "ramp", 0),      # paired heads
    (1, 700, 3, 1, 128, "f16", "ramp", 0),       # one head per wave, V rows
    (1, 333, 2, 2, 64, "bf16", "step", 0),
    (2, 300, 6, 2, 128, "f16", "step", 0),
    (1, 520, 7, 1, 128, "bf16", "step", 200),    # window: the first tiles drop out
    (2, 410, 8, 2, 64, "f16", "peaked4", 0),
    (1, 600, 7, 1, 128, "bf16", "peaked8", 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_max_free_softmax_matches_oracle(torch_gpu, case):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    B, S, Hq, Hkv, D, dtype, pattern, window = case
    _say("sum-checked softmax", case)
    rng = np.random.default_rng(S * 7 + Hq + D)
    q, k, v = _structured(rng, B, S, Hq, Hkv, D, dtype, pattern)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    qd, kd, vd = _dev(torch, q, dtype), _dev(torch, k, dtype), _dev(torch, v, dtype)
    o1, l1 = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale, window=window)
    o2, l2, _ = fa.prefill(qd, kd, vd, causal=True, softmax_scale=scale, window=window,
                           want_row_sum=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, scale=scale, causal=True, dtype=dtype, window=window)
    seen = np.isfinite(ref["lse"])
    seen_o = np.transpose(seen, (0, 2, 1))
    for name, o, lse in (("max-free", o1, l1), ("max-tracking", o2, l2)):
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        err_o = np.abs(o[seen_o] - ref["o"][seen_o]).max()
        err_l = np.abs(lse[seen] - ref["lse"][seen]).max()
        assert err_o <= O_TOL and err_l <= LSE_TOL, \
            f"{name}: O err {err_o:.3e}, LSE err {err_l:.3e}"
