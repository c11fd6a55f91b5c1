"""The allocation-free single-launch decode (fa_decode_fused_noalloc) against
the workspace form (fa_decode_fused) and the fp64 oracle (needs an MI355X).

fa_decode_fused_noalloc runs fa_decode_fused's kernels on a library-owned
static scratch array per GPU, for callers that cannot allocate. Two calls in a
row through the C ABI, the second with a smaller input (and then the first
shape again), each compared with fa_decode_fused on a fresh zero-filled
workspace: the same bytes, and both within the decode gate of the oracle
(|O| error <= 2e-3, natural-log LSE error <= 1e-4; "66 · D2: explicit K+V
register staging ...", sections 3.2 and 5.2, for the partials and their
combine, "STAGE_D.md — FMHA Kernel Development", D5c for the single launch).
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


def _dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


def _case(lens, hq, hkv, D, dtype, seed):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    offs = np.concatenate([[0], np.cumsum(lens.astype(np.int64))[:-1]]).astype(np.int64)
    T = int(lens.sum())
    return {"q": inputs.draw_half(rng, (len(lens), hq, D), dtype),
            "k_cache": inputs.draw_half(rng, (T, hkv, D), dtype),
            "v_cache": inputs.draw_half(rng, (T, hkv, D), dtype),
            "kv_lens": lens, "kv_offsets": offs, "hq": hq, "hkv": hkv, "D": D, "dtype": dtype}


CALLS = [
    # the 1641-token GQA decode (28 query / 4 KV heads), then a smaller mixed
    # batch (lengths 1, 100, 333), then the first shape again
    ([1641], 28, 4, 128, "f16", 3),
    ([1, 100, 333], 8, 2, 64, "bf16", 5),
    ([1641], 28, 4, 128, "f16", 7),
]


def test_noalloc_decode_matches_workspace_form(torch_gpu):
    from flashattention_attention_amd import fa
    torch = torch_gpu
    for i, (lens, hq, hkv, D, dtype, seed) in enumerate(CALLS):
        print(f"[case] noalloc decode call {i}: lens {lens} heads {hq}/{hkv} D {D} {dtype}",
              flush=True)
        x = _case(lens, hq, hkv, D, dtype, seed)
        q, kc, vc = (_dev(torch, x[n], dtype) for n in ("q", "k_cache", "v_cache"))
        offs = torch.from_numpy(x["kv_offsets"]).cuda()
        kl = torch.from_numpy(x["kv_lens"]).cuda()
        sl, ms = fa.decode_plan(lens, hq, hkv, D)
        scale = float(np.float32(1 / np.sqrt(D)))
        B = len(lens)
        assert fa.decode_fused_workspace_size(B, hq, hkv, D, ms) <= fa.DECODE_NOALLOC_SCRATCH_BYTES
        o_n = torch.full((B, hq, D), float("nan"), device="cuda")
        l_n = torch.full((B, hq), float("nan"), device="cuda")
        fa.decode_fused_noalloc(q, kc, vc, offs, kl, split_len=sl, max_splits=ms,
                                softmax_scale=scale, out=o_n, lse=l_n)
        o_w, l_w = fa.decode_fused(q, kc, vc, offs, kl, split_len=sl, max_splits=ms,
                                   softmax_scale=scale)
        torch.cuda.synchronize()
        o_n, l_n, o_w, l_w = (t.cpu().numpy() for t in (o_n, l_n, o_w, l_w))
        assert o_n.tobytes() == o_w.tobytes() and l_n.tobytes() == l_w.tobytes()
        ref = oracle.decode(x["q"], x["k_cache"], x["v_cache"], x["kv_offsets"], x["kv_lens"],
                            scale=scale, dtype=dtype)
        err_o = float(np.abs(o_n - ref["o"]).max())
        err_l = float(np.abs(l_n - ref["lse"]).max())
        assert err_o <= O_TOL and err_l <= LSE_TOL, (i, err_o, err_l)
