"""C-ABI checks that need no GPU: the library loads, exports what include/fa.h
declares, plans deterministically, and rejects invalid arguments on the host
before any HIP call (so nothing is ever launched here)."""
import ctypes
import os

import pytest

from flashattention_attention_amd import fa

pytestmark = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                                reason="libfa.so not built")

ALIGNED = 0x10000          # never dereferenced: every call below fails validation first


def _gpu_visible():
    # Counting devices does not initialise HIP on this image.
    import torch
    return torch.cuda.device_count() > 0


def test_exports_every_declared_symbol():
    names = fa.declared_functions()
    assert set(names) == {"fa_prefill_fwd", "fa_prefill_pack_v", "fa_prefill_fwd_packed",
                          "fa_prefill_workspace_size", "fa_decode_plan",
                          "fa_decode_split_partial", "fa_decode_merge_lse", "fa_decode_fused",
                          "fa_decode_fused_noalloc",
                          "fa_decode_fused_workspace_size", "fa_decode_fused_waves",
                          "fa_attn_merge", "fa_prefill_fwd_packed_split",
                          "fa_prefill_split_workspace_size", "fa_prefill_split_units",
                          "fa_prefill_trio", "fa_status_string", "fa_last_error"}
    lib = ctypes.CDLL(fa.library_path())
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = fa.load_library()
    assert lib.fa_status_string(0) == b"FA_OK"
    assert lib.fa_status_string(1) == b"FA_ERR_INVALID_ARG"
    assert lib.fa_status_string(2) == b"FA_ERR_UNSUPPORTED"
    assert lib.fa_status_string(3) == b"FA_ERR_HIP"


def _plan(lens, hq, hkv, d=128, cus=256):
    lib = fa.load_library()
    sl, ms = ctypes.c_int(), ctypes.c_int()
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    st = lib.fa_decode_plan(arr if lens is not None else None, len(lens), hq, hkv, d, cus,
                            ctypes.byref(sl), ctypes.byref(ms))
    return st, sl.value, ms.value


@pytest.mark.parametrize("lens,hq,hkv,d", [([1641], 28, 4, 128),
                                           ([512 + 997 * i for i in range(32)], 32, 8, 128),
                                           ([1, 29, 52], 4, 2, 64), ([1], 1, 1, 256),
                                           ([100000] * 3, 16, 2, 128)])
def test_decode_plan_is_pure_and_covers_lengths(lens, hq, hkv, d):
    st, sl, ms = _plan(lens, hq, hkv, d)
    assert st == 0
    assert sl % 16 == 0 and sl >= 16
    assert ms == -(-max(lens) // sl)
    assert (st, sl, ms) == _plan(lens, hq, hkv, d)


def test_decode_plan_prefers_one_round():
    # 32 long sequences x 8 KV heads: the chosen split keeps the wave count
    # within one round of resident waves (256 CUs x 8).
    lens = [int(x) for x in __import__("numpy").random.default_rng(4).integers(512, 32769, 32)]
    st, sl, ms = _plan(lens, 32, 8, 128)
    waves = sum(-(-L // sl) for L in lens) * 8
    assert st == 0 and waves <= 2048


@pytest.mark.parametrize("args", [
    dict(lens=[0]), dict(lens=[5, -1]), dict(hq=0), dict(hkv=3), dict(cus=0), dict(d=96),
])
def test_decode_plan_rejects(args):
    kw = dict(lens=[10], hq=4, hkv=2, d=128, cus=256)
    kw.update(args)
    st, _, _ = _plan(kw["lens"], kw["hq"], kw["hkv"], kw["d"], kw["cus"])
    assert st in (fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED)


def _prefill(**kw):
    base = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, o=ALIGNED, lse=ALIGNED, row_sum=None,
                B=1, Sq=128, Skv=128, Hq=4, Hkv=2, D=128, dtype=0, causal=1, scale=0.125,
                unnorm=0, qs=(128 * 4 * 128, 4 * 128, 128), ks=(128 * 2 * 128, 2 * 128, 128),
                os=(128 * 4 * 128, 4 * 128, 128), ws=ALIGNED, wsb=1 << 40, lens=None, win=0,
                sink=None)
    base.update(kw)
    b = base
    lib = fa.load_library()
    return lib.fa_prefill_fwd(b["q"], *b["qs"], b["k"], *b["ks"], b["v"], *b["ks"],
                              b["o"], *b["os"], b["lse"], b["row_sum"], b["B"], b["Sq"],
                              b["Skv"], b["Hq"], b["Hkv"], b["D"], b["dtype"], b["causal"],
                              b["scale"], b["unnorm"], b["lens"], b["win"], b["sink"], b["ws"],
                              b["wsb"], None)


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lse=None), 1), (dict(unnorm=1), 1),
    (dict(B=0), 1), (dict(Sq=0), 1), (dict(Skv=64), 1), (dict(Hkv=3), 1), (dict(Hq=0), 1),
    (dict(D=96), 2), (dict(D=1024), 2), (dict(dtype=7), 2),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=0.0), 1),
    (dict(scale=-1.0), 1), (dict(q=ALIGNED + 2), 1), (dict(o=ALIGNED + 4), 1),
    (dict(qs=(128 * 4 * 128, 4 * 128 + 4, 128)), 1), (dict(os=(128, 2, 128)), 1),
    (dict(ks=(-8, 256, 128)), 1), (dict(Sq=2**31 - 1, Skv=2**31 - 1, Hq=128), 2),
    # bf16 (and fp16 at head_dim 256) run the V repack: the workspace is checked
    (dict(ws=None, dtype=1), 1), (dict(wsb=1000, dtype=1), 1), (dict(ws=ALIGNED + 16, dtype=1), 1),
    (dict(ws=None, D=256), 1),
    # fp16 at head_dim <= 128 reads V's rows: no workspace needed; the call passes
    # its host checks and fails only at the launch (no GPU here)
    (dict(ws=None, wsb=0), 3), (dict(ws=None, wsb=0, D=64), 3),
    (dict(win=-1), 1), (dict(lens=ALIGNED + 2), 1), (dict(sink=ALIGNED + 2), 1),
])
def test_prefill_validation(kw, status):
    st = _prefill(**kw)
    assert st == status, fa.load_library().fa_last_error()
    assert fa.load_library().fa_last_error() != b""


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(v=None), 1), (dict(B=0), 1), (dict(Skv=0), 1), (dict(D=96), 2), (dict(dtype=3), 2),
    (dict(v=ALIGNED + 2), 1), (dict(vs=(128 * 2 * 128, 2 * 128 + 4, 128)), 1),
    (dict(ws=None), 1), (dict(wsb=1000), 1), (dict(ws=ALIGNED + 64), 1),
])
def test_prefill_pack_v_validation(kw, status):
    b = dict(v=ALIGNED, vs=(128 * 2 * 128, 2 * 128, 128), B=1, Skv=128, Hkv=2, D=128, dtype=0,
             ws=ALIGNED, wsb=1 << 40)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_prefill_pack_v(b["v"], *b["vs"], b["B"], b["Skv"], b["Hkv"], b["D"], b["dtype"],
                               b["ws"], b["wsb"], None)
    assert st == status, lib.fa_last_error()


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(lse=None), 1), (dict(unnorm=1), 1),
    (dict(Skv=64), 1), (dict(Hkv=3), 1), (dict(D=1024), 2), (dict(scale=0.0), 1),
    (dict(ws=None), 1), (dict(wsb=1000), 1), (dict(qs=(128 * 4 * 128, 4 * 128 + 4, 128)), 1),
    (dict(win=-3), 1), (dict(lens=ALIGNED + 1), 1),
])
def test_prefill_fwd_packed_validation(kw, status):
    b = dict(q=ALIGNED, k=ALIGNED, o=ALIGNED, lse=ALIGNED, row_sum=None, B=1, Sq=128, Skv=128,
             Hq=4, Hkv=2, D=128, dtype=0, causal=1, scale=0.125, unnorm=0,
             qs=(128 * 4 * 128, 4 * 128, 128), ks=(128 * 2 * 128, 2 * 128, 128),
             os=(128 * 4 * 128, 4 * 128, 128), ws=ALIGNED, wsb=1 << 40, lens=None, win=0,
             sink=None)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_prefill_fwd_packed(b["q"], *b["qs"], b["k"], *b["ks"], b["o"], *b["os"],
                                   b["lse"], b["row_sum"], b["B"], b["Sq"], b["Skv"], b["Hq"],
                                   b["Hkv"], b["D"], b["dtype"], b["causal"], b["scale"],
                                   b["unnorm"], b["lens"], b["win"], b["sink"], b["ws"],
                                   b["wsb"], None)
    assert st == status, lib.fa_last_error()


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lens=None), 1), (dict(Hkv=3), 1), (dict(D=80), 2),
    (dict(dtype=2), 2), (dict(split=0), 1), (dict(split=24), 1), (dict(ms=0), 1),
    (dict(scale=float("nan")), 1), (dict(k=ALIGNED + 8), 1), (dict(st=100), 1),
])
def test_decode_partial_validation(kw, status):
    b = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, offs=ALIGNED, lens=ALIGNED, po=ALIGNED,
             pl=ALIGNED, B=1, Hq=4, Hkv=2, D=128, dtype=0, scale=0.1, split=32, ms=4, st=256)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_decode_split_partial(b["q"], 512, 128, b["k"], b["v"], b["st"], 128, b["offs"],
                                     b["lens"], b["B"], b["Hq"], b["Hkv"], b["D"], b["dtype"],
                                     b["scale"], b["split"], b["ms"], b["po"], b["pl"], None)
    assert st == status


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(po=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(split=0), 1), (dict(ms=0), 1),
    (dict(D=100), 2),
])
def test_decode_merge_validation(kw, status):
    b = dict(po=ALIGNED, pl=ALIGNED, lens=ALIGNED, o=ALIGNED, lse=ALIGNED, B=1, Hq=4, D=128,
             split=32, ms=4)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_decode_merge_lse(b["po"], b["pl"], b["lens"], b["B"], b["Hq"], b["D"],
                                 b["split"], b["ms"], b["o"], b["lse"], None)
    assert st == status


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lens=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(Hkv=3), 1), (dict(D=80), 2), (dict(dtype=2), 2), (dict(split=24), 1), (dict(ms=0), 1),
    (dict(scale=0.0), 1), (dict(ws=None), 1), (dict(wsb=100), 1), (dict(ws=ALIGNED + 64), 1),
    (dict(B=16385, Hq=2, Hkv=2), 2),
])
def test_decode_fused_validation(kw, status):
    b = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, offs=ALIGNED, lens=ALIGNED, o=ALIGNED, lse=ALIGNED,
             B=1, Hq=4, Hkv=2, D=128, dtype=0, scale=0.1, split=32, ms=4, ws=ALIGNED, wsb=1 << 40)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_decode_fused(b["q"], 512, 128, b["k"], b["v"], 256, 128, b["offs"], b["lens"],
                             b["B"], b["Hq"], b["Hkv"], b["D"], b["dtype"], b["scale"],
                             b["split"], b["ms"], b["o"], b["lse"], b["ws"], b["wsb"], None)
    assert st == status, lib.fa_last_error()


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(lse=None), 1), (dict(q=None), 1), (dict(D=96), 2),
    (dict(Hkv=3), 1), (dict(split=24), 1),
    # needs more scratch than the library's 16 MiB array: unsupported, use the workspace form
    (dict(B=64, Hq=32, Hkv=8, ms=64), 2),
    # more arrival counters than the fixed 64 KiB region holds
    (dict(B=20000, Hq=4, Hkv=2, ms=1), 2),
])
def test_decode_fused_noalloc_validation(kw, status):
    # the allocation-free form checks as the workspace form does, plus its
    # scratch limit, all on the host before any HIP call
    b = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, offs=ALIGNED, lens=ALIGNED, o=ALIGNED, lse=ALIGNED,
             B=1, Hq=4, Hkv=2, D=128, dtype=0, scale=0.1, split=32, ms=4)
    b.update(kw)
    lib = fa.load_library()
    assert lib.fa_decode_fused_workspace_size(64, 32, 8, 128, 64) > 16 << 20
    st = lib.fa_decode_fused_noalloc(b["q"], 512, 128, b["k"], b["v"], 256, 128, b["offs"],
                                     b["lens"], b["B"], b["Hq"], b["Hkv"], b["D"], b["dtype"],
                                     b["scale"], b["split"], b["ms"], b["o"], b["lse"], None)
    assert st == status, lib.fa_last_error()


def test_decode_fused_workspace_size():
    lib = fa.load_library()
    # one round of resident waves and more than 16 splits: groups of 4 (latency-bound)
    assert lib.fa_decode_fused_waves(1, 28, 4, 128, 52) == 4
    assert lib.fa_decode_fused_waves(1, 28, 4, 256, 52) == 4
    # 16 splits or fewer, or more than one round (bandwidth-bound): one wave
    assert lib.fa_decode_fused_waves(1, 28, 4, 128, 16) == 1
    assert lib.fa_decode_fused_waves(32, 28, 4, 128, 25) == 1      # 32 x 4 x 25 > 2048
    assert lib.fa_decode_fused_waves(2, 28, 4, 128, 25) == 4       # 2 x 28 x 25 <= 2048
    assert lib.fa_decode_fused_waves(1, 28, 4, 96, 4) == 0
    assert lib.fa_decode_fused_waves(1, 28, 3, 128, 4) == 0

    def up(x):
        return (x + 255) // 256 * 256
    # 1 sequence, 28/4 heads (7 per wave -> 4 head groups), 52 splits -> 13 work-groups
    want = 65536 + up(28 * 13 * 4) + up(28 * 13 * 128 * 4)     # fixed counter region first
    assert lib.fa_decode_fused_workspace_size(1, 28, 4, 128, 52) == want
    # 32 sequences, 32/8 heads (4 per wave), head_dim 256, 40 splits: more than one
    # round of resident waves -> one split per work-group
    want = 65536 + up(32 * 32 * 40 * 4) + up(32 * 32 * 40 * 256 * 4)
    assert lib.fa_decode_fused_workspace_size(32, 32, 8, 256, 40) == want
    # 13 splits: one per work-group
    want = 65536 + up(32 * 32 * 13 * 4) + up(32 * 32 * 13 * 128 * 4)
    assert lib.fa_decode_fused_workspace_size(32, 32, 8, 128, 13) == want
    assert lib.fa_decode_fused_workspace_size(1, 4, 3, 128, 4) == 0
    assert lib.fa_decode_fused_workspace_size(1, 4, 2, 96, 4) == 0


@pytest.mark.skipif("_gpu_visible()", reason="host-validation probes run only without a GPU")
@pytest.mark.parametrize("kw,status", [
    (dict(oa=None), 1), (dict(la=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(ob=ALIGNED, lb=None), 1), (dict(ob=None, lb=ALIGNED), 1), (dict(B=0), 1),
    (dict(D=96), 2), (dict(oa=ALIGNED + 4), 1), (dict(sink=ALIGNED + 1), 1),
    (dict(oas=(512, 128, 130)), 1), (dict(os_=(-4, 128, 128)), 1),
])
def test_attn_merge_validation(kw, status):
    b = dict(oa=ALIGNED, oas=(512 * 4, 512, 128), la=ALIGNED, ob=ALIGNED, obs=(512 * 4, 512, 128),
             lb=ALIGNED, sink=None, B=1, S=4, H=4, D=128, o=ALIGNED, os_=(512 * 4, 512, 128),
             lse=ALIGNED)
    b.update(kw)
    lib = fa.load_library()
    st = lib.fa_attn_merge(b["oa"], *b["oas"], b["la"], b["ob"], *b["obs"], b["lb"], b["sink"],
                           b["B"], b["S"], b["H"], b["D"], b["o"], *b["os_"], b["lse"], None)
    assert st == status, lib.fa_last_error()


def test_workspace_size():
    lib = fa.load_library()
    assert lib.fa_prefill_workspace_size(1, 3314, 4, 128) == 1 * 4 * 52 * 64 * 128 * 2
    assert lib.fa_prefill_workspace_size(2, 64, 1, 64) == 2 * 1 * 1 * 64 * 64 * 2
    assert lib.fa_prefill_workspace_size(1, 100, 2, 256) == 1 * 2 * 4 * 32 * 256 * 2   # 32-key tiles
    assert lib.fa_prefill_workspace_size(1, 70, 2, 256) == 1 * 2 * 3 * 32 * 256 * 2
    assert lib.fa_prefill_workspace_size(0, 64, 1, 64) == 0
    assert lib.fa_prefill_workspace_size(1, 100, 2, 512) == 1 * 2 * 4 * 32 * 512 * 2   # 32-key tiles


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((1, 8, 1, 64), dtype=torch.float16)
    with pytest.raises(fa.FAError):
        fa.prefill(q, q, q)


def test_binding_rejects_bad_host_arguments():
    """The binding's own checks fire before any library call (no GPU needed)."""
    import torch
    o = torch.zeros((1, 4, 2, 64))
    lse = torch.zeros((1, 2, 4))
    with pytest.raises(fa.FAError):
        fa.attn_merge(o, lse)                              # CPU tensors
    with pytest.raises(fa.FAError):
        fa.attn_merge(o, lse, o_b=o)                       # o_b without lse_b
    q = torch.zeros((1, 4, 64), dtype=torch.float16)
    kc = torch.zeros((8, 2, 64), dtype=torch.float16)
    lens = torch.tensor([8], dtype=torch.int32)
    offs = torch.tensor([0], dtype=torch.int64)
    with pytest.raises(fa.FAError):
        fa.decode_fused(q, kc, kc, offs, lens, split_len=16, max_splits=1)
    with pytest.raises(fa.FAError):
        fa.prefill(torch.zeros((1, 8, 2, 64), dtype=torch.float16),
                   torch.zeros((1, 8, 1, 64), dtype=torch.float16),
                   torch.zeros((1, 8, 1, 64), dtype=torch.float16), window=-1)
