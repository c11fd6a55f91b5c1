"""The compiler's resource report for the attention kernels (CPU only).

The prefill kernels are built for two waves per SIMD, i.e. 256 registers per
lane, and sit at that budget. A spill inside a tile loop is reloaded through
vector memory, and the wait for that reload also waits for the K/V tile DMAs
in flight, so the prefetch serialises behind the compute (the head_dim 512
kernel once lost a quarter of its speed that way). build() records the
compiler's per-kernel report (_build/kernel_resources.json); these tests pin
the properties the measured speeds rely on. They skip where the library has
not been built in this tree.
"""
import json
import os

import pytest

from flashattention_attention_amd import build


def _report():
    if not os.path.exists(build.RESOURCES):
        pytest.skip("library not built in this tree (run build() first)")
    with open(build.RESOURCES) as f:
        return json.load(f)


def _pick(rep, *needles):
    return {k: v for k, v in rep.items() if any(n in k for n in needles)}


def test_parse_resource_remarks():
    text = "\n".join([
        "a.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 130 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 3 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     LDS Size [bytes/block]: 65536 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: warning: unrelated",
    ])
    assert build.parse_resource_remarks(text) == {
        "_Z3fooPf": {"vgprs": 130, "scratch_bytes": 16, "waves_per_simd": 3},
        "_Z3barv": {"lds_bytes": 65536},
    }


def test_prefill_kernels_run_two_waves_without_scratch():
    rep = _report()
    ks = _pick(rep, "prefill_kernelILi64E", "prefill_kernelILi128E", "prefill_kernelILi256E",
               "prefill512_kernel")
    # head_dim 64 and 128: {bf16, fp16} x {normalized, un-normalized} x {1, 2 heads},
    # plus the key-split form ({bf16, fp16} x {1, 2 heads}, normalized), the
    # fp16 form that reads V's rows ({normalized, un-normalized} x {1, 2 heads})
    # and, at head_dim 128 with one head per work-group, the three-per-CU form
    # ({bf16, fp16} x {normalized, un-normalized});
    # head_dim 256 and 512: {bf16, fp16} x {normalized, un-normalized}
    # (template arguments: D, bf16, exact max, heads, split, V rows, three per CU)
    assert len(ks) == 44, sorted(ks)
    assert len([k for k in ks if "ELb1ELb0ELb0EEEvNS" in k]) == 8, sorted(ks)
    vrow = [k for k in ks if "ELb0ELb1ELb0EEEvNS" in k]
    assert len(vrow) == 8 and all("ILi64ELb0E" in k or "ILi128ELb0E" in k for k in vrow), vrow
    trio = [k for k in ks if "ELb0ELb0ELb1EEEvNS" in k]
    assert len(trio) == 4 and all("ILi128E" in k and "ELi1ELb0ELb0ELb1EEEvNS" in k
                                  for k in trio), trio
    for name, r in ks.items():
        assert r["scratch_bytes"] == 0 and r["vgpr_spill"] == 0, (name, r)
        if name in trio:
            # three work-groups of four waves per compute unit
            assert r["waves_per_simd"] == 3 and r["lds_bytes"] <= 160 * 1024 // 3, (name, r)
        else:
            assert r["waves_per_simd"] == 2, (name, r)
            assert r["lds_bytes"] <= 160 * 1024, (name, r)
    # head_dim 256 keeps its tile stages and O staging within 80 KB, so two
    # work-groups share a compute unit
    for name, r in _pick(rep, "prefill_kernelILi256E").items():
        assert r["lds_bytes"] <= 80 * 1024, (name, r)


def test_benchmarked_decode_kernels_keep_occupancy():
    # The fp16 decode instances the benchmark times: group of 4 (long decode,
    # both forms) and one head per wave (the 1641-token decode, both forms).
    rep = _report()
    for needle in ("decode_partial_kernelILi128ELi4ELb0EE", "decode_partial_kernelILi128ELi1ELb0EE",
                   "decode_fused_kernelILi128ELi4ELb0ELi1EE",
                   "decode_fused_kernelILi128ELi1ELb0ELi4EE"):
        ks = _pick(rep, needle)
        assert len(ks) == 1, (needle, sorted(ks))
        (name, r), = ks.items()
        assert r["scratch_bytes"] == 0 and r["waves_per_simd"] >= 2, (name, r)
    for name, r in _pick(rep, "decode_", "branch_merge_kernel", "vt_pack_kernel").items():
        assert r["scratch_bytes"] == 0, (name, r)
