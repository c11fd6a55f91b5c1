"""Build libfa.so (gfx950 only) in-tree with hipcc.

    python -m flashattention_attention_amd.build [--resource-usage]

The library is written next to this file; the Python binding loads it from
there. Every build compiles from scratch (a few tens of seconds).

Every build also records the compiler's per-kernel resource report (registers,
scratch bytes per lane, waves per SIMD, LDS bytes) in
_build/kernel_resources.json: the attention kernels run at two waves per SIMD
with the whole register budget in use, and a spill inside a tile loop stalls
the K/V prefetch (its reload waits on every DMA in flight), so the report is
checked by the test suite. --resource-usage prints the raw remarks as well.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_prefill.hip", "fa_decode.hip", "fa_merge.hip"]
ARCH = "gfx950"
# Per-source flags. The decode kernels keep their MFMA accumulators in VGPRs
# (the AGPR form made the register allocator copy every accumulator between
# the two files on each block, which cost the multi-head decode its second
# wave per SIMD).
EXTRA = {"fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed-FP32 VALU ops stay disabled on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


RESOURCES = os.path.join(PKG, "_build", "kernel_resources.json")
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
           "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "waves_per_simd",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text: str) -> dict:
    """{mangled kernel name: {field: int}} from -Rpass-analysis=kernel-resource-usage."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark:\s+(.*?)\s+\[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        body = m.group(1)
        if body.startswith("Function Name: "):
            cur = out.setdefault(body[len("Function Name: "):].strip(), {})
            continue
        key, _, val = body.rpartition(": ")
        if cur is not None and key.strip() in _FIELDS and val.strip().lstrip("-").isdigit():
            cur[_FIELDS[key.strip()]] = int(val)
    return out


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    objs = []
    resources = {}
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in SOURCES:   # the sources compile concurrently (one process each)
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        hip = src.endswith(".hip")
        lang = ["-x", "hip"] if hip else []
        extra = (["-Rpass-analysis=kernel-resource-usage"] if hip else []) + EXTRA.get(src, [])
        cmd = [hipcc()] + compile_flags() + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, hip, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                      stderr=subprocess.PIPE, text=True)))
    for src, hip, obj, proc in procs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}\n{err}")
        if hip:
            resources.update(parse_resource_remarks(err))
        if resource_usage or verbose:
            sys.stdout.write(err)
        objs.append(obj)
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp_lib = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    path = build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv)
    print("built", path)
