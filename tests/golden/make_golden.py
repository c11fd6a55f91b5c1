"""Writes tests/golden/generator_sha256.json: SHA-256 of the seeded input bits.

Calls only the seeded input generator (no attention arithmetic, no HIP code).
Run from the repository root: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from flashattention_attention_amd import inputs  # noqa: E402


def main():
    out = {}
    for name in (inputs.TINY_CAUSAL.name, inputs.GQA_PREFILL.name, inputs.GQA_DECODE.name):
        cfg = inputs.WORKLOADS[name]
        data = (inputs.make_prefill_inputs(cfg) if isinstance(cfg, inputs.PrefillConfig)
                else inputs.make_decode_inputs(cfg))
        out[name] = {k: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
                     for k, a in sorted(data.items())}
    rng = np.random.default_rng(inputs.LONG_DECODE.seed)
    lens = inputs.decode_lengths(inputs.LONG_DECODE, rng)
    out[inputs.LONG_DECODE.name] = {"kv_lens": hashlib.sha256(lens.tobytes()).hexdigest(),
                                    "sum_kv_lens": int(lens.astype(np.int64).sum())}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "generator_sha256.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
