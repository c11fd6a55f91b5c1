"""fp64 CPU oracle for attention prefill, split-KV decode and the LSE merge.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The product path never does.
"""
from .attention import (attend_rows, decode, decode_split_partials, half_to_f64,
                        merge_branches, merge_partials, num_splits, prefill)

__all__ = ["attend_rows", "decode", "decode_split_partials", "half_to_f64",
           "merge_branches", "merge_partials", "num_splits", "prefill"]
