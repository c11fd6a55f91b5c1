"""MI355X-native exact attention: causal GQA prefill and split-KV decode.

The compute lives in a C-ABI shared library (``libfa.so``, declared in
``include/fa.h``) built from hand-written gfx950 HIP kernels. The Python layer
only marshals torch device tensors into that ABI; it is loaded on first use so
that ``inputs`` can be imported without a built library.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "prefill", "decode_plan", "decode_split_partial", "decode_merge_lse",
           "decode", "library_path"]


def __getattr__(name):
    if name in ("prefill", "decode_plan", "decode_split_partial", "decode_merge_lse", "decode",
                "library_path", "FAError", "load_library"):
        from . import fa as _fa
        return getattr(_fa, name)
    raise AttributeError(name)
