"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to half precision; it
holds none of the attention arithmetic. Both the fp64 oracle (through the
tests) and the HIP path consume the exact same half-precision bit patterns
produced here, so the two sides never disagree about their inputs.

Recipe (one generator per workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal`` in float32;
  * round-to-nearest-even to fp16 (numpy's float32->float16 cast) or to bf16
    (round-to-nearest-even on the fp32 bit pattern);
  * draw order: per-sequence lengths first (batched decode only), then Q, K, V;
  * the large-head workload multiplies the rounded K by 4, which is exact in
    bf16 and makes the softmax rows peaked.

The workloads stand in for the activations of the pages' 7B model (28 query
heads, 4 KV heads, head_dim 128, a 3314-token prompt, a 1641-token KV cache);
those activations are not available, so i.i.d. N(0, 1) draws of the same
shapes replace them.

Arrays are returned as ``numpy.uint16`` half bit patterns with the layouts the
library's C ABI uses: prefill Q/K/V are [B, S, H, D] (D contiguous); decode q
is [B, Hq, D]; the decode KV cache is packed token-major [sum(L_b), Hkv, D]
with sequence b occupying rows kv_offsets[b] .. kv_offsets[b] + kv_lens[b].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

_CHUNK = 1 << 24  # elements drawn per call; the PCG64 stream is chunk-independent


def round_f32_to_half_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16 or bf16 (round-to-nearest-even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        u = u + 0x7FFF + ((u >> 16) & 1)
        return (u >> 16).astype(np.uint16)
    raise ValueError(f"unknown half dtype {dtype!r}")


def half_bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen half bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown half dtype {dtype!r}")


def draw_half(rng: np.random.Generator, shape: Sequence[int], dtype: str,
              mult: float = 1.0) -> np.ndarray:
    """Draw N(0,1) float32 values in ``shape`` and round them to half bits.

    ``mult`` (a power of two) multiplies the rounded values; that is exact for
    the magnitudes N(0,1) produces.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = round_f32_to_half_bits(x, dtype)
    if mult != 1.0:
        if math.frexp(mult)[0] != 0.5:
            raise ValueError("mult must be a power of two")
        for lo in range(0, n, _CHUNK):
            hi = min(n, lo + _CHUNK)
            out[lo:hi] = round_f32_to_half_bits(
                half_bits_to_f32(out[lo:hi], dtype) * np.float32(mult), dtype)
    return out.reshape(shape)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    seqlen_q: int
    seqlen_kv: int
    dtype: str
    causal: bool
    seed: int
    k_mult: float = 1.0
    out_unnormalized: bool = False
    window: int = 0                        # > 0: sliding window over key positions

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the fp32 value the kernel receives."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask leaves visible, per (batch, head)."""
        sq, skv = self.seqlen_q, self.seqlen_kv
        off = skv - sq  # bottom-right alignment: row i sits at position i + off
        total = 0
        for i in range(sq):
            hi = i + off if self.causal else skv - 1
            lo = max(0, i + off - self.window + 1) if self.window > 0 else 0
            total += max(0, hi - lo + 1)
        return total

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*D for Q.K^T plus 2*D for P.V per visible pair."""
        return 4 * self.head_dim * self.visible_pairs() * self.batch * self.n_heads_q


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    dtype: str
    seed: int
    fixed_len: Optional[int] = None        # every sequence has this KV length
    len_range: Optional[tuple] = None      # else lengths ~ U{lo..hi} drawn from the seed

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


# The five workloads, named by what they are.
TINY_CAUSAL = PrefillConfig("tiny_causal_b1_h1_d64_s128_f16", 1, 1, 1, 64, 128, 128, "f16",
                            True, seed=1)
GQA_PREFILL = PrefillConfig("gqa_causal_prefill_b1_h28kv4_d128_s3314_bf16", 1, 28, 4, 128,
                            3314, 3314, "bf16", True, seed=2)
GQA_DECODE = DecodeConfig("gqa_decode_b1_h28kv4_d128_kv1641_f16", 1, 28, 4, 128, "f16",
                          seed=3, fixed_len=1641)
LONG_DECODE = DecodeConfig("batched_long_decode_b32_h32kv8_d128_kv512to32768_f16", 32, 32, 8,
                           128, "f16", seed=4, len_range=(512, 32768))
# The same lengths with the GQA prompt's heads (28 query / 4 KV: seven query
# heads per wave, the decode form with Q.K^T on the matrix cores).
LONG_DECODE_G7 = DecodeConfig("batched_long_decode_b32_h28kv4_d128_kv512to32768_f16", 32, 28, 4,
                              128, "f16", seed=4, len_range=(512, 32768))
LARGE_HEAD = PrefillConfig("large_head_causal_prefill_b2_h16_d256_s8192_bf16_unnorm", 2, 16, 16,
                           256, 8192, 8192, "bf16", True, seed=5, k_mult=4.0,
                           out_unnormalized=True)
# The GQA prompt under a 1024-position sliding window: about 3/5 of the causal
# pairs, with whole key tiles skipped on the left of every query block.
WINDOW_PREFILL = PrefillConfig("gqa_window1024_causal_prefill_b1_h28kv4_d128_s3314_bf16", 1, 28,
                               4, 128, 3314, 3314, "bf16", True, seed=6, window=1024)

# A 512-wide head with every query head on one KV head (the head-dim budget
# case of the FMHA notes' D1.4; their model is multi-query).
HD512_PREFILL = PrefillConfig("mqa_hd512_causal_prefill_b1_h16kv1_d512_s4096_bf16", 1, 16, 1,
                              512, 4096, 4096, "bf16", True, seed=7)

# A long causal prompt over few heads (8 query heads, one per KV head): 64
# query blocks x 8 heads fill 512 work-group slots once, so the launch runs as
# long as its longest block (128 key tiles) unless long blocks are split.
FEW_HEADS_PREFILL = PrefillConfig("few_heads_causal_prefill_b1_h8_d128_s8192_bf16", 1, 8, 8, 128,
                                  8192, 8192, "bf16", True, seed=7)

WORKLOADS = {c.name: c for c in (TINY_CAUSAL, GQA_PREFILL, GQA_DECODE, LONG_DECODE, LONG_DECODE_G7,
                                 LARGE_HEAD,
                                 WINDOW_PREFILL, HD512_PREFILL, FEW_HEADS_PREFILL)}


def make_prefill_inputs(cfg: PrefillConfig, seed: Optional[int] = None) -> dict:
    """Q, K, V half bit patterns for a prefill workload ([B, S, H, D] each)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = draw_half(rng, (cfg.batch, cfg.seqlen_q, cfg.n_heads_q, cfg.head_dim), cfg.dtype)
    k = draw_half(rng, (cfg.batch, cfg.seqlen_kv, cfg.n_heads_kv, cfg.head_dim), cfg.dtype,
                  mult=cfg.k_mult)
    v = draw_half(rng, (cfg.batch, cfg.seqlen_kv, cfg.n_heads_kv, cfg.head_dim), cfg.dtype)
    return {"q": q, "k": k, "v": v}


def decode_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    if cfg.fixed_len is not None:
        return np.full(cfg.batch, cfg.fixed_len, dtype=np.int32)
    lo, hi = cfg.len_range
    return rng.integers(lo, hi + 1, cfg.batch).astype(np.int32)


def make_decode_inputs(cfg: DecodeConfig, seed: Optional[int] = None) -> dict:
    """q [B,Hq,D], packed K/V cache [sum L, Hkv, D], kv_lens int32 [B], kv_offsets int64 [B]."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lens = decode_lengths(cfg, rng)
    offsets = np.zeros(cfg.batch, dtype=np.int64)
    offsets[1:] = np.cumsum(lens.astype(np.int64))[:-1]
    total = int(lens.astype(np.int64).sum())
    q = draw_half(rng, (cfg.batch, cfg.n_heads_q, cfg.head_dim), cfg.dtype)
    k = draw_half(rng, (total, cfg.n_heads_kv, cfg.head_dim), cfg.dtype)
    v = draw_half(rng, (total, cfg.n_heads_kv, cfg.head_dim), cfg.dtype)
    return {"q": q, "k_cache": k, "v_cache": v, "kv_lens": lens, "kv_offsets": offsets}


def decode_kv_bytes(kv_lens: np.ndarray, n_heads_kv: int, head_dim: int) -> int:
    """Bytes of K plus V a decode pass must read once (2-byte elements)."""
    return int(np.asarray(kv_lens, dtype=np.int64).sum()) * n_heads_kv * head_dim * 2 * 2
