"""fp64 CPU oracle for exact scaled-dot-product attention with a causal mask.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never touches it, and
this module imports nothing from the product package.

What it computes is the plain definition, evaluated in float64 on the exact
values of the half-precision inputs:

    s_ij   = scale * sum_d q[i, d] * k[j, d]        for visible keys j
    m_i    = max_j s_ij
    l_i    = sum_j exp(s_ij - m_i)                  (the row sum)
    U_i    = sum_j exp(s_ij - m_i) * v[j, :]        (un-normalized output)
    O_i    = U_i / l_i,     LSE_i = m_i + ln(l_i)   (natural logarithm)

Sources, by page and section:
  * "STAGE_D.md — FMHA Kernel Development", section "Kernel Output": the kernel
    emits the un-normalized output sum(P*V) with P = exp(S*scale - row_max),
    the row sum, and the log-sum-exp; normalizing outside (O = O_unnorm /
    row_sum) is exact. The page writes the LSE with a ln(2) factor on the row
    max, which only holds for a max kept in base-2 units; the reading taken
    here is the natural-log LSE ln(sum_j exp(s_ij)), independent of any
    internal base.
  * Same page, sections D3/D4: a key is masked when its index is greater than
    the query's position (strict comparison), so the diagonal stays visible.
  * "60 · r57 — FA KV staging double buffering (REVERTED)", section 2.2: K/V
    rows are token-major, row p of KV head hk at p*stride + hk*hd + d; query
    head h reads KV head hk. The h -> hk formula is not printed; the reading
    taken is contiguous groups, hk = h // (Hq / Hkv).
  * "66 · D2: explicit K+V register staging ...", sections 1 and 3.2: decode
    splits the KV length into ranges and runs the softmax over each range
    into a partial; the partials are merged by their LSE. The merge formula
    is not printed; the reading taken is the max-shifted form
    M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s,
    LSE = M + ln(sum w_s), which cannot overflow.

Causal alignment when Sq < Skv is not stated on the pages. The reading taken
is bottom-right: query row i sits at absolute position q_pos = i + (Skv - Sq),
so a single decode query sees every key.

Masks beyond causality ("STAGE_D.md — FMHA Kernel Development", D3: a
per-sequence length input masks every key index at or past that sequence's
length; D4: the causal comparison on the same branch). The pages give the two
as independent conditions; the reading taken is that a key is visible only if
every enabled condition admits it:
  * causal:      j <= q_pos;
  * kv_lens[b]:  j <  kv_lens[b] (a per-sequence valid KV length);
  * window W>0:  j >  q_pos - W (a sliding window of the W positions up to and
                 including q_pos; the pages name sliding-window attention but
                 do not spell out its bound, so this is the plainest reading).
A row with no visible key has no softmax; the reading taken (as for an empty
decode split) is O = 0, row_sum = 0, LSE = row_max = -inf.

Sink logits ("STAGE_D.md — FMHA Kernel Development", D5: a sliding-window
pass and a sink merged through their LSEs, the sink merge folded into the
kernel epilogue in D5d). The pages do not define the sink. The reading taken
is a per-head logit sigma_h that joins every row's softmax as one more term
with no value row, i.e. a branch whose LSE is sigma_h and whose output is 0:
    m_i = max(max_j s_ij, sigma_h),  l_i = sum_j exp(s_ij - m_i) + exp(sigma_h - m_i),
    U_i = sum_j exp(s_ij - m_i) v_j,  O_i = U_i / l_i,  LSE_i = m_i + ln(l_i).
A row with no visible key then has O = 0, LSE = sigma_h. Merging the results
of passes over disjoint key sets (merge_branches) is the same max-shifted
LSE merge as for the decode splits.

This is the two-pass form (max first, then exponentials), not an online
softmax, so it is the definition rather than an algorithm that reaches it.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np


# ----------------------------------------------------------------------------
# Half-precision decoding (exact widening to float64).
# ----------------------------------------------------------------------------

def half_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp16 / bf16 bit patterns (numpy uint16)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _as_f64(x, dtype: Optional[str]) -> np.ndarray:
    """Inputs are either half bit patterns (with dtype) or already real numbers."""
    if dtype is None:
        return np.asarray(x, dtype=np.float64)
    return half_to_f64(x, dtype)


# ----------------------------------------------------------------------------
# Attention over one (batch, head): the definition.
# ----------------------------------------------------------------------------

def attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                q_pos: Optional[np.ndarray], visible: Optional[np.ndarray] = None,
                sink: Optional[float] = None) -> dict:
    """Softmax attention of query rows over keys 0..Skv-1, fp64.

    q_rows [R, D]; k, v [Skv, D]; q_pos [R] absolute query positions (causal:
    key j is visible iff j <= q_pos), or None for no causal mask; visible
    [R, Skv] an optional further boolean mask (True = visible); sink an
    optional sink logit (one more softmax term with no value row).
    Returns o, lse, row_sum (l), o_unnorm (U), row_max (m), each per row; a row
    with no visible key and no sink gets o = o_unnorm = 0, row_sum = 0,
    lse = row_max = -inf.
    """
    scores = (q_rows @ k.T) * float(scale)                       # s_ij
    if q_pos is not None:
        masked = np.arange(k.shape[0])[None, :] > np.asarray(q_pos)[:, None]
        scores = np.where(masked, -np.inf, scores)
    if visible is not None:
        scores = np.where(visible, scores, -np.inf)
    m = scores.max(axis=1)                                       # m_i
    if sink is not None:
        m = np.maximum(m, float(sink))
    empty = np.isneginf(m)
    p = np.exp(scores - np.where(empty, 0.0, m)[:, None])        # masked -> exp(-inf) = 0
    l = p.sum(axis=1)                                            # l_i
    if sink is not None:
        l = l + np.exp(float(sink) - np.where(empty, 0.0, m))
    u = p @ v                                                    # U_i
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(empty[:, None], 0.0, u / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return {"o": o, "lse": lse, "row_sum": l, "o_unnorm": u, "row_max": m}


def prefill(q, k, v, *, scale: float, causal: bool = True, dtype: Optional[str] = None,
            rows: Optional[Iterable[int]] = None, kv_lens=None, window: int = 0,
            sink_logits=None) -> dict:
    """Attention forward for the whole problem (or for the query rows listed).

    q [B, Sq, Hq, D]; k, v [B, Skv, Hkv, D]; half bit patterns when ``dtype``
    is given, real numbers otherwise. ``scale`` is the fp32 softmax scale the
    GPU receives; it is widened to float64 unchanged. ``kv_lens`` [B] (valid KV
    length per sequence) and ``window`` (> 0: sliding window) add the masks
    described in the module docstring; ``sink_logits`` [Hq] adds a per-head
    sink logit.

    Returns float64 arrays: o and o_unnorm [B, R, Hq, Dv]; lse, row_sum and
    row_max [B, Hq, R], where R is Sq or len(rows).
    """
    qf, kf, vf = _as_f64(q, dtype), _as_f64(k, dtype), _as_f64(v, dtype)
    B, Sq, Hq, D = qf.shape
    Skv, Hkv = kf.shape[1], kf.shape[2]
    if Hq % Hkv:
        raise ValueError("n_heads_q must be a multiple of n_heads_kv")
    group = Hq // Hkv
    Dv = vf.shape[3]
    rows = np.arange(Sq) if rows is None else np.asarray(list(rows), dtype=np.int64)
    R = rows.shape[0]
    pos = rows + (Skv - Sq)                                      # absolute query positions
    q_pos = pos if causal else None
    keys = np.arange(Skv)
    out = {"o": np.zeros((B, R, Hq, Dv)), "o_unnorm": np.zeros((B, R, Hq, Dv)),
           "lse": np.zeros((B, Hq, R)), "row_sum": np.zeros((B, Hq, R)),
           "row_max": np.zeros((B, Hq, R))}
    for b in range(B):
        visible = None
        if kv_lens is not None or window > 0:
            visible = np.ones((R, Skv), dtype=bool)
            if kv_lens is not None:
                visible &= keys[None, :] < int(kv_lens[b])
            if window > 0:
                visible &= keys[None, :] > (pos[:, None] - int(window))
        for h in range(Hq):
            hk = h // group
            r = attend_rows(qf[b, rows, h, :], kf[b, :, hk, :], vf[b, :, hk, :], scale, q_pos,
                            visible, None if sink_logits is None else float(sink_logits[h]))
            out["o"][b, :, h, :] = r["o"]
            out["o_unnorm"][b, :, h, :] = r["o_unnorm"]
            out["lse"][b, h, :] = r["lse"]
            out["row_sum"][b, h, :] = r["row_sum"]
            out["row_max"][b, h, :] = r["row_max"]
    return out


# ----------------------------------------------------------------------------
# Decode: one query token per sequence against a packed KV cache.
# ----------------------------------------------------------------------------

def _kv_rows(cache, b: int, hk: int, lo: int, hi: int, kv_offsets, dtype):
    base = int(kv_offsets[b])
    return _as_f64(cache[base + lo: base + hi, hk, :], dtype)


def decode(q, k_cache, v_cache, kv_offsets, kv_lens, *, scale: float,
           dtype: Optional[str] = None) -> dict:
    """Unsplit decode attention: every one of the L_b keys is visible.

    q [B, Hq, D]; caches [total_tokens, Hkv, D]. Returns o [B, Hq, D], lse [B, Hq].
    """
    qf = _as_f64(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(kv_lens[b])
        for h in range(Hq):
            hk = h // group
            k = _kv_rows(k_cache, b, hk, 0, L, kv_offsets, dtype)
            v = _kv_rows(v_cache, b, hk, 0, L, kv_offsets, dtype)
            r = attend_rows(qf[b, h][None, :], k, v, scale, None)
            o[b, h] = r["o"][0]
            lse[b, h] = r["lse"][0]
    return {"o": o, "lse": lse}


def num_splits(kv_len: int, split_len: int) -> int:
    """Splits are consecutive ranges of split_len keys; the last may be shorter."""
    return -(-int(kv_len) // int(split_len))


def decode_split_partials(q, k_cache, v_cache, kv_offsets, kv_lens, *, scale: float,
                          split_len: int, max_splits: int, dtype: Optional[str] = None,
                          heads: Optional[Iterable[int]] = None) -> dict:
    """Per-split partials: for split s of sequence b the keys [s*split_len, min(L_b, (s+1)*split_len)).

    Each partial is the attention restricted to its key range: a normalized
    output O_s and its LSE_s. Splits at or past ceil(L_b / split_len) are empty;
    they are reported as LSE = -inf and O = 0 (a merge gives them weight 0).
    Returns part_o [B, Hq, max_splits, D], part_lse [B, Hq, max_splits],
    n_splits [B].
    """
    qf = _as_f64(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    heads = range(Hq) if heads is None else list(heads)
    part_o = np.zeros((B, Hq, max_splits, D))
    part_lse = np.full((B, Hq, max_splits), -np.inf)
    ns = np.zeros(B, dtype=np.int64)
    for b in range(B):
        L = int(kv_lens[b])
        ns[b] = num_splits(L, split_len)
        if ns[b] > max_splits:
            raise ValueError("max_splits too small for this kv length and split_len")
        for h in heads:
            hk = h // group
            for s in range(ns[b]):
                lo, hi = s * split_len, min(L, (s + 1) * split_len)
                k = _kv_rows(k_cache, b, hk, lo, hi, kv_offsets, dtype)
                v = _kv_rows(v_cache, b, hk, lo, hi, kv_offsets, dtype)
                r = attend_rows(qf[b, h][None, :], k, v, scale, None)
                part_o[b, h, s] = r["o"][0]
                part_lse[b, h, s] = r["lse"][0]
    return {"part_o": part_o, "part_lse": part_lse, "n_splits": ns}


def merge_partials(part_o, part_lse, n_splits) -> dict:
    """Combine split partials by their LSE (max-shifted so nothing overflows).

    part_o [B, Hq, S, D], part_lse [B, Hq, S]; only the first n_splits[b]
    partials of sequence b are read. Returns o [B, Hq, D], lse [B, Hq].
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    B, Hq, _, D = part_o.shape
    o = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        n = int(n_splits[b])
        for h in range(Hq):
            ls = part_lse[b, h, :n]
            M = ls.max()
            w = np.exp(ls - M)
            o[b, h] = (w[:, None] * part_o[b, h, :n]).sum(axis=0) / w.sum()
            lse[b, h] = M + math.log(w.sum())
    return {"o": o, "lse": lse}


def merge_branches(o_parts, lse_parts) -> dict:
    """Merge the results of attention passes over disjoint key sets.

    o_parts: list of normalized outputs [..., D]; lse_parts: list of their
    LSEs [...] (same leading shape). Elementwise over the leading shape, the
    max-shifted LSE merge M = max_b LSE_b, w_b = exp(LSE_b - M),
    O = sum_b w_b O_b / sum_b w_b, LSE = M + ln(sum_b w_b). Where every LSE is
    -inf (no key in any pass) the result is O = 0, LSE = -inf. A sink logit
    sigma enters as a branch with O = 0 and LSE = sigma.
    """
    ls = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])      # [n, ...]
    os_ = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])       # [n, ..., D]
    M = ls.max(axis=0)
    empty = np.isneginf(M)
    w = np.exp(ls - np.where(empty, 0.0, M)[None])
    wsum = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(empty[..., None], 0.0,
                     (w[..., None] * os_).sum(axis=0) / np.where(empty, 1.0, wsum)[..., None])
        lse = np.where(empty, -np.inf, M + np.log(np.where(empty, 1.0, wsum)))
    return {"o": o, "lse": lse}
