"""Python binding of libfa.so (argument marshalling only).

Each function here takes torch tensors that live on an AMD GPU, checks the
shapes and devices, allocates outputs with torch when the caller did not pass
them, and calls the C ABI declared in ``include/fa.h`` on torch's current
HIP stream. Every step of the attention computation runs in the library's
HIP kernels; there is no fallback path. If the library is missing, or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "fa.h")
_lib = None

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F16, FA_BF16 = 0, 1

_i64, _i32, _f32, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_SIGNATURES = {
    "fa_prefill_fwd": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                        _vp, _i64, _i64, _i64, _vp, _vp,
                        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                        _vp, _i32, _vp, _vp, ctypes.c_uint64, _vp], _i32),
    "fa_prefill_pack_v": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                           _vp, ctypes.c_uint64, _vp], _i32),
    "fa_prefill_fwd_packed": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                               _vp, _i64, _i64, _i64, _vp, _vp,
                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                               _vp, _i32, _vp, _vp, ctypes.c_uint64, _vp], _i32),
    "fa_prefill_fwd_packed_split": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                     _vp, _i64, _i64, _i64, _vp, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                     _vp, _i32, _vp, _vp, ctypes.c_uint64, _vp, ctypes.c_uint64,
                                     _vp], _i32),
    "fa_prefill_split_workspace_size": ([_i32, _i32, _i32, _i32], ctypes.c_uint64),
    "fa_prefill_split_units": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                ctypes.POINTER(ctypes.c_uint16), _i32], _i32),
    "fa_prefill_trio": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32], _i32),
    "fa_attn_merge": ([_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp,
                       _i32, _i32, _i32, _i32, _vp, _i64, _i64, _i64, _vp, _vp], _i32),
    "fa_prefill_workspace_size": ([_i32, _i32, _i32, _i32], ctypes.c_uint64),
    "fa_decode_plan": ([ctypes.POINTER(ctypes.c_int32), _i32, _i32, _i32, _i32, _i32,
                        ctypes.POINTER(_i32), ctypes.POINTER(_i32)], _i32),
    "fa_decode_split_partial": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp, _vp],
                                _i32),
    "fa_decode_merge_lse": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "fa_decode_fused": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp,
                         _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp,
                         _vp, ctypes.c_uint64, _vp], _i32),
    "fa_decode_fused_noalloc": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp,
                                 _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp,
                                 _vp], _i32),
    "fa_decode_fused_workspace_size": ([_i32, _i32, _i32, _i32, _i32], ctypes.c_uint64),
    "fa_decode_fused_waves": ([_i32, _i32, _i32, _i32, _i32], _i32),
    "fa_status_string": ([_i32], ctypes.c_char_p),
    "fa_last_error": ([], ctypes.c_char_p),
}


class FAError(RuntimeError):
    """A libfa call returned a non-OK status (or the library is unavailable)."""

    def __init__(self, msg: str, status: int = -1):
        super().__init__(msg)
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libfa.so")


def declared_functions() -> list:
    """Names of the functions include/fa.h declares."""
    text = open(_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)


def load_library():
    """Load libfa.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FAError(f"{path} is not built; run `python -m flashattention_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != FA_OK:
        lib = load_library()
        raise FAError(f"{what}: {lib.fa_status_string(status).decode()}: "
                      f"{lib.fa_last_error().decode()}", status)


def _issue(name: str, args: tuple, keep: tuple, prepare: bool):
    """Call the library entry `name` with marshalled `args`, or (prepare=True)
    return a zero-argument callable that re-issues exactly this call: the
    tensors in `keep` stay referenced by it, and no Python-side checks run per
    call (for launch loops where host overhead would starve the GPU)."""
    fn = getattr(load_library(), name)
    if prepare:
        def call(fn=fn, args=args, keep=keep):
            st = fn(*args)
            if st != FA_OK:
                _check(st, name)
        return call
    _check(fn(*args), name)
    return None


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _on_gpu(*tensors: torch.Tensor) -> torch.device:
    dev = None
    for t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise FAError("every tensor argument must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise FAError("all tensors must be on the same GPU")
    return dev


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _prefill_outputs(q, k, dev, out, lse, row_sum, out_unnormalized, want_row_sum):
    if q.dim() != 4 or k.dim() != 4:
        raise FAError("q, k, v must be 4-D [batch, seq, heads, head_dim]")
    if q.dtype != k.dtype:
        raise FAError("q, k, v must share a dtype")
    for t in (q, k):
        if t.stride(3) != 1:
            raise FAError("head_dim must be the contiguous dimension")
    B, Sq, Hq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D:
        raise FAError("q and k disagree on batch or head_dim")
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    need_rs = out_unnormalized or want_row_sum or row_sum is not None
    if need_rs and row_sum is None:
        row_sum = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    _on_gpu(out, lse, *([row_sum] if row_sum is not None else []))
    if out.dtype != torch.float32 or out.shape != (B, Sq, Hq, D) or out.stride(3) != 1:
        raise FAError("out must be fp32 [B,Sq,Hq,D] with contiguous head_dim")
    for t in (lse, row_sum):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, Hq, Sq)
                              or not t.is_contiguous()):
            raise FAError("lse / row_sum must be contiguous fp32 [B,Hq,Sq]")
    return out, lse, row_sum, need_rs


def _masks(kv_lens, window, batch, dev):
    """Marshal the optional length mask (int32 GPU tensor [batch]) and window."""
    window = int(window)
    if window < 0:
        raise FAError("window must be >= 0")
    if kv_lens is None:
        return None, window
    _on_gpu(kv_lens)
    if kv_lens.device != dev:
        raise FAError("kv_lens must be on the same GPU as q")
    if kv_lens.dtype != torch.int32 or kv_lens.shape != (batch,) or not kv_lens.is_contiguous():
        raise FAError("kv_lens must be a contiguous int32 tensor [batch]")
    return kv_lens, window


def _sinks(sink_logits, n_heads, dev):
    """Check the optional per-head sink logits (fp32 GPU tensor [n_heads])."""
    if sink_logits is None:
        return None
    _on_gpu(sink_logits)
    if sink_logits.device != dev:
        raise FAError("sink_logits must be on the same GPU as the other tensors")
    if sink_logits.dtype != torch.float32 or sink_logits.shape != (n_heads,) \
            or not sink_logits.is_contiguous():
        raise FAError("sink_logits must be a contiguous fp32 tensor [n_heads]")
    return sink_logits


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _workspace(k, dev, workspace):
    B, Skv, Hkv, D = k.shape
    ws_need = load_library().fa_prefill_workspace_size(B, Skv, Hkv, D)
    if workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    _on_gpu(workspace)
    if workspace.numel() * workspace.element_size() < ws_need:
        raise FAError(f"workspace holds {workspace.numel()} bytes, {ws_need} needed")
    return workspace


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True,
            softmax_scale: Optional[float] = None, out_unnormalized: bool = False,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            row_sum: Optional[torch.Tensor] = None, want_row_sum: bool = False,
            workspace: Optional[torch.Tensor] = None, kv_lens: Optional[torch.Tensor] = None,
            window: int = 0, sink_logits: Optional[torch.Tensor] = None,
            split_workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """Attention forward. q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] (fp16/bf16, D contiguous).

    ``kv_lens`` (optional int32 GPU tensor [B]) hides keys j >= kv_lens[b];
    ``window`` > 0 hides keys j <= p - window for the query at position p
    (p = row + Skv - Sq). Rows that see no key come back with o = 0,
    lse = -inf. ``sink_logits`` (optional fp32 GPU tensor [Hq]) adds a per-head
    sink term exp(sink) with no value row to every row's softmax.

    ``workspace`` (optional) is a uint8 GPU tensor of at least
    ``prefill_workspace_size(...)`` bytes; one is allocated when omitted, except
    for fp16 inputs at head_dim <= 128, which need none (one launch reads V's
    rows directly).
    ``split_workspace`` (optional, zero-filled before its first use): run as
    prefill_pack_v + prefill_packed with the key split of the longest query
    blocks (see prefill_packed).

    Returns (o, lse) or (o, lse, row_sum) when ``out_unnormalized`` or
    ``want_row_sum``; o is fp32 [B,Sq,Hq,D] (un-normalized when asked), lse and
    row_sum are fp32 [B,Hq,Sq]. With prepare=True (not with split_workspace),
    returns a callable that repeats the call into the same outputs instead.
    """
    dev = _on_gpu(q, k, v)
    if v.dim() != 4 or k.shape != v.shape or v.dtype != k.dtype:
        raise FAError("k and v must have the same shape and dtype")
    if v.stride(3) != 1:
        raise FAError("head_dim must be the contiguous dimension")
    out, lse, row_sum, need_rs = _prefill_outputs(q, k, dev, out, lse, row_sum,
                                                  out_unnormalized, want_row_sum)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    scale = _default_scale(D) if softmax_scale is None else float(softmax_scale)
    kv_lens, window = _masks(kv_lens, window, B, dev)
    sink_logits = _sinks(sink_logits, Hq, dev)
    # fp16 at head_dim <= 128 reads V's rows directly (one launch, no workspace)
    direct = q.dtype == torch.float16 and D <= 128 and split_workspace is None
    if not direct or workspace is not None:
        workspace = _workspace(k, dev, workspace)
    if split_workspace is not None:
        if prepare:
            raise FAError("prepare=True is not offered with split_workspace")
        prefill_pack_v(v, workspace)
        return prefill_packed(q, k, workspace, causal=causal, softmax_scale=scale,
                              out_unnormalized=out_unnormalized, out=out, lse=lse,
                              row_sum=row_sum, want_row_sum=want_row_sum, kv_lens=kv_lens,
                              window=window, sink_logits=sink_logits,
                              split_workspace=split_workspace)
    args = (q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
            k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
            v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
            out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
            lse.data_ptr(), row_sum.data_ptr() if row_sum is not None else None,
            B, Sq, Skv, Hq, Hkv, D, _dtype_code(q), 1 if causal else 0, scale,
            1 if out_unnormalized else 0, _ptr(kv_lens), window, _ptr(sink_logits),
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            _stream(dev))
    keep = (q, k, v, out, lse, row_sum, kv_lens, sink_logits, workspace)
    call = _issue("fa_prefill_fwd", args, keep, prepare)
    if prepare:
        return call
    return (out, lse, row_sum) if need_rs else (out, lse)


def prefill_pack_v(v: torch.Tensor, workspace: Optional[torch.Tensor] = None, *,
                   prepare: bool = False):
    """Repack V [B,Skv,Hkv,D] into a prefill workspace (returned) for prefill_packed.
    With prepare=True, returns a callable that repeats the call instead."""
    dev = _on_gpu(v)
    if v.dim() != 4 or v.stride(3) != 1:
        raise FAError("v must be 4-D [batch, seq, heads, head_dim] with contiguous head_dim")
    workspace = _workspace(v, dev, workspace)
    B, Skv, Hkv, D = v.shape
    call = _issue("fa_prefill_pack_v", (
        v.data_ptr(), v.stride(0), v.stride(1), v.stride(2), B, Skv, Hkv, D, _dtype_code(v),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(dev)),
        (v, workspace), prepare)
    return call if prepare else workspace


def prefill_packed(q: torch.Tensor, k: torch.Tensor, packed_v: torch.Tensor, *,
                   causal: bool = True, softmax_scale: Optional[float] = None,
                   out_unnormalized: bool = False, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, row_sum: Optional[torch.Tensor] = None,
                   want_row_sum: bool = False, kv_lens: Optional[torch.Tensor] = None,
                   window: int = 0, sink_logits: Optional[torch.Tensor] = None,
                   split_workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """prefill() with V taken from a workspace filled by prefill_pack_v (same shapes).
    With split_workspace (a zero-filled uint8 GPU tensor of at least
    prefill_split_workspace_size(...) bytes, reusable across calls of any shape
    it is large enough for: its arrival counters sit at a fixed place), the key
    ranges of the longest query blocks are split over two work-groups
    (fa_prefill_fwd_packed_split). With prepare=True, returns a callable that
    repeats the call (pass the outputs)."""
    dev = _on_gpu(q, k, packed_v)
    out, lse, row_sum, need_rs = _prefill_outputs(q, k, dev, out, lse, row_sum,
                                                  out_unnormalized, want_row_sum)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    scale = _default_scale(D) if softmax_scale is None else float(softmax_scale)
    kv_lens, window = _masks(kv_lens, window, B, dev)
    sink_logits = _sinks(sink_logits, Hq, dev)
    args = (q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
            k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
            out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
            lse.data_ptr(), row_sum.data_ptr() if row_sum is not None else None,
            B, Sq, Skv, Hq, Hkv, D, _dtype_code(q), 1 if causal else 0, scale,
            1 if out_unnormalized else 0, _ptr(kv_lens), window, _ptr(sink_logits),
            packed_v.data_ptr(), packed_v.numel() * packed_v.element_size())
    keep = (q, k, packed_v, out, lse, row_sum, kv_lens, sink_logits)
    if split_workspace is None:
        call = _issue("fa_prefill_fwd_packed", args + (_stream(dev),), keep, prepare)
    else:
        _on_gpu(split_workspace)
        call = _issue("fa_prefill_fwd_packed_split",
                      args + (split_workspace.data_ptr(),
                              split_workspace.numel() * split_workspace.element_size(),
                              _stream(dev)), keep + (split_workspace,), prepare)
    if prepare:
        return call
    return (out, lse, row_sum) if need_rs else (out, lse)


def attn_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: Optional[torch.Tensor] = None,
               lse_b: Optional[torch.Tensor] = None, *,
               sink_logits: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, prepare: bool = False):
    """Merge two attention passes (and/or a per-head sink) by LSE.

    o_a, o_b: fp32 [B,S,H,D] (D contiguous; decode outputs [B,H,D] count as
    S = 1), lse_a, lse_b: fp32 [B,H,S] (or [B,H]); sink_logits fp32 [H].
    ``out``/``lse`` may be o_a/lse_a (in place). Returns (o, lse), or with
    prepare=True a callable that repeats the call."""
    squeeze = o_a.dim() == 3
    if squeeze:                                  # decode layout: one query per sequence
        o_a, lse_a = o_a.unsqueeze(1), lse_a.unsqueeze(2)
        o_b = o_b.unsqueeze(1) if o_b is not None else None
        lse_b = lse_b.unsqueeze(2) if lse_b is not None else None
        out = out.unsqueeze(1) if out is not None else None
        lse = lse.unsqueeze(2) if lse is not None else None
    if (o_b is None) != (lse_b is None):
        raise FAError("o_b and lse_b go together")
    dev = _on_gpu(o_a, lse_a, *[t for t in (o_b, lse_b) if t is not None])
    if o_a.dim() != 4:
        raise FAError("o_a must be [B,S,H,D] or [B,H,D]")
    B, S, H, D = o_a.shape
    for t in (o_a, o_b):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, S, H, D)
                              or t.stride(3) != 1):
            raise FAError("o_a / o_b must be fp32 of one shape with contiguous head_dim")
    for t in (lse_a, lse_b):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, S)
                              or not t.is_contiguous()):
            raise FAError("lse_a / lse_b must be contiguous fp32 [B,H,S]")
    sink_logits = _sinks(sink_logits, H, dev)
    if out is None:
        out = torch.empty_like(o_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    _on_gpu(out, lse)
    if out.dtype != torch.float32 or out.shape != (B, S, H, D) or out.stride(3) != 1 \
            or lse.dtype != torch.float32 or lse.shape != (B, H, S) or not lse.is_contiguous():
        raise FAError("out / lse have the wrong shape, dtype or layout")
    ob_st = o_b.stride()[:3] if o_b is not None else (0, 0, 0)
    call = _issue("fa_attn_merge", (
        o_a.data_ptr(), *o_a.stride()[:3], lse_a.data_ptr(), _ptr(o_b), *ob_st, _ptr(lse_b),
        _ptr(sink_logits), B, S, H, D, out.data_ptr(), *out.stride()[:3], lse.data_ptr(),
        _stream(dev)), (o_a, lse_a, o_b, lse_b, sink_logits, out, lse), prepare)
    if prepare:
        return call
    return (out.squeeze(1), lse.squeeze(2)) if squeeze else (out, lse)


def prefill_workspace_size(batch: int, seqlen_kv: int, n_heads_kv: int, head_dim: int) -> int:
    """Bytes of workspace fa_prefill_fwd needs for these sizes."""
    return int(load_library().fa_prefill_workspace_size(batch, seqlen_kv, n_heads_kv, head_dim))


def prefill_split_workspace_size(batch: int, seqlen_q: int, n_heads_q: int,
                                 head_dim: int) -> int:
    """Bytes of (zero-filled) split workspace fa_prefill_fwd_packed_split needs."""
    return int(load_library().fa_prefill_split_workspace_size(batch, seqlen_q, n_heads_q,
                                                              head_dim))


def prefill_split_units(batch: int, seqlen_q: int, seqlen_kv: int, n_heads_q: int,
                        n_heads_kv: int, head_dim: int, causal: bool = True,
                        window: int = 0) -> list:
    """The split prefill's work order for a shape (host only): a list of
    (query block, kind) longest first, kind 0 = whole block, 1 / 2 = first /
    second half of its key tiles; empty when the call runs unsplit."""
    lib = load_library()
    buf = (ctypes.c_uint16 * 512)()
    n = lib.fa_prefill_split_units(batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv, head_dim,
                                   1 if causal else 0, window, buf, 512)
    _check(-n if n < 0 else 0, "fa_prefill_split_units")
    return [(buf[i] & 0x3FFF, buf[i] >> 14) for i in range(n)]


def prefill_trio(batch: int, seqlen_q: int, seqlen_kv: int, n_heads_q: int, n_heads_kv: int,
                 head_dim: int, causal: bool = True, window: int = 0) -> bool:
    """Whether the two-launch prefill's attention runs three work-groups per
    compute unit for this shape (host only)."""
    r = load_library().fa_prefill_trio(batch, seqlen_q, seqlen_kv, n_heads_q, n_heads_kv,
                                       head_dim, 1 if causal else 0, window)
    _check(-r if r < 0 else 0, "fa_prefill_trio")
    return r == 1


def decode_plan(kv_lens: Sequence[int], n_heads_q: int, n_heads_kv: int, head_dim: int,
                num_cus: Optional[int] = None) -> Tuple[int, int]:
    """Deterministic (split_len, max_splits) for host-known KV lengths."""
    lens = [int(x) for x in kv_lens]
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    arr = (ctypes.c_int32 * len(lens))(*lens)
    lib = load_library()
    sl, ms = _i32(), _i32()
    st = lib.fa_decode_plan(arr, len(lens), n_heads_q, n_heads_kv, head_dim, num_cus,
                            ctypes.byref(sl), ctypes.byref(ms))
    _check(st, "fa_decode_plan")
    return sl.value, ms.value


def decode_split_partial(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         kv_offsets: torch.Tensor, kv_lens: torch.Tensor, *, split_len: int,
                         max_splits: int, softmax_scale: Optional[float] = None,
                         part_o: Optional[torch.Tensor] = None,
                         part_lse: Optional[torch.Tensor] = None, prepare: bool = False):
    """Split partials. q [B,Hq,D]; caches [T,Hkv,D]; kv_offsets int64 [B]; kv_lens int32 [B].
    With prepare=True, returns a callable that repeats the call instead.

    Returns part_o fp32 [B,Hq,max_splits,D] and part_lse fp32 [B,Hq,max_splits]
    (entries of empty splits are left untouched).
    """
    dev = _check_decode_inputs(q, k_cache, v_cache, kv_offsets, kv_lens)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    scale = _default_scale(D) if softmax_scale is None else float(softmax_scale)
    if part_o is None:
        part_o = torch.empty((B, Hq, max_splits, D), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, max_splits), dtype=torch.float32, device=dev)
    _on_gpu(part_o, part_lse)
    if (part_o.shape != (B, Hq, max_splits, D) or not part_o.is_contiguous()
            or part_o.dtype != torch.float32 or part_lse.shape != (B, Hq, max_splits)
            or not part_lse.is_contiguous() or part_lse.dtype != torch.float32):
        raise FAError("part_o / part_lse have the wrong shape, dtype or layout")
    call = _issue("fa_decode_split_partial", (
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), kv_offsets.data_ptr(), kv_lens.data_ptr(),
        B, Hq, Hkv, D, _dtype_code(q), scale, split_len, max_splits,
        part_o.data_ptr(), part_lse.data_ptr(), _stream(dev)),
        (q, k_cache, v_cache, kv_offsets, kv_lens, part_o, part_lse), prepare)
    return call if prepare else (part_o, part_lse)


def _check_decode_inputs(q, k_cache, v_cache, kv_offsets, kv_lens):
    dev = _on_gpu(q, k_cache, v_cache, kv_offsets, kv_lens)
    if q.dim() != 3 or k_cache.dim() != 3 or k_cache.shape != v_cache.shape:
        raise FAError("q must be [B,Hq,D] and the caches [T,Hkv,D] of equal shape")
    if k_cache.stride() != v_cache.stride():
        raise FAError("k_cache and v_cache must share strides")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise FAError("q and the caches must share a dtype")
    if kv_offsets.dtype != torch.int64 or kv_lens.dtype != torch.int32:
        raise FAError("kv_offsets must be int64 and kv_lens int32")
    if q.stride(2) != 1 or k_cache.stride(2) != 1:
        raise FAError("head_dim must be contiguous")
    B, Hq, D = q.shape
    if k_cache.shape[2] != D or kv_offsets.shape != (B,) or kv_lens.shape != (B,):
        raise FAError("shape mismatch between q, caches, kv_offsets and kv_lens")
    if not (kv_offsets.is_contiguous() and kv_lens.is_contiguous()):
        raise FAError("kv_offsets and kv_lens must be contiguous")
    return dev


def decode_fused_workspace_size(batch: int, n_heads_q: int, n_heads_kv: int, head_dim: int,
                                max_splits: int) -> int:
    """Bytes of (zero-filled) workspace fa_decode_fused needs."""
    return int(load_library().fa_decode_fused_workspace_size(batch, n_heads_q, n_heads_kv,
                                                             head_dim, max_splits))


def decode_fused(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 kv_offsets: torch.Tensor, kv_lens: torch.Tensor, *, split_len: int,
                 max_splits: int, softmax_scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, prepare: bool = False):
    """Split-KV decode in one launch. Same inputs as decode_split_partial; returns
    o fp32 [B,Hq,D] and lse fp32 [B,Hq] (or, with prepare=True, a callable that
    repeats the call). ``workspace``: a uint8 GPU tensor of at least
    decode_fused_workspace_size(...) bytes that was zero-filled before its
    first use (torch.zeros); one is allocated when omitted."""
    dev = _check_decode_inputs(q, k_cache, v_cache, kv_offsets, kv_lens)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    scale = _default_scale(D) if softmax_scale is None else float(softmax_scale)
    need = decode_fused_workspace_size(B, Hq, Hkv, D, max_splits)
    if workspace is None:
        workspace = torch.zeros(max(1, need), dtype=torch.uint8, device=dev)
    _on_gpu(workspace)
    if workspace.numel() * workspace.element_size() < need:
        raise FAError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _on_gpu(out, lse)
    if out.shape != (B, Hq, D) or lse.shape != (B, Hq) or not out.is_contiguous() \
            or not lse.is_contiguous() or out.dtype != torch.float32 \
            or lse.dtype != torch.float32:
        raise FAError("out / lse must be contiguous fp32 [B,Hq,D] / [B,Hq]")
    call = _issue("fa_decode_fused", (
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), kv_offsets.data_ptr(), kv_lens.data_ptr(),
        B, Hq, Hkv, D, _dtype_code(q), scale, split_len, max_splits,
        out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(dev)),
        (q, k_cache, v_cache, kv_offsets, kv_lens, out, lse, workspace), prepare)
    return call if prepare else (out, lse)


DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_fused_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         kv_offsets: torch.Tensor, kv_lens: torch.Tensor, *, split_len: int,
                         max_splits: int, softmax_scale: Optional[float] = None,
                         out: torch.Tensor, lse: torch.Tensor, prepare: bool = False):
    """decode_fused with the library's own scratch (fa_decode_fused_noalloc):
    the caller passes the outputs (contiguous fp32 [B,Hq,D] and [B,Hq]) and
    nothing is allocated. Calls that overlap in time on one GPU must not be
    issued (they share that GPU's scratch)."""
    dev = _check_decode_inputs(q, k_cache, v_cache, kv_offsets, kv_lens)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    scale = _default_scale(D) if softmax_scale is None else float(softmax_scale)
    _on_gpu(out, lse)
    if out.shape != (B, Hq, D) or lse.shape != (B, Hq) or not out.is_contiguous() \
            or not lse.is_contiguous() or out.dtype != torch.float32 \
            or lse.dtype != torch.float32:
        raise FAError("out / lse must be contiguous fp32 [B,Hq,D] / [B,Hq]")
    call = _issue("fa_decode_fused_noalloc", (
        q.data_ptr(), q.stride(0), q.stride(1), k_cache.data_ptr(), v_cache.data_ptr(),
        k_cache.stride(0), k_cache.stride(1), kv_offsets.data_ptr(), kv_lens.data_ptr(),
        B, Hq, Hkv, D, _dtype_code(q), scale, split_len, max_splits,
        out.data_ptr(), lse.data_ptr(), _stream(dev)),
        (q, k_cache, v_cache, kv_offsets, kv_lens, out, lse), prepare)
    return call if prepare else (out, lse)


def decode_merge_lse(part_o: torch.Tensor, part_lse: torch.Tensor, kv_lens: torch.Tensor, *,
                     split_len: int, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, prepare: bool = False):
    """Merge partials by LSE. Returns o fp32 [B,Hq,D] and lse fp32 [B,Hq]; with
    prepare=True, a callable that repeats the call instead."""
    dev = _on_gpu(part_o, part_lse, kv_lens)
    B, Hq, S, D = part_o.shape
    if part_lse.shape != (B, Hq, S) or kv_lens.shape != (B,) or kv_lens.dtype != torch.int32:
        raise FAError("part_lse / kv_lens shape mismatch")
    if not (part_o.is_contiguous() and part_lse.is_contiguous() and kv_lens.is_contiguous()):
        raise FAError("merge inputs must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _on_gpu(out, lse)
    if out.shape != (B, Hq, D) or lse.shape != (B, Hq) or not out.is_contiguous() \
            or not lse.is_contiguous():
        raise FAError("out / lse shape mismatch")
    call = _issue("fa_decode_merge_lse", (
        part_o.data_ptr(), part_lse.data_ptr(), kv_lens.data_ptr(), B, Hq, D, split_len, S,
        out.data_ptr(), lse.data_ptr(), _stream(dev)), (part_o, part_lse, kv_lens, out, lse),
        prepare)
    return call if prepare else (out, lse)


def decode(q, k_cache, v_cache, kv_offsets, kv_lens, *, split_len: int, max_splits: int,
           softmax_scale: Optional[float] = None, part_o=None, part_lse=None, out=None,
           lse=None):
    """Split partials followed by the LSE merge (two launches on the current stream)."""
    po, pl = decode_split_partial(q, k_cache, v_cache, kv_offsets, kv_lens, split_len=split_len,
                                  max_splits=max_splits, softmax_scale=softmax_scale,
                                  part_o=part_o, part_lse=part_lse)
    return decode_merge_lse(po, pl, kv_lens, split_len=split_len, out=out, lse=lse)
