"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole hot path on one model shape (28 query heads,
4 KV heads, head_dim 128): the causal GQA prefill of a 3314-token prompt (bf16)
followed by a single-token split-KV decode against a 1641-token fp16 KV cache
(split partials and their LSE merge, in one launch; the two-launch form is
reported beside it). Inputs are synthetic N(0,1) draws, resident in HBM
before the timed region.

Prints one JSON line. ``value`` is the prefill's algorithmic throughput in
TFLOP/s (4 * head_dim FLOPs per visible query/key pair, per query head) over
both of its launches (V repack + attention), timed with HIP events (without
system fence) on the launch stream; the roofline entry uses the attention
launch alone. The same line carries the
decode timings, the batched long-context decode (32 sequences, 512..32768
tokens), the large-head prefill (head_dim 256, 8192 tokens), the GQA prompt
under a 1024-position sliding window (with and without sinks), a head_dim
512 multi-query prefill and a long few-head prompt with and without the key
split of its longest blocks as extra measurements, a roofline entry per kernel
family, and the fp64 CPU oracle's throughput on a bounded sample of the
prefill workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_DENSE_TFLOPS = 2516.6     # 256 CU x 4096 FLOP/clk x 2.4 GHz (dense)
MI355X_HBM_GBPS = 8000.0


def _dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).cuda()


class _HipEvent:
    """A HIP timing event recorded on the current stream without the
    system-scope release fence that a default event adds (that fence costs a
    few microseconds per record and would be timed as part of the kernels
    around it). The launches are ordered on the stream, so each timestamp is
    taken after the preceding kernel has completed."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch has loaded
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls._hip = lib
        return cls._hip

    def __init__(self, torch):
        import ctypes
        self._torch = torch
        self._ev = ctypes.c_void_p()
        st = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev),
                                                 0x20000000)   # hipEventDisableSystemFence
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")

    def record(self):
        st = self._lib().hipEventRecord(self._ev, self._torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        st = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


def _events(torch, n):
    return [_HipEvent(torch) for _ in range(n)]


def prefill_setup(torch, fa, cfg, sink_logits=None, tensors=None, split=False):
    """Prepared (pack, attention) calls for a prefill workload; `tensors`, when
    a dict, receives the output tensors. split: the attention call with the key
    split of the longest query blocks (fa_prefill_fwd_packed_split)."""
    from flashattention_attention_amd import inputs
    x = inputs.make_prefill_inputs(cfg)
    q, k, v = (_dev(torch, x[n], cfg.dtype) for n in ("q", "k", "v"))
    B, Sq, Hq, D = x["q"].shape
    o = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    # row sums only where the workload asks for them (un-normalized output):
    # the others state O and the LSE as their outputs
    rs = (torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
          if cfg.out_unnormalized else None)

    ws = torch.empty(fa.prefill_workspace_size(B, cfg.seqlen_kv, cfg.n_heads_kv, D),
                     dtype=torch.uint8, device="cuda")

    # prepared calls: marshalled once, so a launch costs a few microseconds of host
    # time and the host stays ahead of the GPU inside the timed loops
    sws = None
    if split:
        sws = torch.zeros(fa.prefill_split_workspace_size(B, Sq, Hq, D), dtype=torch.uint8,
                          device="cuda")
        rs = None   # (row sums would turn the split off)
    pack = fa.prefill_pack_v(v, workspace=ws, prepare=True)
    attn = fa.prefill_packed(q, k, ws, causal=cfg.causal, softmax_scale=cfg.scale,
                             out_unnormalized=cfg.out_unnormalized, out=o, lse=lse, row_sum=rs,
                             window=cfg.window, sink_logits=sink_logits, split_workspace=sws,
                             prepare=True)
    if tensors is not None:
        tensors.update(o=o, lse=lse)

    def run():
        pack()
        attn()
    return run, pack, attn


def prefill_direct_setup(torch, fa, cfg):
    """The one-call fa_prefill_fwd for a workload, prepared (fp16 at head_dim
    <= 128 is a single launch that reads V's rows; other inputs run the V
    repack and the attention kernel inside the call)."""
    from flashattention_attention_amd import inputs
    x = inputs.make_prefill_inputs(cfg)
    q, k, v = (_dev(torch, x[n], cfg.dtype) for n in ("q", "k", "v"))
    return fa.prefill(q, k, v, causal=cfg.causal, softmax_scale=cfg.scale,
                      out_unnormalized=cfg.out_unnormalized, window=cfg.window,
                      prepare=True)


def prefill_kernel_name(cfg, split=False, vrow=False):
    """The attention kernel's template name as rocprofv3 reports it (vrow: the
    one-launch fp16 form that reads V's rows)."""
    if cfg.head_dim == 512:
        return (f"prefill512_kernel<{str(cfg.dtype == 'bf16').lower()}, "
                f"{str(cfg.out_unnormalized).lower()}>")
    from flashattention_attention_amd import fa
    group = cfg.n_heads_q // cfg.n_heads_kv
    hp = 2 if cfg.head_dim <= 128 and group % 2 == 0 else 1
    trio = (not split and not vrow and
            fa.prefill_trio(cfg.batch, cfg.seqlen_q, cfg.seqlen_kv, cfg.n_heads_q,
                            cfg.n_heads_kv, cfg.head_dim, cfg.causal, cfg.window))
    # template arguments: head_dim, bf16, exact running max (un-normalized
    # output or row sums), heads per work-group, key split, V rows, three per CU
    return (f"prefill_kernel<{cfg.head_dim}, {str(cfg.dtype == 'bf16').lower()}, "
            f"{str(cfg.out_unnormalized).lower()}, {hp}, {str(split).lower()}, "
            f"{str(vrow).lower()}, {str(trio).lower()}>")


def decode_kernel_name(cfg):
    """The partial kernel's name for a decode that spans several rounds of
    resident waves (the batched workload): the widest heads-per-wave choice."""
    group = cfg.n_heads_q // cfg.n_heads_kv
    g = next(x for x in range(8, 0, -1) if group % x == 0)
    return f"decode_partial_kernel<{cfg.head_dim}, {g}, {str(cfg.dtype == 'bf16').lower()}>"


def source_digest(name):
    """Short digest of a kernel source file: the traffic counters in profiles/
    apply only to the source they were taken from."""
    import hashlib
    path = os.path.join(ROOT, "flashattention_attention_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel, workload, source):
    """HBM bytes per launch (read + write, copy-calibrated) recorded in
    profiles/hbm_traffic_counters.md for this kernel, workload and source
    digest, else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    if not os.path.exists(path):
        return None
    import re
    for line in open(path):
        m = re.match(r"^traffic kernel=(.+?) workload=(\S+) source=(\S+) read_bytes=(\d+) "
                     r"write_bytes=(\d+)\s*$", line.strip())
        if m and m.group(1) == kernel and m.group(2) == workload and m.group(3) == source_digest(source):
            return int(m.group(4)) + int(m.group(5))
    return None


_DECODE_INPUTS = {}


def decode_inputs(cfg):
    """Seeded decode inputs, drawn once per workload (the batched long decode's
    1.3 G half values take tens of seconds to draw)."""
    from flashattention_attention_amd import inputs
    if cfg.name not in _DECODE_INPUTS:
        _DECODE_INPUTS[cfg.name] = inputs.make_decode_inputs(cfg)
    return _DECODE_INPUTS[cfg.name]


def decode_setup(torch, fa, cfg, split_len=None, head_major=False):
    """head_major: the same caches stored [Hkv, T, D] (passed as [T, Hkv, D] views
    with a head stride of T*D); the default is token-major [T, Hkv, D]."""
    from flashattention_attention_amd import inputs
    x = decode_inputs(cfg)
    q, kc, vc = (_dev(torch, x[n], cfg.dtype) for n in ("q", "k_cache", "v_cache"))
    if head_major:
        kc, vc = (t.permute(1, 0, 2).contiguous().permute(1, 0, 2) for t in (kc, vc))
    offs = torch.from_numpy(x["kv_offsets"]).cuda()
    lens = torch.from_numpy(x["kv_lens"]).cuda()
    if split_len is None:
        split_len, max_splits = fa.decode_plan(x["kv_lens"], cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim)
    else:
        max_splits = -(-int(x["kv_lens"].max()) // split_len)
    B, Hq, D = x["q"].shape
    po = torch.empty((B, Hq, max_splits, D), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, Hq, max_splits), dtype=torch.float32, device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    partial = fa.decode_split_partial(q, kc, vc, offs, lens, split_len=split_len,
                                      max_splits=max_splits, softmax_scale=cfg.scale,
                                      part_o=po, part_lse=pl, prepare=True)
    merge = fa.decode_merge_lse(po, pl, lens, split_len=split_len, out=o, lse=lse, prepare=True)
    ws = torch.zeros(fa.decode_fused_workspace_size(B, Hq, cfg.n_heads_kv, D, max_splits),
                     dtype=torch.uint8, device="cuda")
    fused = fa.decode_fused(q, kc, vc, offs, lens, split_len=split_len, max_splits=max_splits,
                            softmax_scale=cfg.scale, out=o, lse=lse, workspace=ws, prepare=True)

    kv_bytes = inputs.decode_kv_bytes(x["kv_lens"], cfg.n_heads_kv, cfg.head_dim)
    alg_bytes = kv_bytes + q.numel() * 2 + o.numel() * 4 + lse.numel() * 4
    n_parts = int(sum(-(-int(L) // split_len) for L in x["kv_lens"])) * Hq
    part_bytes = 2 * n_parts * (D + 1) * 4           # written once, read once
    return partial, merge, {"split_len": split_len, "max_splits": max_splits,
                            "kv_bytes": kv_bytes, "alg_bytes": alg_bytes,
                            "partial_bytes": part_bytes, "fused": fused}


def time_calls(torch, fns, iters, flush=None):
    """Median / min per-call duration (ms) of each fn, HIP events on the current stream.
    Each iteration starts behind a long kernel (the cache flush, else a ~50 us spin)
    so that the host has enqueued every timed launch before the GPU reaches it."""
    per = [[] for _ in fns]
    for _ in range(iters):
        if flush is not None:
            flush()
        else:
            torch.cuda._sleep(120000)
        evs = _events(torch, len(fns) + 1)
        evs[0].record()
        for i, fn in enumerate(fns):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        for i in range(len(fns)):
            per[i].append(evs[i].elapsed_time(evs[i + 1]))
    return [_stats(p) for p in per]


def warm_up(torch, fns, ms=30.0):
    """Run fns back to back for at least ``ms`` of wall time before a line is
    timed. The matrix-core prompts run ~7 % slower for the first few
    milliseconds after a pause (the head_dim 256 prompt: 1140 us per call
    after 3 warm-up calls, 1069 us after 50); the headline step's 200 warm-up
    steps take ~25 ms."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for f in fns:
            f()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                return n


def _stats(p):
    """Median, min and mean of interval times (ms), the min/median spread, and
    how many intervals exceed 1.5x the median (a host stall inside an event
    interval shows as such an outlier; the median is what the lines report)."""
    med = statistics.median(p)
    return {"median_ms": med, "min_ms": min(p), "mean_ms": statistics.mean(p),
            "spread": round((med - min(p)) / med, 4) if med > 0 else 0.0,
            "outliers": sum(1 for x in p if x > 1.5 * med)}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _nproc():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _prefill_pairs(cfg, rows):
    """Visible (query, key) pairs of the listed rows (causal, bottom-right)."""
    off = cfg.seqlen_kv - cfg.seqlen_q
    if not cfg.causal:
        return len(rows) * cfg.seqlen_kv
    return int(sum(min(cfg.seqlen_kv, r + off + 1) for r in rows))


def _oracle_prefill_rate(cfg, x, rows):
    import oracle
    t0 = time.perf_counter()
    oracle.prefill(x["q"], x["k"], x["v"], scale=cfg.scale, causal=cfg.causal, dtype=cfg.dtype,
                   rows=rows)
    dt = time.perf_counter() - t0
    flops = 4 * cfg.head_dim * cfg.n_heads_q * cfg.batch * _prefill_pairs(cfg, rows)
    return flops, dt


def cpu_baseline(budget_s=20.0):
    """The fp64 oracle timed on this host. The contract figure: a bounded sample
    of the GQA prompt (rows spread over the sequence, all heads), doubled until
    ~budget_s / 2 of CPU work (the whole prompt takes ~2 s on 16 threads), and
    the same oracle on one thread. per_config: the oracle on every workload,
    whole or on a stated sample, in the unit of the GPU figure."""
    import oracle
    from flashattention_attention_amd import inputs
    threads = _blas_threads()
    cfg = inputs.GQA_PREFILL
    x = inputs.make_prefill_inputs(cfg)
    n, spent, last = 16, 0.0, None
    while True:
        rows = np.unique(np.linspace(0, cfg.seqlen_q - 1, n).astype(np.int64))
        flops, dt = _oracle_prefill_rate(cfg, x, rows)
        spent += dt
        last = (len(rows), dt, flops)
        if spent >= budget_s / 2 or n >= cfg.seqlen_q:
            break
        n *= 2
    nrows, dt, flops = last
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "nproc": _nproc(), "kind": "oracle",
           "sample": f"{nrows} query rows evenly spaced over the 3314-token prompt, all "
                     f"{cfg.n_heads_q} heads, fp64 two-pass definition ({flops / 1e9:.2f} "
                     f"GFLOP in {dt:.2f} s)"}
    try:                                   # the same oracle on one thread, a smaller sample
        from threadpoolctl import threadpool_limits
        rows = np.unique(np.linspace(0, cfg.seqlen_q - 1, 128).astype(np.int64))
        with threadpool_limits(limits=1):
            f1, dt1 = _oracle_prefill_rate(cfg, x, rows)
        out["single_thread"] = {"value": f1 / dt1 / 1e12, "unit": "TFLOP/s",
                                "sample": f"{len(rows)} query rows, all heads "
                                          f"({f1 / 1e9:.2f} GFLOP in {dt1:.2f} s)"}
    except ImportError:
        pass

    per = {cfg.name: {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s",
                      "seconds": round(dt, 3), "sample": f"{nrows} of {cfg.seqlen_q} rows"}}
    # the tiny prompt, whole
    tcfg = inputs.TINY_CAUSAL
    tx = inputs.make_prefill_inputs(tcfg)
    rows = np.arange(tcfg.seqlen_q)
    f, d = _oracle_prefill_rate(tcfg, tx, rows)
    per[tcfg.name] = {"value": round(f / d / 1e12, 6), "unit": "TFLOP/s",
                      "us_per_call": round(d * 1e6, 1), "seconds": round(d, 4),
                      "sample": "whole problem"}
    # the large-head prompt: 32 rows evenly spaced, every head of both batch entries
    hcfg = inputs.LARGE_HEAD
    hx = inputs.make_prefill_inputs(hcfg)
    rows = np.unique(np.linspace(0, hcfg.seqlen_q - 1, 32).astype(np.int64))
    f, d = _oracle_prefill_rate(hcfg, hx, rows)
    per[hcfg.name] = {"value": round(f / d / 1e12, 5), "unit": "TFLOP/s", "seconds": round(d, 3),
                      "sample": f"{len(rows)} of {hcfg.seqlen_q} rows, all 32 (batch, head)"}
    del hx
    # decode: the 1641-token call whole; the batched long decode on a sample of
    # (sequence, head) pairs, its whole-call time scaled by the keys visited
    for dcfg, n_pairs in ((inputs.GQA_DECODE, None), (inputs.LONG_DECODE, 16)):
        dx = decode_inputs(dcfg)
        kv_bytes = inputs.decode_kv_bytes(dx["kv_lens"], dcfg.n_heads_kv, dcfg.head_dim)
        if n_pairs is None:
            t0 = time.perf_counter()
            oracle.decode(dx["q"], dx["k_cache"], dx["v_cache"], dx["kv_offsets"],
                          dx["kv_lens"], scale=dcfg.scale, dtype=dcfg.dtype)
            call_s = time.perf_counter() - t0
            sample = "whole call"
        else:
            rng = np.random.default_rng(dcfg.seed)
            picks = sorted({(int(b), int(h)) for b, h in
                            zip(rng.integers(0, dcfg.batch, n_pairs),
                                rng.integers(0, dcfg.n_heads_q, n_pairs))})
            group = dcfg.n_heads_q // dcfg.n_heads_kv
            t0 = time.perf_counter()
            for b, h in picks:
                hk = h // group
                oracle.decode(dx["q"][b:b + 1, h:h + 1], dx["k_cache"][:, hk:hk + 1],
                              dx["v_cache"][:, hk:hk + 1], dx["kv_offsets"][b:b + 1],
                              dx["kv_lens"][b:b + 1], scale=dcfg.scale, dtype=dcfg.dtype)
            dt_s = time.perf_counter() - t0
            keys_sample = sum(int(dx["kv_lens"][b]) for b, _ in picks)
            keys_all = int(dx["kv_lens"].sum()) * dcfg.n_heads_q
            call_s = dt_s * keys_all / keys_sample
            sample = (f"{len(picks)} (sequence, head) pairs in {dt_s:.2f} s, the whole call "
                      f"scaled by the keys visited")
        per[dcfg.name] = {"us_per_call": round(call_s * 1e6, 1),
                          "value": round(kv_bytes / call_s / 1e9, 3), "unit": "GB/s",
                          "sample": sample}
    out["per_config"] = per
    return out


def device_info(torch):
    """CUs and peak engine clock as the device reports them, and the dense
    bf16/fp16 MFMA peak they imply (4096 FLOP per clock per CU), next to the
    datasheet figure the rooflines use."""
    dev = torch.cuda.current_device()
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "mfma_bf16_dense_tflops_datasheet": MI355X_BF16_DENSE_TFLOPS}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, dev) == 0 and khz.value > 0:  # clock, kHz
            info["peak_clock_mhz"] = khz.value / 1000
            info["mfma_bf16_dense_tflops_from_device"] = round(
                props.multi_processor_count * 4096 * khz.value * 1e3 / 1e12, 1)
    except OSError:
        pass
    return info


def run_profiling_aid(torch, fa, inputs, args):
    """Single-component runs for rocprofv3 counter passes (no JSON contract line)."""
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        fns = [lambda: dst.copy_(src)]
        label = f"copy {args.copy_bytes} bytes"
    elif args.only in ("prefill", "large_head", "window", "hd512", "few_heads_split"):
        cfg = {"prefill": inputs.GQA_PREFILL, "large_head": inputs.LARGE_HEAD,
               "window": inputs.WINDOW_PREFILL, "hd512": inputs.HD512_PREFILL,
               "few_heads_split": inputs.FEW_HEADS_PREFILL}[args.only]
        _, pack, attn = prefill_setup(torch, fa, cfg, split=args.only == "few_heads_split")
        fns, label = [pack, attn], cfg.name
    elif args.only == "prefill_f16":
        cfg = dataclasses.replace(inputs.GQA_PREFILL, dtype="f16",
                                  name=inputs.GQA_PREFILL.name.replace("_bf16", "_f16"))
        fns, label = [prefill_direct_setup(torch, fa, cfg)], cfg.name
    elif args.only == "sink":
        cfg = inputs.WINDOW_PREFILL
        tens = {}
        _, pack, attn = prefill_setup(torch, fa, cfg, tensors=tens)
        sinks = torch.linspace(-2.0, 6.0, cfg.n_heads_q, dtype=torch.float32, device="cuda")
        merge = fa.attn_merge(tens["o"], tens["lse"], sink_logits=sinks, out=tens["o"],
                              lse=tens["lse"], prepare=True)
        fns, label = [pack, attn, merge], cfg.name + "_sink"
    else:
        cfg = {"decode": inputs.GQA_DECODE, "long_decode": inputs.LONG_DECODE,
               "long_decode_h28kv4": inputs.LONG_DECODE_G7}[args.only]
        part, merge, info = decode_setup(torch, fa, cfg)
        fns, label = [part, merge, info["fused"]], cfg.name
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    r = time_calls(torch, fns, args.steps)
    print(f"[profiling aid] {label}: " + ", ".join(f"{x['median_ms'] * 1e3:.2f} us" for x in r),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)   # ~30 ms: lets the clocks settle
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--split-sweep", action="store_true",
                    help="also time the single-token decode at several split lengths")
    ap.add_argument("--only", choices=["prefill", "decode", "long_decode", "large_head",
                                              "window", "hd512", "sink", "few_heads_split",
                                              "prefill_f16", "long_decode_h28kv4"],
                    help="profiling aid: run only this component (warmup + steps) and exit")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="profiling aid: time a plain device-to-device copy of this many "
                         "bytes (the reference for scaling HBM traffic counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    from flashattention_attention_amd import fa, inputs
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    if args.copy_bytes or args.only:
        run_profiling_aid(torch, fa, inputs, args)
        return
    pcfg, dcfg = inputs.GQA_PREFILL, inputs.GQA_DECODE
    print(f"[bench] {props.name} cus={props.multi_processor_count}; preparing inputs",
          file=sys.stderr, flush=True)

    prefill, p_pack, p_attn = prefill_setup(torch, fa, pcfg)
    d_partial, d_merge, dinfo = decode_setup(torch, fa, dcfg)
    d_fused = dinfo["fused"]       # split partials and their merge in one launch

    def step():
        prefill()
        d_fused()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps

    # the timed region: K whole steps, an event between consecutive launches
    evs = [_events(torch, 4) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = evs[i]
        e[0].record()
        p_pack()
        e[1].record()
        p_attn()
        e[2].record()
        d_fused()
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = statistics.mean(e[0].elapsed_time(e[3]) for e in evs)

    def launch_stats(a, b):
        return _stats([e[a].elapsed_time(e[b]) for e in evs])
    st_pack, st_attn, st_dec = (launch_stats(i, i + 1) for i in range(3))
    # per-launch medians over the K steps (robust to a host stall in one interval)
    pack_mean, attn_mean = st_pack["median_ms"], st_attn["median_ms"]
    pre_mean = pack_mean + attn_mean
    flops = pcfg.flops()
    value = flops / (pre_mean * 1e-3) / 1e12
    attn_tflops = flops / (attn_mean * 1e-3) / 1e12
    dec_us = st_dec["median_ms"] * 1e3
    print(f"[bench] timed {K} steps: {step_ms * 1e3:.1f} us per step; prefill "
          f"{pre_mean * 1e3:.1f} us, decode {dec_us:.1f} us", file=sys.stderr, flush=True)

    pk = prefill_kernel_name(pcfg)
    rooflines = {
        "prefill_gqa_s3314": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                              "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(attn_tflops / MI355X_BF16_DENSE_TFLOPS, 4),
                              "traffic": measured_traffic(pk, pcfg.name, "fa_prefill.hip"),
                              "kernel": pk, "us_per_launch": round(attn_mean * 1e3, 2),
                              "per_launch": f"{flops / 1e9:.2f} GFLOP (4 * head_dim per "
                                            f"visible query/key pair and query head)"}}
    line = {
        "metric": "causal GQA prefill attention TFLOP/s (3314 tokens, 28/4 heads, hd 128, bf16)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "wall_ms_per_step": round(wall / K * 1e3, 4),
        "timing": "HIP events between consecutive launches of K eager steps on the launch "
                  "stream (prepared calls keep the host ahead of the GPU); per-launch figures "
                  "are medians over the K steps, ms_per_step the mean step interval",
        "config": {"workload": f"{pcfg.name} + {dcfg.name}", "global_batch": 1,
                   "seq_len": pcfg.seqlen_q, "kv_len_decode": 1641, "parallelism": "none"},
        "prefill": {"us_per_call": round(pre_mean * 1e3, 2), "gflop": round(flops / 1e9, 3),
                    "v_repack_us": round(pack_mean * 1e3, 2),
                    "attention_us": round(attn_mean * 1e3, 2),
                    "attention_us_min": round(st_attn["min_ms"] * 1e3, 2),
                    "attention_spread": st_attn["spread"],
                    "attention_outliers": st_attn["outliers"],
                    "frac_mfma_peak": round(value / MI355X_BF16_DENSE_TFLOPS, 4)},
        "decode_gqa_kv1641": {
            "split_len": dinfo["split_len"], "max_splits": dinfo["max_splits"],
            "us_per_call": round(dec_us, 2), "launches": 1,
            "spread": st_dec["spread"],
            "alg_gbps": round(dinfo["alg_bytes"] / (dec_us * 1e-6) / 1e9, 1),
            "cache": "as left by the preceding prefill in the step"},
    }

    if not args.no_extras:
        flush_buf = torch.empty(1 << 27, dtype=torch.float32, device="cuda")   # 512 MB

        def flush():
            flush_buf.zero_()

        # single-token decode: cold (flushed) and hot, in one launch and in two
        fc = time_calls(torch, [d_fused], 20, flush=flush)
        fh = time_calls(torch, [d_fused], 50)
        line["decode_gqa_kv1641"]["cold_us"] = round(fc[0]["median_ms"] * 1e3, 2)
        line["decode_gqa_kv1641"]["hot_us"] = round(fh[0]["median_ms"] * 1e3, 2)
        cold = time_calls(torch, [d_partial, d_merge], 20, flush=flush)
        hot = time_calls(torch, [d_partial, d_merge], 50)
        line["decode_gqa_kv1641"]["two_launches"] = {
            "cold_us": round((cold[0]["median_ms"] + cold[1]["median_ms"]) * 1e3, 2),
            "hot_us": round((hot[0]["median_ms"] + hot[1]["median_ms"]) * 1e3, 2),
            "partial_us_hot": round(hot[0]["median_ms"] * 1e3, 2),
            "merge_us_hot": round(hot[1]["median_ms"] * 1e3, 2)}
        if args.split_sweep:
            sweep = {}
            for sl in (16, 32, 48, 64, 112, 208):
                p2, m2, _ = decode_setup(torch, fa, dcfg, split_len=sl)
                c = time_calls(torch, [p2, m2], 20, flush=flush)
                sweep[sl] = round((c[0]["median_ms"] + c[1]["median_ms"]) * 1e3, 2)
            line["decode_gqa_kv1641"]["cold_us_by_split_len"] = sweep
        print("[bench] long decode", file=sys.stderr, flush=True)

        lcfg = inputs.LONG_DECODE
        if args.split_sweep:
            sweep = {}
            for sl in (512, 1024, 1536, 2048, 3072, 4096):
                p2, m2, i2 = decode_setup(torch, fa, lcfg, split_len=sl)
                c = time_calls(torch, [p2, m2], 5, flush=flush)
                sweep[sl] = round((c[0]["median_ms"] + c[1]["median_ms"]) * 1e3, 1)
                del p2, m2
            line["decode_batched_long_us_by_split_len"] = sweep
        l_partial, l_merge, linfo = decode_setup(torch, fa, lcfg)
        for _ in range(3):
            l_partial(); l_merge()
        r = time_calls(torch, [l_partial, l_merge], 20, flush=flush)
        tot_ms = r[0]["median_ms"] + r[1]["median_ms"]
        rf = time_calls(torch, [linfo["fused"]], 20, flush=flush)
        fused_ms = rf[0]["median_ms"]
        part_gbps = (linfo["kv_bytes"] + 0.0) / (r[0]["median_ms"] * 1e-3) / 1e9
        line["decode_batched_long"] = {
            "workload": lcfg.name, "split_len": linfo["split_len"],
            "max_splits": linfo["max_splits"], "kv_gb": round(linfo["kv_bytes"] / 1e9, 4),
            "us_per_call": round(tot_ms * 1e3, 1),
            "partial_us": round(r[0]["median_ms"] * 1e3, 1),
            "merge_us": round(r[1]["median_ms"] * 1e3, 1),
            "alg_gbps": round(linfo["alg_bytes"] / (tot_ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(linfo["alg_bytes"] / (tot_ms * 1e-3) / 1e9 / MI355X_HBM_GBPS,
                                   4),
            "partial_bytes_overhead_gb": round(linfo["partial_bytes"] / 1e9, 4),
            "fused_single_launch_us": round(fused_ms * 1e3, 1),
            "fused_frac_hbm_peak": round(linfo["alg_bytes"] / (fused_ms * 1e-3) / 1e9
                                         / MI355X_HBM_GBPS, 4),
            "cache": "flushed (512 MB write) before every call"}
        # The same decode on head-major caches (each wave's K and V rows then
        # lie in one contiguous stream instead of every Hkv-th 256 bytes).
        h_partial, h_merge, _ = decode_setup(torch, fa, lcfg, head_major=True)
        for _ in range(3):
            h_partial(); h_merge()
        rh = time_calls(torch, [h_partial, h_merge], 20, flush=flush)
        h_ms = rh[0]["median_ms"] + rh[1]["median_ms"]
        line["decode_batched_long"]["head_major_caches"] = {
            "us_per_call": round(h_ms * 1e3, 1), "partial_us": round(rh[0]["median_ms"] * 1e3, 1),
            "frac_hbm_peak": round(linfo["alg_bytes"] / (h_ms * 1e-3) / 1e9 / MI355X_HBM_GBPS, 4)}
        del h_partial, h_merge
        # The same lengths at 28/4 heads: seven query heads per wave, Q.K^T on
        # the matrix cores.
        gcfg = inputs.LONG_DECODE_G7
        g_partial, g_merge, ginfo = decode_setup(torch, fa, gcfg)
        for _ in range(3):
            g_partial(); g_merge(); ginfo["fused"]()
        rg = time_calls(torch, [g_partial, g_merge], 20, flush=flush)
        rgf = time_calls(torch, [ginfo["fused"]], 20, flush=flush)
        g_ms = rg[0]["median_ms"] + rg[1]["median_ms"]
        g_gbps = ginfo["kv_bytes"] / (rg[0]["median_ms"] * 1e-3) / 1e9
        gk = decode_kernel_name(gcfg)
        rooflines["decode_partial_batched_long_h28kv4"] = {
            "bound": "hbm", "achieved": round(g_gbps, 1), "peak": MI355X_HBM_GBPS,
            "unit": "GB/s", "frac": round(g_gbps / MI355X_HBM_GBPS, 4),
            "traffic": measured_traffic(gk, gcfg.name, "fa_decode.hip"), "kernel": gk,
            "us_per_launch": round(rg[0]["median_ms"] * 1e3, 1),
            "per_launch": f"{ginfo['kv_bytes'] / 1e9:.4f} GB of K+V (each cached key and value "
                          f"row read once)"}
        line["decode_batched_long_h28kv4"] = {
            "workload": gcfg.name, "split_len": ginfo["split_len"],
            "max_splits": ginfo["max_splits"], "kv_gb": round(ginfo["kv_bytes"] / 1e9, 4),
            "us_per_call": round(g_ms * 1e3, 1), "partial_us": round(rg[0]["median_ms"] * 1e3, 1),
            "frac_hbm_peak": round(ginfo["alg_bytes"] / (g_ms * 1e-3) / 1e9 / MI355X_HBM_GBPS, 4),
            "fused_single_launch_us": round(rgf[0]["median_ms"] * 1e3, 1),
            "fused_frac_hbm_peak": round(ginfo["alg_bytes"] / (rgf[0]["median_ms"] * 1e-3) / 1e9
                                         / MI355X_HBM_GBPS, 4),
            "cache": "flushed (512 MB write) before every call"}
        del g_partial, g_merge, ginfo
        dk = decode_kernel_name(lcfg)
        rooflines["decode_partial_batched_long"] = {
            "bound": "hbm", "achieved": round(part_gbps, 1), "peak": MI355X_HBM_GBPS,
            "unit": "GB/s", "frac": round(part_gbps / MI355X_HBM_GBPS, 4),
            "traffic": measured_traffic(dk, lcfg.name, "fa_decode.hip"), "kernel": dk,
            "us_per_launch": round(r[0]["median_ms"] * 1e3, 1),
            "per_launch": f"{linfo['kv_bytes'] / 1e9:.4f} GB of K+V (each cached key and value "
                          f"row read once)"}
        nw = fa.load_library().fa_decode_fused_waves(lcfg.batch, lcfg.n_heads_q, lcfg.n_heads_kv,
                                                     lcfg.head_dim, linfo["max_splits"])
        fk = decode_kernel_name(lcfg).replace("decode_partial_kernel", "decode_fused_kernel")
        fk = fk[:-1] + f", {nw}>"
        f_gbps = linfo["kv_bytes"] / (fused_ms * 1e-3) / 1e9
        rooflines["decode_fused_batched_long"] = {
            "bound": "hbm", "achieved": round(f_gbps, 1), "peak": MI355X_HBM_GBPS,
            "unit": "GB/s", "frac": round(f_gbps / MI355X_HBM_GBPS, 4),
            "traffic": measured_traffic(fk, lcfg.name, "fa_decode.hip"), "kernel": fk,
            "us_per_launch": round(fused_ms * 1e3, 1),
            "per_launch": f"{linfo['kv_bytes'] / 1e9:.4f} GB of K+V (each cached key and value "
                          f"row read once)"}
        del l_partial, l_merge, linfo
        torch.cuda.empty_cache()
        print("[bench] tiny prefill", file=sys.stderr, flush=True)
        tcfg = inputs.TINY_CAUSAL          # latency-bound: one work-group, two tiles
        t_call = prefill_direct_setup(torch, fa, tcfg)   # fp16, head_dim 64: one launch
        warm_up(torch, [t_call])
        r = time_calls(torch, [t_call], 20)
        line["prefill_tiny"] = {"workload": tcfg.name,
                                "us_per_call": round(r[0]["median_ms"] * 1e3, 2),
                                "launches": 1,
                                "mflop": round(tcfg.flops() / 1e6, 3)}
        del t_call
        print("[bench] GQA prefill, fp16 one-launch form", file=sys.stderr, flush=True)
        gcfg = dataclasses.replace(inputs.GQA_PREFILL, dtype="f16",
                                   name=inputs.GQA_PREFILL.name.replace("_bf16", "_f16"))
        g_call = prefill_direct_setup(torch, fa, gcfg)
        warm_up(torch, [g_call])
        r = time_calls(torch, [g_call], 20)
        gt = gcfg.flops() / (r[0]["median_ms"] * 1e-3) / 1e12
        line["prefill_gqa_f16"] = {"workload": gcfg.name, "launches": 1,
                                   "us_per_call": round(r[0]["median_ms"] * 1e3, 1),
                                   "spread": r[0]["spread"], "tflops": round(gt, 2),
                                   "frac_mfma_peak": round(gt / MI355X_BF16_DENSE_TFLOPS, 4)}
        vk = prefill_kernel_name(gcfg, vrow=True)
        rooflines["prefill_gqa_s3314_f16_one_launch"] = {
            "bound": "mfma", "achieved": round(gt, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gt / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(vk, gcfg.name, "fa_prefill.hip"), "kernel": vk,
            "us_per_launch": round(r[0]["median_ms"] * 1e3, 2),
            "per_launch": f"{gcfg.flops() / 1e9:.2f} GFLOP (fp16 peak = bf16 peak)"}
        del g_call
        print("[bench] large-head prefill", file=sys.stderr, flush=True)

        hcfg = inputs.LARGE_HEAD
        h_run, h_pack, h_attn = prefill_setup(torch, fa, hcfg)
        warm_up(torch, [h_run])
        r = time_calls(torch, [h_pack, h_attn], 15)
        hf = hcfg.flops()
        h_ms = r[0]["median_ms"] + r[1]["median_ms"]
        ht = hf / (h_ms * 1e-3) / 1e12
        ha = hf / (r[1]["median_ms"] * 1e-3) / 1e12
        line["prefill_large_head"] = {"workload": hcfg.name,
                                      "us_per_call": round(h_ms * 1e3, 1),
                                      "attention_us": round(r[1]["median_ms"] * 1e3, 1),
                                      "attention_spread": r[1]["spread"],
                                      "tflops": round(ht, 2),
                                      "frac_mfma_peak": round(ht / MI355X_BF16_DENSE_TFLOPS, 4)}
        hk = prefill_kernel_name(hcfg)
        rooflines["prefill_large_head"] = {
            "bound": "mfma", "achieved": round(ha, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ha / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(hk, hcfg.name, "fa_prefill.hip"), "kernel": hk,
            "us_per_launch": round(r[1]["median_ms"] * 1e3, 1),
            "per_launch": f"{hf / 1e12:.4f} TFLOP"}
        del h_run, h_pack, h_attn
        print("[bench] windowed prefill", file=sys.stderr, flush=True)

        wcfg = inputs.WINDOW_PREFILL
        w_run, w_pack, w_attn = prefill_setup(torch, fa, wcfg)
        warm_up(torch, [w_run])
        r = time_calls(torch, [w_pack, w_attn], 20)
        wf = wcfg.flops()
        w_ms = r[0]["median_ms"] + r[1]["median_ms"]
        wa = wf / (r[1]["median_ms"] * 1e-3) / 1e12
        line["prefill_window"] = {"workload": wcfg.name, "window": wcfg.window,
                                  "us_per_call": round(w_ms * 1e3, 1),
                                  "attention_us": round(r[1]["median_ms"] * 1e3, 1),
                                  "attention_spread": r[1]["spread"],
                                  "tflops": round(wf / (w_ms * 1e-3) / 1e12, 2),
                                  "frac_mfma_peak": round(wf / (w_ms * 1e-3) / 1e12
                                                          / MI355X_BF16_DENSE_TFLOPS, 4)}
        wk = prefill_kernel_name(wcfg)
        rooflines["prefill_window1024"] = {
            "bound": "mfma", "achieved": round(wa, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(wa / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(wk, wcfg.name, "fa_prefill.hip"), "kernel": wk,
            "us_per_launch": round(r[1]["median_ms"] * 1e3, 1),
            "per_launch": f"{wf / 1e12:.4f} TFLOP (visible pairs only)"}
        del w_run, w_pack, w_attn
        print("[bench] windowed prefill with sinks", file=sys.stderr, flush=True)

        # The same windowed prompt with a per-head sink logit (synthetic values):
        # folded into the attention epilogue, or merged by a separate in-place
        # pass over the attention's output.
        sinks = torch.linspace(-2.0, 6.0, wcfg.n_heads_q, dtype=torch.float32, device="cuda")
        tens = {}
        _, s_pack, s_attn = prefill_setup(torch, fa, wcfg, sink_logits=sinks)
        _, p_pack2, p_attn2 = prefill_setup(torch, fa, wcfg, tensors=tens)
        s_merge = fa.attn_merge(tens["o"], tens["lse"], sink_logits=sinks, out=tens["o"],
                                lse=tens["lse"], prepare=True)
        warm_up(torch, [s_pack, s_attn, p_pack2, p_attn2, s_merge])
        rf = time_calls(torch, [s_pack, s_attn], 20)
        ru = time_calls(torch, [p_pack2, p_attn2, s_merge], 20)
        fused_ms = rf[0]["median_ms"] + rf[1]["median_ms"]
        unf_ms = ru[0]["median_ms"] + ru[1]["median_ms"] + ru[2]["median_ms"]
        o_t, l_t = tens["o"], tens["lse"]
        merge_bytes = 2 * (o_t.numel() + l_t.numel()) * 4 + sinks.numel() * 4
        merge_gbps = merge_bytes / (ru[2]["median_ms"] * 1e-3) / 1e9
        line["prefill_window_sink"] = {
            "workload": wcfg.name + "_sink", "sinks": "linspace(-2, 6) over the 28 heads",
            "fused_epilogue_us": round(fused_ms * 1e3, 1),
            "unfused_us": round(unf_ms * 1e3, 1),
            "merge_pass_us": round(ru[2]["median_ms"] * 1e3, 1),
            "fused_tflops": round(wf / (fused_ms * 1e-3) / 1e12, 2)}
        rooflines["attn_merge_sink"] = {
            "bound": "hbm", "achieved": round(merge_gbps, 1), "peak": MI355X_HBM_GBPS,
            "unit": "GB/s", "frac": round(merge_gbps / MI355X_HBM_GBPS, 4),
            "traffic": measured_traffic("branch_merge_kernel<128>", wcfg.name + "_sink",
                                        "fa_merge.hip"),
            "kernel": "branch_merge_kernel<128>",
            "us_per_launch": round(ru[2]["median_ms"] * 1e3, 1),
            "per_launch": f"{merge_bytes / 1e6:.2f} MB (O and LSE read and written once)"}
        del s_pack, s_attn, p_pack2, p_attn2, s_merge, tens
        print("[bench] few-heads prefill, unsplit and with the key split", file=sys.stderr,
              flush=True)

        # One round of very unequal blocks (8 heads x 64 query blocks on 512
        # slots): the longest blocks' key ranges split over two work-groups.
        fcfg = inputs.FEW_HEADS_PREFILL
        units = fa.prefill_split_units(fcfg.batch, fcfg.seqlen_q, fcfg.seqlen_kv, fcfg.n_heads_q,
                                       fcfg.n_heads_kv, fcfg.head_dim, fcfg.causal, fcfg.window)
        _, fu_pack, fu_attn = prefill_setup(torch, fa, fcfg)
        _, fs_pack, fs_attn = prefill_setup(torch, fa, fcfg, split=True)
        warm_up(torch, [fu_pack, fu_attn, fs_pack, fs_attn])
        ru = time_calls(torch, [fu_pack, fu_attn], 20)
        rs = time_calls(torch, [fs_pack, fs_attn], 20)
        ff = fcfg.flops()
        fu_tf = ff / (ru[1]["median_ms"] * 1e-3) / 1e12
        fs_tf = ff / (rs[1]["median_ms"] * 1e-3) / 1e12
        line["prefill_few_heads"] = {
            "workload": fcfg.name, "split_blocks": sum(1 for _, k in units if k == 1),
            "blocks": -(-fcfg.seqlen_q // 128),
            "attention_us_unsplit": round(ru[1]["median_ms"] * 1e3, 1),
            "attention_us_split": round(rs[1]["median_ms"] * 1e3, 1),
            "tflops_unsplit": round(fu_tf, 2), "tflops_split": round(fs_tf, 2),
            "v_repack_us": round(rs[0]["median_ms"] * 1e3, 1)}
        fk = prefill_kernel_name(fcfg, split=True)
        rooflines["prefill_few_heads_split"] = {
            "bound": "mfma", "achieved": round(fs_tf, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(fs_tf / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(fk, fcfg.name, "fa_prefill.hip"), "kernel": fk,
            "us_per_launch": round(rs[1]["median_ms"] * 1e3, 1),
            "per_launch": f"{ff / 1e12:.4f} TFLOP"}
        del fu_pack, fu_attn, fs_pack, fs_attn
        print("[bench] head_dim 512 prefill", file=sys.stderr, flush=True)

        xcfg = inputs.HD512_PREFILL
        x_run, x_pack, x_attn = prefill_setup(torch, fa, xcfg)
        warm_up(torch, [x_run])
        r = time_calls(torch, [x_pack, x_attn], 20)
        xf = xcfg.flops()
        x_ms = r[0]["median_ms"] + r[1]["median_ms"]
        xa = xf / (r[1]["median_ms"] * 1e-3) / 1e12
        line["prefill_hd512"] = {"workload": xcfg.name, "us_per_call": round(x_ms * 1e3, 1),
                                 "attention_us": round(r[1]["median_ms"] * 1e3, 1),
                                 "attention_spread": r[1]["spread"],
                                 "tflops": round(xf / (x_ms * 1e-3) / 1e12, 2),
                                 "frac_mfma_peak": round(xf / (x_ms * 1e-3) / 1e12
                                                         / MI355X_BF16_DENSE_TFLOPS, 4)}
        xk = prefill_kernel_name(xcfg)
        rooflines["prefill_hd512"] = {
            "bound": "mfma", "achieved": round(xa, 2), "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(xa / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(xk, xcfg.name, "fa_prefill.hip"), "kernel": xk,
            "us_per_launch": round(r[1]["median_ms"] * 1e3, 1),
            "per_launch": f"{xf / 1e12:.4f} TFLOP"}
        del x_run, x_pack, x_attn
        del flush_buf

    line["roofline"] = rooflines["prefill_gqa_s3314"]
    line["rooflines"] = rooflines
    line["device"] = device_info(torch)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
