"""Benchmark of the exact blockwise attention hot path on one MI355X.

One step = one pass of the whole forward hot path over one batch of synthetic input.
For the headline workload (a Qwen2.5-7B-shaped GQA layer, 28 query / 4 key-value heads
x 128, one rank's share of a 4-way Ulysses split at 32K tokens):

    ulysses_permute(q, k, v)       sequence shards -> rank 0's head shard (one launch)
    attn_fwd                       causal, GQA 7:1, S = 32768, bf16 in, fp32 accumulate
    ulysses_permute(o)             head shard -> sequence shards

Prints ONE JSON line.  ``value`` is the algorithmic attention TFLOP/s of the whole step
(inputs resident in HBM; flops use the causal S^2/2 convention, 2 flops per MAC);
``roofline`` reports the attention kernel alone, timed with HIP events on the stream it
runs on; ``cpu_baseline`` times the fp64 CPU oracle on whole heads of the same workload's
own seeded inputs, for a bounded time.  The default run also times the other workloads
of the same hot path (the 8K Llama-7B-shaped causal layer, one rank's share of an 8-way
ring at 32K -- fused and chunk by chunk with the merge -- the 16K causal backward, the
FP8 forward of the 32K GQA shape, and the packed-document forward and backward) and
reports each as extra keys.  ``--workload`` selects another workload as the
headline of the line instead.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "causal bf16 attention fwd TFLOP/s + % of MFMA peak at S=32K, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense bf16 MFMA)
PEAK_F32_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2      # 256 CU x 2.4 GHz x 8192 flop/clk/CU (dense fp8 MFMA)
PEAK_HBM_GBPS = 8000.0
HEADLINE = "qwen7b_ulysses4_rank0_32k"


def visible_pairs(Sq, Skv, num_chunks, causal, q_offset, kv_offset):
    """(query, key) pairs counted for flops: all pairs if non-causal; with the causal
    mask, chunk by chunk with the continuous S^2/2 convention (a chunk entirely in the
    future counts 0, one entirely in the past counts Sq*L, a straddling one its area)."""
    if not causal:
        return float(Sq) * Skv
    L = Skv // num_chunks

    def G(x, c, m):  # integral of clamp(t - c, 0, m) dt from -inf to x
        t = x - c
        if t <= 0:
            return 0.0
        if t <= m:
            return 0.5 * t * t
        return 0.5 * m * m + (t - m) * m

    total = 0.0
    for ch in range(num_chunks):
        c = kv_offset + ch * L
        total += G(q_offset + Sq, c, L) - G(q_offset, c, L)
    return total


def attn_flops(B, Hq, Sq, Skv, D, num_chunks=1, causal=True, q_offset=0, kv_offset=0):
    return 4.0 * B * Hq * D * visible_pairs(Sq, Skv, num_chunks, causal, q_offset, kv_offset)


ROOT = os.path.dirname(os.path.abspath(__file__))
COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_qwen7b_gqa_32k_counters.md")
FWD_SOURCES = ("long_context_exact_tiled_amd/csrc/attn_fwd.hip",
               "long_context_exact_tiled_amd/csrc/common.h")


def measured_traffic():
    """HBM bytes per launch of the headline attention kernel, from the committed counter
    summary (FETCH_SIZE/WRITE_SIZE scaled by a plain copy of known size) -- or None when
    the kernel source no longer matches the profiled one."""
    import hashlib
    import re
    try:
        text = open(COUNTERS).read()
        h = hashlib.sha1()
        for f in FWD_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        want = re.search(r"source_sha1:\s*([0-9a-f]{40})", text).group(1)
        val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text).group(1)
    except (OSError, AttributeError):
        return None
    return int(val) if h.hexdigest() == want else None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def blas_vendor() -> str:
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{cfg.get('name', '?')} {cfg.get('version', '')}".strip()
    except Exception:
        return "unknown"


# ------------------------------------------------------------------ CPU oracle baseline

def _workload_inputs_f64(w):
    """The workload's own seeded inputs as the oracle reads them (fp64 of the bf16
    values): q, k, v (and dO for a backward), plus cu_seqlens for packed documents."""
    import oracle
    import seeded_inputs as si
    if w.ulysses_P:  # the head shard of rank r, moved by the oracle's own permute
        srcs = si.draw_ulysses_sources(w.seed)
        q, k, v = (oracle.seq_to_head(s, w.ulysses_P, w.ulysses_rank)[None] for s in srcs)
        return [si.as_f64(x, "bf16") for x in (q, k, v)], None
    xs = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype, with_dout=w.backward)
    cu = si.draw_doc_offsets(w.seed, w.q_shape[2]) if w.packed_docs else None
    return [si.as_f64(x, w.dtype) for x in xs], cu


def cpu_baseline(w, budget_s: float = 20.0):
    """Time the fp64 oracle on whole query heads (every row) of the workload's own seeded
    inputs, head after head until the time budget is spent (at least one head).

    ``value`` credits the algorithmic work of the heads done with the same convention as
    the GPU line (causal S^2/2, 2 flops per MAC; 2.5x the forward for a backward);
    ``value_full_matrix`` credits what the oracle actually computes (every masked score of
    the full matrix)."""
    import oracle
    xs, cu = _workload_inputs_f64(w)
    B, Hq, Sq, D = w.q_shape
    Hkv, Skv = w.kv_shape[1], w.kv_shape[2]
    group = Hq // Hkv
    fp8_codes = None
    if w.fp8:  # the inputs' codes are set up once, like the GPU side's inputs
        from oracle import fp8 as ofp8
        fp8_codes = [ofp8.quantize_heads(x.astype(np.float32)) for x in xs[:3]]
    fwd_mult = 2.5 if w.backward else 1.0
    done, done_full, units, t0 = 0.0, 0.0, 0, time.perf_counter()
    if w.backward:  # one key/value head (with its group of query heads) per unit
        q64, k64, v64, do64 = xs
        unit_list = list(range(Hkv))
    else:
        q64, k64, v64 = xs[:3]
        unit_list = list(range(Hq))
    for u in unit_list:
        if w.backward:
            if cu is not None:
                hs = slice(u * group, (u + 1) * group)
                oracle.varlen_attention_bwd(q64[:, hs], k64[:, u:u + 1], v64[:, u:u + 1],
                                            do64[:, hs], cu, causal=w.causal)
                pairs = sum(visible_pairs(b - a, b - a, 1, w.causal, 0, 0)
                            for a, b in zip(cu, cu[1:]))
                full = sum(float(b - a) ** 2 for a, b in zip(cu, cu[1:]))
            else:
                oracle.attention_bwd_heads(q64, k64, v64, do64, [(0, u)], causal=w.causal,
                                           q_offset=w.q_offset, kv_offset=w.kv_offset)
                pairs = visible_pairs(Sq, Skv, w.num_chunks, w.causal, w.q_offset,
                                      w.kv_offset)
                full = float(Sq) * Skv
            done += fwd_mult * 4.0 * D * pairs * group
            done_full += fwd_mult * 4.0 * D * full * group
        else:
            g = u // group
            if fp8_codes is not None:
                from oracle import fp8 as ofp8
                (qc, qd), (kc, kd), (vc, vd) = fp8_codes
                ofp8.fp8_attention(qc[:, u:u + 1], kc[:, g:g + 1], vc[:, g:g + 1],
                                   qd[:, u:u + 1], kd[:, g:g + 1], vd[:, g:g + 1],
                                   causal=w.causal, q_offset=w.q_offset, kv_offset=w.kv_offset)
            elif cu is not None:
                oracle.varlen_attention(q64[:, u:u + 1], k64[:, g:g + 1], v64[:, g:g + 1], cu,
                                        causal=w.causal)
            else:
                oracle.full_attention(q64[:, u:u + 1], k64[:, g:g + 1], v64[:, g:g + 1],
                                      causal=w.causal, q_offset=w.q_offset,
                                      kv_offset=w.kv_offset)
            if cu is not None:
                pairs = sum(visible_pairs(b - a, b - a, 1, w.causal, 0, 0)
                            for a, b in zip(cu, cu[1:]))
                full = sum(float(b - a) ** 2 for a, b in zip(cu, cu[1:]))
            else:
                pairs = visible_pairs(Sq, Skv, w.num_chunks, w.causal, w.q_offset, w.kv_offset)
                full = float(Sq) * Skv
            done += 4.0 * D * pairs
            done_full += 4.0 * D * full
        units += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    what = ("key/value head(s) with their query-head group" if w.backward else "query head(s)")
    kind = "backward" if w.backward else ("fp8 forward" if w.fp8 else "forward")
    return {
        "value": done / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
        "kind": "oracle",
        "value_full_matrix": done_full / dt / 1e12,
        "blas": blas_vendor(),
        "sample": f"{units} of {len(unit_list)} {what}, every row, of workload {w.name}'s own "
                  f"seeded inputs (q {list(w.q_shape)}, k/v {list(w.kv_shape)}"
                  f"{', causal' if w.causal else ''}"
                  f"{', rank 0 head shard via the oracle permute' if w.ulysses_P else ''}"
                  f"{', packed documents' if cu is not None else ''}); {kind} oracle, fp64 "
                  f"NumPy on {blas_vendor()}; it computes every masked score of the full "
                  f"matrix: value credits the causal S^2/2 work like the GPU line, "
                  f"value_full_matrix the S^2 it computes; {dt:.1f} s",
    }


# ------------------------------------------------------------------ GPU workloads

def setup_workload(w, chunked, dev):
    """Device inputs and the step's three parts for workload w: pre() (layout / quantize),
    attn() (the timed attention kernel(s)), post(); plus flops, bytes moved by pre/post,
    the roofline peak and extra report keys."""
    import torch
    import long_context_exact_tiled_amd as ra
    import seeded_inputs as si

    B, Hq, Sq, D = w.q_shape
    Skv = w.kv_shape[2]

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16) \
            .to(dev) if w.dtype == "bf16" else torch.from_numpy(x).to(dev)

    flops = attn_flops(B, Hq, Sq, Skv, D, w.num_chunks, w.causal, w.q_offset, w.kv_offset)
    extra, moved = {}, 0
    peak = PEAK_FP8_TFLOPS if w.fp8 else (PEAK_BF16_TFLOPS if w.dtype == "bf16"
                                          else PEAK_F32_TFLOPS)
    noop = lambda: None  # noqa: E731
    pre = post = noop
    if w.ulysses_P:
        qs, ks, vs = (to_dev(x) for x in si.draw_ulysses_sources(w.seed))
        P, r = w.ulysses_P, w.ulysses_rank
        o_seq = torch.zeros_like(qs)
        qh = torch.empty(qs.shape[2] // P, P * qs.shape[1], D, dtype=qs.dtype, device=dev)
        kh = torch.empty(ks.shape[2] // P, P * ks.shape[1], D, dtype=ks.dtype, device=dev)
        vh = torch.empty_like(kh)
        o = torch.empty_like(qh)
        lse = torch.empty(1, qh.shape[0], qh.shape[1], dtype=torch.float32, device=dev)
        moved = 2 * (qh.numel() + 2 * kh.numel() + o.numel()) * qh.element_size()

        def pre():
            ra.ulysses_permute_multi([qs, ks, vs], P, r, 0, outs=[qh, kh, vh])

        def attn():
            ra.attn_fwd(qh.unsqueeze(0), kh.unsqueeze(0), vh.unsqueeze(0), causal=True,
                        out=o.unsqueeze(0), lse=lse)

        def post():
            ra.ulysses_permute(o, P, r, 1, out=o_seq)
    elif w.fp8:
        # bf16 inputs -> e4m3 codes with per-head scales (v transposed), then the fp8
        # attention; the quantization is the step's "pre" part and is reported apart
        q, k, v = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype))
        f8 = torch.float8_e4m3fn
        qc = torch.empty(q.shape, dtype=f8, device=dev)
        kc = torch.empty(k.shape, dtype=f8, device=dev)
        vtc = torch.empty(B, k.shape[1], D, (Skv + 15) // 16 * 16, dtype=f8, device=dev)
        qd = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        kd = torch.empty(B, k.shape[1], dtype=torch.float32, device=dev)
        vd = torch.empty_like(kd)
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        # quantizer traffic: two reads of the bf16 inputs (max pass, convert pass) and
        # one write of the codes
        extra["quantize_bytes"] = int(2 * (q.numel() + k.numel() + v.numel()) * 2
                                      + q.numel() + k.numel() + vtc.numel())
        extra["kernel"] = "attn_fwd_fp8"

        def pre():  # q, k and v in one two-launch call
            ra.fp8_quantize_multi([q, k, v], [False, False, True], outs=[qc, kc, vtc],
                                  descales=[qd, kd, vd], workspace=ws)

        def attn():
            ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=w.causal, out=o, lse=lse)
    elif w.packed_docs:
        q, k, v = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype))
        cu = si.draw_doc_offsets(w.seed, Sq)
        cud = torch.tensor(cu, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        flops = sum(attn_flops(B, Hq, b - a, b - a, D, 1, w.causal) for a, b in zip(cu, cu[1:]))
        extra["documents"] = len(cu) - 1
        if w.backward:
            ra.attn_fwd_varlen(q, k, v, cud, causal=w.causal, out=o, lse=lse)
            do = to_dev(si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype, with_dout=True)[3])
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(max(ra.attn_bwd_workspace_size(q, k, causal=w.causal), 256),
                             dtype=torch.uint8, device=dev)
            flops *= 2.5
            extra["kernel"] = "attn_bwd_varlen (delta + dkdv + dq)"

            def attn():
                ra.attn_bwd_varlen(q, k, v, o, do, lse, cud, causal=w.causal, dq=dq, dk=dk,
                                   dv=dv, workspace=ws)
        else:
            extra["kernel"] = "attn_fwd_varlen"

            def attn():
                ra.attn_fwd_varlen(q, k, v, cud, causal=w.causal, out=o, lse=lse)
    elif w.backward:
        q, k, v, do = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype,
                                                      with_dout=True))
        kw = dict(causal=w.causal, num_chunks=w.num_chunks, start_chunk=w.start_chunk,
                  q_offset=w.q_offset, kv_offset=w.kv_offset)
        o, lse = ra.attn_fwd(q, k, v, **kw)
        ws = torch.empty(max(ra.attn_bwd_workspace_size(q, k, **kw), 256),
                         dtype=torch.uint8, device=dev)
        flops *= 2.5  # five matrix products per (query, key) pair against the forward's two
        if chunked:
            # one ring rank's backward as the ring delivers the chunks: one accumulating
            # step per visible chunk into fp32 accumulators (zeroed before each pass)
            dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
            dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
            dv = torch.zeros(v.shape, dtype=torch.float32, device=dev)
            extra["kernel"] = "attn_bwd_accum per visible chunk (delta + dkdv + dq each)"

            def pre():
                dq.zero_()
                dk.zero_()
                dv.zero_()

            def attn():
                ra.ring_attn_bwd_chunked(q, k, v, o, do, lse, dq_acc=dq, dk_acc=dk, dv_acc=dv,
                                         workspace=ws, **kw)
        else:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            extra["kernel"] = "attn_bwd (delta + dkdv + dq)"

            def attn():
                ra.attn_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    else:
        q, k, v = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        kw = dict(causal=w.causal, num_chunks=w.num_chunks, start_chunk=w.start_chunk,
                  q_offset=w.q_offset, kv_offset=w.kv_offset)
        if chunked:
            extra["kernel"] = "attn_fwd per visible chunk (fp32 partials) + lse_merge"

            def attn():
                ra.ring_attn_chunked(q, k, v, **kw)

            # the merge alone: partials of the visible chunks computed once, then
            # lse_merge timed by itself (HBM-bound: every partial read once, the result
            # written once)
            L = Skv // w.num_chunks
            chunks = ra.ring_visible_chunks(Sq, Skv, num_chunks=w.num_chunks,
                                            start_chunk=w.start_chunk, causal=w.causal,
                                            q_offset=w.q_offset, kv_offset=w.kv_offset)
            parts = [ra.attn_fwd(q, k[:, :, c * L:(c + 1) * L], v[:, :, c * L:(c + 1) * L],
                                 causal=w.causal, q_offset=w.q_offset,
                                 kv_offset=w.kv_offset + c * L, out_dtype=torch.float32)
                     for c in chunks]
            mo, ml = ra.lse_merge([x[0] for x in parts], [x[1] for x in parts])
            mbytes = sum(x[0].numel() * 4 + x[1].numel() * 4 for x in parts) + \
                mo.numel() * mo.element_size() + ml.numel() * 4

            def merge():
                ra.lse_merge([x[0] for x in parts], [x[1] for x in parts], out=mo, lse=ml)
            extra["_merge"] = (merge, mbytes, len(parts))
        else:
            def attn():
                ra.attn_fwd(q, k, v, out=o, lse=lse, **kw)
    return dict(pre=pre, attn=attn, post=post, flops=flops, moved=moved, peak=peak, extra=extra)


def time_step(s, warmup, steps, stream):
    """W untimed steps, then K timed ones with HIP events on the stream around each part.
    Returns (total ms per step, attention ms per step list, pre+post ms list)."""
    import torch
    for _ in range(warmup):
        s["pre"](); s["attn"](); s["post"]()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for e in ev:
        e[0].record(stream)
        s["pre"]()
        e[1].record(stream)
        s["attn"]()
        e[2].record(stream)
        s["post"]()
        e[3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    side_ms = [e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in ev]
    return total_ms / steps, attn_ms, side_ms


def time_calls(fn, stream, reps=5, inner=20):
    """Median per-call ms of `inner` back-to-back calls, over `reps` samples."""
    import torch
    fn()
    torch.cuda.synchronize()
    mt = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(inner):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        mt.append(e0.elapsed_time(e1) / inner)
    return float(np.median(mt))


# The other workloads of the hot path, reported beside the headline in the default run:
# (report key, workload, chunk by chunk)
SECONDARY = [
    ("llama7b_8k_fwd", "llama7b_causal_8k", False),
    ("ring8_rank3_32k_fused_fwd", "ring8_rank3_32k", False),
    ("ring8_rank3_32k_chunked_fwd", "ring8_rank3_32k", True),
    ("llama7b_16k_bwd", "llama7b_causal_bwd_16k", False),
    ("qwen7b_gqa_32k_fp8_fwd", "qwen7b_gqa_32k_fp8", False),
    ("qwen7b_packed_32k_fwd", "qwen7b_packed_32k", False),
    ("qwen7b_packed_32k_bwd", "qwen7b_packed_bwd_32k", False),
]


def secondary_lines(dev, stream, min_warmup_ms=150.0, steps=20):
    """Attention TFLOP/s and fraction of peak of each secondary workload (warm clocks:
    untimed calls for at least min_warmup_ms first), the merge's GB/s for the chunked
    ring share."""
    import torch
    import seeded_inputs as si
    out = {}
    for key, name, chunked in SECONDARY:
        w = si.WORKLOADS[name]
        s = setup_workload(w, chunked, dev)
        s["attn"]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        s["attn"]()
        torch.cuda.synchronize()
        est_ms = max((time.perf_counter() - t0) * 1e3, 0.05)
        warm = int(min(400, max(5, math.ceil(min_warmup_ms / est_ms))))
        _, attn_ms, _ = time_step(s, warm, steps, stream)
        ms = float(np.median(attn_ms))
        tf = s["flops"] / (ms * 1e-3) / 1e12
        out[f"{key}_ms"] = ms
        out[f"{key}_tflops"] = tf
        out[f"{key}_frac"] = tf / s["peak"]
        if "quantize_bytes" in s["extra"]:  # the FP8 step's quantization of q, k, v
            qms = time_calls(s["pre"], stream)
            out[f"{key}_quantize_ms"] = qms
            out[f"{key}_quantize_GBps"] = s["extra"]["quantize_bytes"] / (qms * 1e-3) / 1e9
        if "_merge" in s["extra"]:
            merge, mbytes, nparts = s["extra"]["_merge"]
            mms = time_calls(merge, stream)
            out["ring8_rank3_32k_merge_parts"] = nparts
            out["ring8_rank3_32k_merge_ms"] = mms
            out["ring8_rank3_32k_merge_GBps"] = mbytes / (mms * 1e-3) / 1e9
            out["ring8_rank3_32k_merge_frac_of_hbm_peak"] = \
                out["ring8_rank3_32k_merge_GBps"] / PEAK_HBM_GBPS
        del s
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # untimed steps: the GPU's clocks take tens of milliseconds of load to settle (five
    # warm-up steps of the headline measured 2 % slower than a hundred)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads reported beside the headline")
    ap.add_argument("--chunked", action="store_true",
                    help="ring workloads: one attn_fwd per visible chunk + lse_merge "
                         "(backward: one attn_bwd_accum per visible chunk)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: every box here has a single MI355X, and the multi-GPU "
              "ring/Ulysses exchange is not part of this build (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    s = setup_workload(w, args.chunked, dev)
    flops, moved, peak, extra = s["flops"], s["moved"], s["peak"], s["extra"]

    ms_step, attn_ms, side_ms = time_step(s, args.warmup, args.steps, stream)
    attn_avg = float(np.mean(attn_ms))
    achieved = flops / (attn_avg * 1e-3) / 1e12
    if w.fp8:
        extra["quantize_ms_per_step"] = float(np.mean(side_ms))
        extra["quantize_GBps"] = extra["quantize_bytes"] / (np.mean(side_ms) * 1e-3) / 1e9
    if moved:
        extra["permute_ms_per_step"] = float(np.mean(side_ms))
        extra["permute_GBps"] = moved / (np.mean(side_ms) * 1e-3) / 1e9
        # cold-cache rate: reading 1 GiB evicts the 256 MB Infinity Cache (and the L2s)
        # before each pass.  A flush by writing 1 GiB evicts them too but leaves them full
        # of dirty lines whose write-back then runs inside the timed pass; that rate is
        # reported beside it (permute_cold_write_flush_*).
        scratch = torch.zeros(1 << 27, dtype=torch.int64, device=dev)

        def cold_passes(flush):
            cold = []
            for _ in range(5):
                flush()
                e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record(stream)
                s["pre"]()
                e1.record(stream)
                flush()
                e2, e3 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e2.record(stream)
                s["post"]()
                e3.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) + e2.elapsed_time(e3))
            return float(np.median(cold))

        ms_r = cold_passes(lambda: scratch.sum())
        ms_w = cold_passes(lambda: scratch.zero_())
        del scratch
        extra["permute_cold_ms_per_step"] = ms_r
        extra["permute_cold_GBps"] = moved / (ms_r * 1e-3) / 1e9
        extra["permute_cold_write_flush_ms_per_step"] = ms_w
        extra["permute_cold_write_flush_GBps"] = moved / (ms_w * 1e-3) / 1e9
    merge = extra.pop("_merge", None)
    if merge is not None:
        fn, mbytes, nparts = merge
        mms = time_calls(fn, stream)
        extra["merge_parts"] = nparts
        extra["merge_ms"] = mms
        extra["merge_GBps"] = mbytes / (mms * 1e-3) / 1e9
        extra["merge_frac_of_hbm_peak"] = extra["merge_GBps"] / PEAK_HBM_GBPS
    extra["attn_fwd_ms"] = attn_avg
    extra["attn_fwd_ms_median"] = float(np.median(attn_ms))
    extra["attn_fwd_ms_min"] = float(np.min(attn_ms))
    extra["attn_flops"] = flops
    kernel = extra.pop("kernel", "attn_fwd")
    del s
    torch.cuda.empty_cache()
    if w.name == HEADLINE and not args.chunked and not args.no_secondary:
        extra.update(secondary_lines(dev, stream))

    line = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if w.fp8 else w.dtype,
        "data": "synthetic: N(0,1) from PCG64(seed), rounded to bf16 (RNE)",
        "config": {"workload": w.name, "q_shape": list(w.q_shape), "kv_shape": list(w.kv_shape),
                   "causal": w.causal, "num_chunks": w.num_chunks, "start_chunk": w.start_chunk,
                   "q_offset": w.q_offset, "ulysses_P": w.ulysses_P,
                   "ulysses_rank": w.ulysses_rank, "parallelism": "1 GPU (one rank's share)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "kernel": kernel},
        "cpu_baseline": None,
        **extra,
    }
    if w.name == HEADLINE and not args.chunked:
        line["roofline"]["traffic"] = measured_traffic()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
