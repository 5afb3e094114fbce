"""Benchmark of the exact blockwise attention hot path on one MI355X.

One step = one pass of the whole forward hot path over one batch of synthetic input.
For the headline workload (a Qwen2.5-7B-shaped GQA layer, 28 query / 4 key-value heads
x 128, one rank's share of a 4-way Ulysses split at 32K tokens):

    ulysses_permute(q), (k), (v)   sequence shards -> rank 0's head shard
    attn_fwd                       causal, GQA 7:1, S = 32768, bf16 in, fp32 accumulate
    ulysses_permute(o)             head shard -> sequence shards

Prints ONE JSON line.  ``value`` is the algorithmic attention TFLOP/s of the whole step
(inputs resident in HBM; flops use the causal S^2/2 convention, 2 flops per MAC);
``roofline`` reports the attention kernel alone, timed with HIP events on the stream it
runs on; ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload.  Other workloads can be selected with --workload.
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


def cpu_baseline(w, budget_s: float = 15.0):
    """Time the fp64 oracle on blocks of query rows spread over the sequence."""
    import oracle
    import seeded_inputs as si

    B, Hq, Sq, D = w.q_shape
    Skv = w.kv_shape[2]
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    k = rng.standard_normal((1, 1, Skv, D), dtype=np.float32)
    v = rng.standard_normal((1, 1, Skv, D), dtype=np.float32)
    k64 = si.bf16_bits_to_f32(si.bf16_bits(k)).astype(np.float64)
    v64 = si.bf16_bits_to_f32(si.bf16_bits(v)).astype(np.float64)
    blk = 128
    # Passes over the sequence (a fresh random order of its 128-row blocks each, one pass
    # per query head at most) until the time budget is spent.
    starts = []
    for _ in range(B * Hq):
        order = list(range(0, Sq, blk))
        rng.shuffle(order)
        starts += order
    if w.fp8:  # the context's codes are set up once, like the inputs, before timing
        from oracle import fp8 as ofp8
        kc, kdd = ofp8.quantize_heads(k64.astype(np.float32))
        vc, vdd = ofp8.quantize_heads(v64.astype(np.float32))
    done_flops, rows, t0 = 0.0, 0, time.perf_counter()
    cu = si.draw_doc_offsets(w.seed, Sq) if w.packed_docs else None
    for a in starts:
        qb = si.bf16_bits_to_f32(si.bf16_bits(
            rng.standard_normal((1, 1, blk, D), dtype=np.float32))).astype(np.float64)
        if cu is not None:  # rows of one document against that document's keys
            d = max(i for i in range(len(cu) - 1) if cu[i] <= a)
            lo, hi = cu[d], cu[d + 1]
            n = min(blk, hi - a)
            kk, vv = k64[:, :, lo:hi], v64[:, :, lo:hi]
            if w.backward:
                nk = min(hi - lo, a - lo + n) if w.causal else hi - lo
                oracle.attention_bwd(qb[:, :, :n], kk[:, :, :nk], vv[:, :, :nk], qb[:, :, :n],
                                     causal=w.causal, q_offset=a - lo)
                done_flops += 2.5 * attn_flops(1, 1, n, hi - lo, D, 1, w.causal, a - lo, 0)
            else:
                oracle.full_attention(qb[:, :, :n], kk, vv, causal=w.causal, q_offset=a - lo)
                done_flops += attn_flops(1, 1, n, hi - lo, D, 1, w.causal, a - lo, 0)
        elif w.fp8:  # the fp8 oracle: quantize the block (per-head rule), then exact
            # attention of the dequantized values over the context quantized up front
            qc, qdd = ofp8.quantize_heads(qb.astype(np.float32))
            ofp8.fp8_attention(qc, kc, vc, qdd, kdd, vdd, causal=w.causal,
                               q_offset=w.q_offset + a, kv_offset=w.kv_offset)
            done_flops += attn_flops(1, 1, blk, Skv, D, 1, w.causal, w.q_offset + a,
                                     w.kv_offset)
        elif w.backward:  # all five products for the block's (query, key) pairs
            nk = min(Skv, w.q_offset + a + blk - w.kv_offset) if w.causal else Skv
            oracle.attention_bwd(qb, k64[:, :, :nk], v64[:, :, :nk], qb, causal=w.causal,
                                 q_offset=w.q_offset + a, kv_offset=w.kv_offset)
            done_flops += 2.5 * attn_flops(1, 1, blk, Skv, D, 1, w.causal, w.q_offset + a,
                                           w.kv_offset)
        else:
            oracle.full_attention(qb, k64, v64, causal=w.causal, q_offset=w.q_offset + a,
                                  kv_offset=w.kv_offset)
            done_flops += attn_flops(1, 1, blk, Skv, D, 1, w.causal, w.q_offset + a,
                                     w.kv_offset)
        rows += blk
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{rows} query rows ({rows // blk} blocks of {blk} at random positions, "
                  f"{math.ceil(rows / Sq)} pass(es) over the sequence) of one head against its "
                  f"{'causal ' if w.causal else ''}"
                  f"{'own document' if cu is not None else str(Skv) + '-key context'}, "
                  f"{'backward' if w.backward else ('fp8 forward' if w.fp8 else 'forward')} "
                  f"oracle{' (context quantized before timing)' if w.fp8 else ''}, fp64 "
                  f"NumPy, {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # untimed steps: the GPU's clocks take tens of milliseconds of load to settle (five
    # warm-up steps of the headline measured 2 % slower than a hundred)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="qwen7b_ulysses4_rank0_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
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
    import long_context_exact_tiled_amd as ra
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Sq, D = w.q_shape
    Skv = w.kv_shape[2]

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev) \
            if w.dtype == "bf16" else torch.from_numpy(x).to(dev)

    flops = attn_flops(B, Hq, Sq, Skv, D, w.num_chunks, w.causal, w.q_offset, w.kv_offset)
    extra = {}
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
            ra.ulysses_permute(qs, P, r, 0, out=qh)
            ra.ulysses_permute(ks, P, r, 0, out=kh)
            ra.ulysses_permute(vs, P, r, 0, out=vh)

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
        moved = 0
        # quantizer traffic: two reads of the bf16 inputs (max pass, convert pass) and
        # one write of the codes
        extra["quantize_bytes"] = int(2 * (q.numel() + k.numel() + v.numel()) * 2
                                      + q.numel() + k.numel() + vtc.numel())
        extra["kernel"] = "attn_fwd_fp8"

        def pre():
            ra.fp8_quantize(q, out=qc, descale=qd, workspace=ws)
            ra.fp8_quantize(k, out=kc, descale=kd, workspace=ws)
            ra.fp8_quantize(v, transpose=True, out=vtc, descale=vd, workspace=ws)

        def attn():
            ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=w.causal, out=o, lse=lse)

        def post():
            pass
    elif w.packed_docs:
        q, k, v = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype))
        cu = si.draw_doc_offsets(w.seed, Sq)
        cud = torch.tensor(cu, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        flops = sum(attn_flops(B, Hq, b - a, b - a, D, 1, w.causal) for a, b in zip(cu, cu[1:]))
        moved = 0
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

        def pre():
            pass

        def post():
            pass
    elif w.backward:
        q, k, v, do = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype,
                                                      with_dout=True))
        kw = dict(causal=w.causal, num_chunks=w.num_chunks, start_chunk=w.start_chunk,
                  q_offset=w.q_offset, kv_offset=w.kv_offset)
        o, lse = ra.attn_fwd(q, k, v, **kw)
        ws = torch.empty(max(ra.attn_bwd_workspace_size(q, k, **kw), 256),
                         dtype=torch.uint8, device=dev)
        flops *= 2.5  # five matrix products per (query, key) pair against the forward's two
        moved = 0
        if args.chunked:
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

            def pre():
                pass

            def attn():
                ra.attn_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

        def post():
            pass
    else:
        q, k, v = (to_dev(x) for x in si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        moved = 0
        kw = dict(causal=w.causal, num_chunks=w.num_chunks, start_chunk=w.start_chunk,
                  q_offset=w.q_offset, kv_offset=w.kv_offset)

        def pre():
            pass

        if args.chunked:
            extra["kernel"] = "attn_fwd per visible chunk (fp32 partials) + lse_merge"

            def attn():
                ra.ring_attn_chunked(q, k, v, **kw)
        else:
            def attn():
                ra.attn_fwd(q, k, v, out=o, lse=lse, **kw)

        def post():
            pass

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        pre(); attn(); post()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for s in range(args.steps):
        ev[s][0].record(stream)
        pre()
        ev[s][1].record(stream)
        attn()
        ev[s][2].record(stream)
        post()
        ev[s][3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    perm_ms = [e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in ev]
    attn_avg = float(np.mean(attn_ms))
    achieved = flops / (attn_avg * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if w.fp8 else (PEAK_BF16_TFLOPS if w.dtype == "bf16"
                                          else PEAK_F32_TFLOPS)
    if w.fp8:
        extra["quantize_ms_per_step"] = float(np.mean(perm_ms))
        extra["quantize_GBps"] = extra["quantize_bytes"] / (np.mean(perm_ms) * 1e-3) / 1e9
    if moved:
        extra["permute_ms_per_step"] = float(np.mean(perm_ms))
        extra["permute_GBps"] = moved / (np.mean(perm_ms) * 1e-3) / 1e9
        # cold-cache rate: a 1 GiB write evicts the 256 MB Infinity Cache before each pass
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(5):
            scratch.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pre()
            e1.record(stream)
            scratch.zero_()
            e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e2.record(stream)
            post()
            e3.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1) + e2.elapsed_time(e3))
        del scratch
        extra["permute_cold_ms_per_step"] = float(np.median(cold))
        extra["permute_cold_GBps"] = moved / (np.median(cold) * 1e-3) / 1e9
    if args.chunked and not w.backward and not w.fp8:
        # the merge alone: partials of the visible chunks computed once, then lse_merge
        # timed by itself (HBM-bound: every partial read once, the result written once)
        L = w.kv_shape[2] // w.num_chunks
        chunks = ra.ring_visible_chunks(w.q_shape[2], w.kv_shape[2], num_chunks=w.num_chunks,
                                        start_chunk=w.start_chunk, causal=w.causal,
                                        q_offset=w.q_offset, kv_offset=w.kv_offset)
        parts = [ra.attn_fwd(q, k[:, :, c * L:(c + 1) * L], v[:, :, c * L:(c + 1) * L],
                             causal=w.causal, q_offset=w.q_offset,
                             kv_offset=w.kv_offset + c * L, out_dtype=torch.float32)
                 for c in chunks]
        mo, ml = ra.lse_merge([x[0] for x in parts], [x[1] for x in parts])
        torch.cuda.synchronize()
        mt = []
        for _ in range(5):  # 20 back-to-back merges per sample
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                ra.lse_merge([x[0] for x in parts], [x[1] for x in parts], out=mo, lse=ml)
            e1.record(stream)
            torch.cuda.synchronize()
            mt.append(e0.elapsed_time(e1) / 20)
        mbytes = sum(x[0].numel() * 4 + x[1].numel() * 4 for x in parts) + \
            mo.numel() * mo.element_size() + ml.numel() * 4
        extra["merge_parts"] = len(parts)
        extra["merge_ms"] = float(np.median(mt))
        extra["merge_GBps"] = mbytes / (np.median(mt) * 1e-3) / 1e9
        extra["merge_frac_of_hbm_peak"] = extra["merge_GBps"] / PEAK_HBM_GBPS
        del parts
    extra["attn_fwd_ms"] = attn_avg
    extra["attn_fwd_ms_median"] = float(np.median(attn_ms))
    extra["attn_fwd_ms_min"] = float(np.min(attn_ms))
    extra["attn_flops"] = flops

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
                     "frac": achieved / peak, "traffic": None,
                     "kernel": extra.pop("kernel", "attn_fwd")},
        "cpu_baseline": None,
        **extra,
    }
    if w.name == "qwen7b_ulysses4_rank0_32k" and not args.chunked:
        line["roofline"]["traffic"] = measured_traffic()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
