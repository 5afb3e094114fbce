"""GPU parity of the FP8 path: ra_fp8_quantize (bit-exact codes and descales) and
ra_attn_fwd_fp8 (against exact attention of the dequantized inputs).

Inputs of the attention tests are quantized by the oracle on the CPU, so no GPU result
feeds the reference.  Tolerance (derived in the oracle's fp8 module): the GPU rounds
the attention weights (scaled by 2^6) to e4m3 for the P V product, which gives the
element-wise bound  2^-4 sum_j p_j |v_j| + 2^-16 n_sub max_j |v_j|  (oracle.fp8.
p_rounding_bound); on top of it come the bf16 rounding of o (2^-9 |o|, taken as 2^-8 of
the reference) and fp32 arithmetic (1e-5).  lse is formed from the unrounded fp32
weights: max abs 1e-3 (the bf16 forward's stated bound; fp32 sums of up to 32K terms).
"""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
from oracle import fp8 as ofp8
import seeded_inputs as si
from _gpu import require_gpu, sample_rows, say, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _codes_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda().view(torch.float8_e4m3fn)


def _codes_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


# ---------------------------------------------------------------------------- quantizer

QCASES = [  # shape, transpose, per-head magnitudes
    ((1, 3, 100, 128), False, (1.0, 30.0, 1e-3)),
    ((1, 3, 100, 128), True, (1.0, 30.0, 1e-3)),
    ((2, 2, 37, 64), True, (5.0, 0.0, 0.2, 1.0)),   # an all-zero head
    ((2, 2, 37, 64), False, (5.0, 0.0, 0.2, 1.0)),
    ((1, 1, 4096, 128), True, (3.0,)),
    ((1, 2, 1, 16), True, (1.0, 2.0)),
    ((1, 2, 0, 64), True, (1.0, 1.0)),              # no tokens: descale 1, nothing else
    # row lengths whose 16-byte pieces do not divide a block's threads (48: 6 per row,
    # 42 rows per pass, 4 threads idle) or fill it with few rows (256: 8 rows per pass),
    # with several row ranges per head and ragged last passes
    ((1, 2, 3001, 48), False, (2.0, 0.5)),
    ((1, 2, 3001, 48), True, (2.0, 0.5)),
    ((1, 1, 701, 256), False, (7.0,)),
    ((1, 1, 701, 256), True, (7.0,)),
]


@pytest.mark.parametrize("case", QCASES, ids=lambda c: f"{c[0]}-t{int(c[1])}")
def test_quantize_bit_exact(case):
    shape, transpose, mags = case
    say(f"fp8 quantize {shape} transpose={transpose}")
    B, H = shape[:2]
    rng = np.random.default_rng(sum(shape) + transpose)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.asarray(mags, dtype=np.float32).reshape(B, H, 1, 1)
    bits = si.bf16_bits(x)
    x32 = si.bf16_bits_to_f32(bits)
    codes_ref, desc_ref = ofp8.quantize_heads(x32)
    if transpose:
        codes_ref = ofp8.transpose_codes(codes_ref)
    xd = _bf16_dev(bits)
    # fill the outputs first so that unwritten bytes fail
    out = torch.full(codes_ref.shape, 0x55, dtype=torch.uint8, device="cuda").view(
        torch.float8_e4m3fn)
    desc = torch.full((B, H), float("nan"), device="cuda")
    ra.fp8_quantize(xd, transpose=transpose, out=out, descale=desc)
    torch.cuda.synchronize()
    assert np.array_equal(desc.cpu().numpy(), desc_ref)
    got = _codes_np(out)
    bad = np.argwhere(got != codes_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"


def test_quantize_multi_bit_exact():
    """q, k (rows) and v (transposed) of different shapes in one two-launch call: every
    code and descale bitwise the oracle's, and the same as three single calls."""
    say("fp8 quantize multi")
    rng = np.random.default_rng(5)
    shapes = [((1, 7, 300, 128), False), ((1, 1, 300, 128), False), ((1, 1, 300, 128), True),
              ((2, 3, 37, 64), True)]
    xs, refs = [], []
    for shape, t in shapes:
        x = rng.standard_normal(shape).astype(np.float32) * rng.uniform(0.1, 30.0)
        bits = si.bf16_bits(x)
        c, d = ofp8.quantize_heads(si.bf16_bits_to_f32(bits))
        refs.append((ofp8.transpose_codes(c) if t else c, d))
        xs.append(_bf16_dev(bits))
    outs = [torch.full(r[0].shape, 0x55, dtype=torch.uint8, device="cuda").view(
        torch.float8_e4m3fn) for r in refs]
    descs = [torch.full(r[1].shape, float("nan"), device="cuda") for r in refs]
    ra.fp8_quantize_multi(xs, [t for _, t in shapes], outs=outs, descales=descs)
    singles = [ra.fp8_quantize(x, transpose=t) for x, (_, t) in zip(xs, shapes)]
    torch.cuda.synchronize()
    for o, d, (cref, dref), (so, sd) in zip(outs, descs, refs, singles):
        assert np.array_equal(d.cpu().numpy(), dref)
        assert np.array_equal(_codes_np(o), cref)
        assert torch.equal(o.view(torch.uint8), so.view(torch.uint8))
        assert torch.equal(d, sd)


def test_quantize_strided_source():
    """A [B, S, H, D] buffer viewed as [B, H, S, D] quantizes like its contiguous copy."""
    say("fp8 quantize strided source")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 50, 4, 64)).astype(np.float32)
    bits = si.bf16_bits(x)
    xd = _bf16_dev(bits).permute(0, 2, 1, 3)
    codes, desc = ra.fp8_quantize(xd, transpose=True)
    ref_codes, ref_desc = ofp8.quantize_heads(si.bf16_bits_to_f32(bits).transpose(0, 2, 1, 3))
    torch.cuda.synchronize()
    assert np.array_equal(desc.cpu().numpy(), ref_desc)
    assert np.array_equal(_codes_np(codes), ofp8.transpose_codes(ref_codes))


# ---------------------------------------------------------------------------- attention

def _fp8_inputs(B, Hq, Hkv, Sq, Skv, D, seed):
    q, k, v = si.draw_qkv(seed, (B, Hq, Sq, D), (B, Hkv, Skv, D), "bf16")
    (qc, qd), (kc, kd), (vc, vd) = (ofp8.quantize_heads(si.bf16_bits_to_f32(t)) for t in (q, k, v))
    vtc = ofp8.transpose_codes(vc)
    dev = (_codes_dev(qc), _codes_dev(kc), _codes_dev(vtc),
           *(torch.from_numpy(d).cuda() for d in (qd, kd, vd)))
    deq = (ofp8.dequantize(qc, qd), ofp8.dequantize(kc, kd), ofp8.dequantize(vc, vd))
    return dev, deq


def _check(o_got, l_got, o_ref, l_ref, bound, what):
    assert np.isfinite(o_got).all(), f"{what}: non-finite o"
    err = np.abs(o_got - o_ref)
    tol = bound + 2.0 ** -8 * np.abs(o_ref) + 1e-5
    worst = float((err / tol).max(initial=0.0))
    print(f"[parity] {what}: max|err|={err.max(initial=0):.3e} mean|err|="
          f"{err.mean() if err.size else 0:.3e} max err/bound={worst:.3f} "
          f"mean bound={bound.mean() if bound.size else 0:.3e}", flush=True)
    assert worst <= 1.0, f"{what}: error exceeds the derived bound ({worst:.3f} x)"
    assert np.array_equal(np.isneginf(l_got), np.isneginf(l_ref)), f"{what}: -inf pattern"
    fin = np.isfinite(l_ref)
    lerr = float(np.abs(l_got[fin] - l_ref[fin]).max(initial=0.0))
    assert lerr <= 1e-3, f"{what}: lse max abs err {lerr}"


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off
    # (fused ring chunks are whole 16-key units; their last tiles are ragged)
    (1, 2, 2, 300, 300, 128, True, 1, 0, 0, 0),
    (2, 4, 2, 200, 336, 64, False, 3, 1, 0, 0),
    (1, 4, 1, 256, 256, 128, True, 4, 1, 0, 0),
    (1, 2, 2, 144, 432, 128, True, 3, 2, 288, 0),
    (1, 2, 1, 70, 432, 64, False, 3, 0, 0, 0),
    (1, 3, 1, 100, 5 * 48, 128, True, 5, 3, 96, 0),
    (1, 7, 1, 333, 333, 128, True, 1, 0, 0, 0),
    (1, 2, 2, 200, 200, 128, True, 1, 0, 0, 100),   # rows with no visible key
    (1, 2, 2, 1, 1, 64, True, 1, 0, 0, 0),
    (1, 2, 2, 64, 0, 128, False, 1, 0, 0, 0),       # no keys at all
    (1, 6, 2, 700, 700, 64, True, 1, 0, 0, 0),      # 64-dim grouped heads, several tiles
    (1, 2, 2, 256, 768, 64, True, 3, 1, 256, 0),    # 64-dim causal ring share, fused
    (2, 3, 1, 250, 250, 128, True, 1, 0, 0, 0),     # two batches, work-counter order
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_small_fp8(case):
    B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off = case
    say(f"fp8 attn {case}")
    (qc, kc, vtc, qd, kd, vd), (q, k, v) = _fp8_inputs(B, Hq, Hkv, Sq, Skv, D,
                                                        sum(map(ord, str(case))) % 1009)
    kw = dict(causal=causal, num_chunks=P, start_chunk=start, q_offset=q_off, kv_offset=kv_off)
    o = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.full_attention(q, k, v, causal=causal, q_offset=q_off,
                                         kv_offset=kv_off)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Sq)]
    bound = ofp8.p_rounding_bound(q, k, v, rows, causal=causal, q_offset=q_off,
                                  kv_offset=kv_off).reshape(o_ref.shape)
    _check(to_np64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, bound, "o")


def test_fp32_output_and_explicit_scale():
    say("fp8 attn fp32 output, scale 0.05")
    (qc, kc, vtc, qd, kd, vd), (q, k, v) = _fp8_inputs(1, 4, 2, 190, 190, 128, 21)
    o, lse = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=True, scale=0.05,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.full_attention(q, k, v, causal=True, scale=0.05)
    rows = [(0, h, i) for h in range(4) for i in range(190)]
    bound = ofp8.p_rounding_bound(q, k, v, rows, causal=True, scale=0.05).reshape(o_ref.shape)
    _check(o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref,
           l_ref, bound, "o fp32")


def test_fp8_deterministic():
    say("fp8 attn determinism")
    (qc, kc, vtc, qd, kd, vd), _ = _fp8_inputs(1, 4, 1, 700, 700, 128, 31)
    a = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=True)
    b = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.fixture(scope="module")
def qwen32k_fp8():
    """The headline attention shape (q [1, 7, 32768, 128], k, v [1, 1, 32768, 128],
    causal) in fp8, run once: the quantizer's codes for the bf16 tensors (bit-exact), then
    the attention on the oracle's codes."""
    w = si.WORKLOADS["qwen7b_gqa_32k_fp8"]
    say(f"workload {w.name}")
    q, k, v = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, "bf16")
    qx, kx, vx = (si.bf16_bits_to_f32(t) for t in (q, k, v))
    (qc, qd), (kc, kd), (vc, vd) = (ofp8.quantize_heads(t) for t in (qx, kx, vx))
    vtc = ofp8.transpose_codes(vc)
    gq, gqd = ra.fp8_quantize(_bf16_dev(q))
    gk, gkd = ra.fp8_quantize(_bf16_dev(k))
    gv, gvd = ra.fp8_quantize(_bf16_dev(v), transpose=True)
    torch.cuda.synchronize()
    for got, ref, name in ((gq, qc, "q"), (gk, kc, "k"), (gv, vtc, "vt")):
        assert np.array_equal(_codes_np(got), ref), f"{name} codes differ"
    for got, ref in ((gqd, qd), (gkd, kd), (gvd, vd)):
        assert np.array_equal(got.cpu().numpy(), ref)
    del gq, gk, gv
    o, lse = ra.attn_fwd_fp8(_codes_dev(qc), _codes_dev(kc), _codes_dev(vtc),
                             *(torch.from_numpy(d).cuda() for d in (qd, kd, vd)), causal=True)
    torch.cuda.synchronize()
    deq = (ofp8.dequantize(qc, qd), ofp8.dequantize(kc, kd), ofp8.dequantize(vc, vd))
    return w, to_np64(o), lse.cpu().numpy().astype(np.float64), deq


def test_qwen7b_gqa_32k_fp8_workload_sampled_rows(qwen32k_fp8):
    w, o_n, l_n, (q64, k64, v64) = qwen32k_fp8
    B, Hq, Sq, D = w.q_shape
    idx = sample_rows(B, Hq, Sq, per_head=4, seed=w.seed)
    o_ref, l_ref = oracle.attention_rows(q64, k64, v64, idx, causal=True)
    bound = ofp8.p_rounding_bound(q64, k64, v64, idx, causal=True)
    got_o = np.stack([o_n[b, h, i] for (b, h, i) in idx])
    got_l = np.array([l_n[b, h, i] for (b, h, i) in idx])
    _check(got_o, got_l, o_ref, l_ref, bound, "o sampled")


@pytest.mark.parametrize("h", [0, 3, 6])
def test_qwen7b_gqa_32k_fp8_workload_whole_head(qwen32k_fp8, h):
    """Every row of query head h within the derived bound."""
    w, o_n, l_n, (q64, k64, v64) = qwen32k_fp8
    o_ref, l_ref = oracle.full_attention(q64[:, h:h + 1], k64, v64, causal=True)
    bound = ofp8.p_rounding_bound_head(q64, k64, v64, 0, h, causal=True)
    _check(o_n[0, h], l_n[0, h], o_ref[0, 0], l_ref[0, 0], bound, f"o head {h} (all rows)")


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_ring_chunked_and_fused(causal):
    """One device's ring share in fp8, chunk by chunk (fp32 partials + lse_merge) and
    fused: both within the derived bound of the exact result.  Merging weighs each
    chunk's error by the chunk's share of the row, so the bound carries over."""
    B, Hq, Hkv, Sq, P, L, start, q_off = 1, 4, 2, 256, 4, 208, 1, 500
    say(f"fp8 ring causal={causal}")
    (qc, kc, vtc, qd, kd, vd), (q, k, v) = _fp8_inputs(B, Hq, Hkv, Sq, P * L, 128,
                                                        77 + int(causal))
    kw = dict(causal=causal, num_chunks=P, start_chunk=start, q_offset=q_off)
    o_c, l_c = ra.ring_attn_fp8_chunked(qc, kc, vtc, qd, kd, vd, **kw)
    o_f, l_f = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.full_attention(q, k, v, causal=causal, q_offset=q_off)
    rows = [(0, h, i) for h in range(Hq) for i in range(Sq)]
    bound = ofp8.p_rounding_bound(q, k, v, rows, causal=causal,
                                  q_offset=q_off).reshape(o_ref.shape)
    for o, l, what in ((o_c, l_c, "chunked"), (o_f, l_f, "fused")):
        _check(to_np64(o), l.cpu().numpy().astype(np.float64), o_ref, l_ref, bound, what)


def test_fp8_work_counter_changes_order_not_results():
    """The FP8 kernel takes query tiles from the stream's work counter when B*Hq is not a
    multiple of 8: bitwise the outputs of the fixed order, whatever the counter held,
    and the counter is left as it was."""
    say("fp8 work counter")
    (qc, kc, vtc, qd, kd, vd), _ = _fp8_inputs(1, 7, 1, 900, 900, 128, 33)
    o0, l0 = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=True, sched=False)
    ra._sched_counter(qc)
    ctr = ra._SCHED[(qc.device.index, torch.cuda.current_stream(qc.device).cuda_stream)]
    for start in (0, 77, 2**33 + 5):
        ctr.fill_(start)
        o1, l1 = ra.attn_fwd_fp8(qc, kc, vtc, qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), start
        assert torch.equal(l1.view(torch.int32), l0.view(torch.int32)), start
        assert int(ctr.item()) == start
    ctr.zero_()
