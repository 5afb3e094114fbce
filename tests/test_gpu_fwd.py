"""GPU parity of ra_attn_fwd (and the chunk-by-chunk ring share) against the CPU oracle.

Small cases compare every element; the full-size workloads compare every row of whole
heads (all 7 query heads of the 32K GQA headline, three heads of each 32-head workload)
plus sampled rows of every head.  Inputs come from ``seeded_inputs`` (N(0,1), bf16
rounded by RNE for bf16 cases); the oracle reads the rounded values exactly.
"""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import (check_lse, check_o, gather_lse, gather_rows, require_gpu, sample_rows, say,
                  to_dev, to_np64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run_case(dtype, D, causal, B, Hq, Hkv, Sq, Skv, P=1, start=0, q_off=0, kv_off=0,
              seed=0, out_f32=False, scale=None):
    say(f"fwd {dtype} D={D} causal={causal} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} P={P} "
        f"start={start} q_off={q_off} kv_off={kv_off} out_f32={out_f32}")
    q, k, v = si.draw_qkv(seed, (B, Hq, Sq, D), (B, Hkv, Skv, D), dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out = torch.full(qd.shape, float("nan"), dtype=torch.float32 if out_f32 else qd.dtype,
                     device="cuda")
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ra.attn_fwd(qd, kd, vd, causal=causal, num_chunks=P, start_chunk=start, q_offset=q_off,
                kv_offset=kv_off, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    q64, k64, v64 = si.as_f64(q, dtype), si.as_f64(k, dtype), si.as_f64(v, dtype)
    o_ref, l_ref = oracle.full_attention(q64, k64, v64, causal=causal, scale=scale,
                                         q_offset=q_off, kv_offset=kv_off)
    tol_dtype = dtype
    check_o(to_np64(out), o_ref, tol_dtype)
    check_lse(to_np64(lse), l_ref, tol_dtype)
    return out, lse


CASES = [
    # dtype, D, causal, B, Hq, Hkv, Sq, Skv, P, start, q_off, kv_off
    ("bf16", 128, True, 2, 4, 2, 300, 300, 1, 0, 0, 0),
    ("bf16", 128, False, 1, 2, 2, 300, 513, 3, 2, 0, 0),
    ("bf16", 64, True, 1, 4, 4, 333, 333, 3, 1, 0, 0),
    ("bf16", 64, False, 2, 2, 1, 129, 200, 1, 0, 0, 0),
    ("bf16", 128, True, 1, 7, 1, 700, 700, 1, 0, 0, 0),          # GQA 7:1
    ("bf16", 128, True, 1, 4, 4, 256, 1024, 4, 2, 512, 0),       # one ring rank's share
    ("bf16", 128, True, 1, 2, 2, 200, 200, 1, 0, 0, 100),        # rows with no visible key
    ("bf16", 128, True, 1, 2, 2, 1, 1, 1, 0, 0, 0),
    ("bf16", 128, True, 1, 2, 1, 130, 64, 1, 0, 70, 0),
    ("bf16", 128, True, 1, 2, 1, 300, 800, 8, 5, 500, 0),        # 100-key chunks (< one tile)
    ("bf16", 64, True, 2, 2, 2, 260, 520, 4, 3, 130, 0),         # D=64 causal ring share
    ("f32", 128, True, 1, 2, 2, 200, 200, 2, 1, 0, 0),
    ("f32", 64, False, 2, 2, 1, 150, 260, 4, 3, 0, 0),
    ("f32", 64, True, 1, 3, 3, 190, 380, 2, 1, 190, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_small_parity(case):
    dtype, D, causal, B, Hq, Hkv, Sq, Skv, P, start, q_off, kv_off = case
    _run_case(dtype, D, causal, B, Hq, Hkv, Sq, Skv, P, start, q_off, kv_off, seed=sum(map(ord, str(case))) % 997)


@pytest.mark.parametrize("D,causal,P,start", [(128, True, 1, 0), (64, False, 1, 0),
                                             (128, True, 4, 2), (64, True, 3, 1)])
def test_running_max_moves(D, causal, P, start):
    """Scores that grow along the key axis (keys scaled up to 9x) after three keys scaled
    6x at the start: a row's first tile max is far above most later scores, and later
    tiles rise far above it, so the running max has to move many times (about one tile in
    five of these rows, by a CPU count of the rule) and the rescaled tiles include masked
    diagonal ones."""
    dtype, Sq, Skv = "bf16", 400, 1200
    q_off = Skv - Sq if causal else 0
    say(f"fwd running max D={D} causal={causal} P={P} start={start}")
    q, k, v = si.draw_qkv(77 + D, (1, 2, Sq, D), (1, 2, Skv, D), dtype)
    kf = si.bf16_bits_to_f32(k)
    kf = kf * (np.float32(1.0) + np.arange(Skv, dtype=np.float32) / np.float32(150.0))[:, None]
    kf[:, :, :3] *= np.float32(6.0)
    k = si.bf16_bits(kf)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    o, lse = ra.attn_fwd(qd, kd, vd, causal=causal, num_chunks=P, start_chunk=start,
                         q_offset=q_off)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.full_attention(si.as_f64(q, dtype), si.as_f64(k, dtype),
                                         si.as_f64(v, dtype), causal=causal, q_offset=q_off)
    check_o(to_np64(o), o_ref, dtype)
    check_lse(to_np64(lse), l_ref, dtype)


def test_fp32_partial_output_from_bf16():
    _run_case("bf16", 128, True, 1, 2, 2, 200, 400, 2, 1, 200, 0, seed=5, out_f32=True)


def test_explicit_scale():
    _run_case("bf16", 64, False, 1, 2, 2, 100, 100, seed=6, scale=0.3)


def test_empty_key_axis():
    say("fwd empty key axis")
    q = torch.randn(1, 2, 70, 128, device="cuda").bfloat16()
    k = torch.empty(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    o, lse = ra.attn_fwd(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_empty_query_axis_is_noop():
    q = torch.empty(1, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 10, 128, device="cuda").bfloat16()
    o, lse = ra.attn_fwd(q, k, k)
    assert o.shape == (1, 2, 0, 128)


def test_strided_bshd_layout():
    """q/k/v/o as [B, S, H, D] memory viewed as [B, H, S, D] (heads inside a token row)."""
    say("fwd BSHD strided views")
    dtype = "bf16"
    q, k, v = si.draw_qkv(11, (1, 300, 4, 128), (1, 300, 2, 128), dtype)
    qd, kd, vd = (to_dev(x, dtype).transpose(1, 2) for x in (q, k, v))
    out = torch.empty(1, 300, 4, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True, out=out)
    torch.cuda.synchronize()
    t = lambda x: si.as_f64(x, dtype).transpose(0, 2, 1, 3)
    o_ref, l_ref = oracle.full_attention(t(q), t(k), t(v), causal=True)
    check_o(to_np64(o), o_ref, dtype)
    check_lse(to_np64(lse), l_ref, dtype)


def test_deterministic():
    say("fwd determinism")
    q, k, v = (torch.randn(1, 4, 500, 128, device="cuda").bfloat16() for _ in range(3))
    a = ra.attn_fwd(q, k, v, causal=True, num_chunks=4, start_chunk=1)
    b = ra.attn_fwd(q, k, v, causal=True, num_chunks=4, start_chunk=1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_ring_tiny_f32_workload():
    """Tiny ring simulation: fp32, [1,2,256,64], 4 chunks from chunk 1, non-causal."""
    w = si.WORKLOADS["ring_tiny_f32"]
    say(f"workload {w.name}")
    q, k, v = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    o, lse = ra.attn_fwd(qd, kd, vd, causal=w.causal, num_chunks=w.num_chunks,
                         start_chunk=w.start_chunk)
    torch.cuda.synchronize()
    q64, k64, v64 = (si.as_f64(x, "f32") for x in (q, k, v))
    o_ring, l_ring = oracle.ring_attention(q64, k64, v64, num_chunks=w.num_chunks,
                                           start_chunk=w.start_chunk, causal=w.causal)
    check_o(to_np64(o), o_ring, "f32", "o vs naive chunk fold")
    check_lse(to_np64(lse), l_ring, "f32", "lse vs naive chunk fold")
    o_full, l_full = oracle.full_attention(q64, k64, v64)
    check_o(to_np64(o), o_full, "f32", "o vs full attention")
    check_lse(to_np64(lse), l_full, "f32", "lse vs full attention")


def _sampled_check(w, o_np, l_np, q64, k64, v64, what, per_head=6):
    B, H, S, _ = w.q_shape
    idx = sample_rows(B, H, S, per_head=per_head, seed=w.seed)
    o_ref, l_ref = oracle.attention_rows(q64, k64, v64, idx, causal=w.causal,
                                         q_offset=w.q_offset, kv_offset=w.kv_offset)
    check_o(gather_rows(o_np, idx).astype(np.float64), o_ref, w.dtype, f"{what} o (sampled)")
    check_lse(gather_lse(l_np, idx).astype(np.float64), l_ref, w.dtype, f"{what} lse (sampled)")
    assert np.isfinite(o_np).all() and np.isfinite(l_np).all()


def _whole_head_check(w, o_np, l_np, q64, k64, v64, h, what):
    """Every row of query head h against the oracle (its key/value head by the grouping)."""
    group = w.q_shape[1] // w.kv_shape[1]
    g = h // group
    o_ref, l_ref = oracle.full_attention(q64[:, h:h + 1], k64[:, g:g + 1], v64[:, g:g + 1],
                                         causal=w.causal, q_offset=w.q_offset,
                                         kv_offset=w.kv_offset)
    check_o(o_np[:, h:h + 1].astype(np.float64), o_ref, w.dtype, f"{what} o head {h} (all rows)")
    check_lse(l_np[:, h:h + 1].astype(np.float64), l_ref, w.dtype,
              f"{what} lse head {h} (all rows)")


# Full-size workloads.  Each runs once on the GPU, in the launch configuration bench.py
# times (module-scoped fixtures); every row of whole heads is then compared with the
# oracle, one head per test so that each test stays short, and sampled rows (tile
# edges, both ends, random rows) of every head.

@pytest.fixture(scope="module")
def llama8k():
    w = si.WORKLOADS["llama7b_causal_8k"]
    say(f"workload {w.name}")
    q, k, v = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ra.attn_fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    res = (w, o.float().cpu().numpy(), lse.cpu().numpy(),
           *(si.as_f64(x, "bf16") for x in (q, k, v)))
    del qd, kd, vd, o, lse
    return res


def test_llama_causal_8k_workload_sampled(llama8k):
    w, o_np, l_np, q64, k64, v64 = llama8k
    _sampled_check(w, o_np, l_np, q64, k64, v64, w.name)


@pytest.mark.parametrize("h", [0, 13, 31])
def test_llama_causal_8k_workload_whole_head(llama8k, h):
    w, o_np, l_np, q64, k64, v64 = llama8k
    _whole_head_check(w, o_np, l_np, q64, k64, v64, h, w.name)


@pytest.fixture(scope="module")
def ring32k():
    w = si.WORKLOADS["ring8_rank3_32k"]
    q, k, v = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    say(f"workload {w.name} fused")
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True, num_chunks=w.num_chunks,
                         start_chunk=w.start_chunk, q_offset=w.q_offset)
    torch.cuda.synchronize()
    say(f"workload {w.name} chunk-by-chunk + merge")
    assert ra.ring_visible_chunks(4096, 32768, num_chunks=8, start_chunk=3, causal=True,
                                  q_offset=w.q_offset) == [3, 0, 1, 2]
    o2, lse2 = ra.ring_attn_chunked(qd, kd, vd, causal=True, num_chunks=w.num_chunks,
                                    start_chunk=w.start_chunk, q_offset=w.q_offset)
    torch.cuda.synchronize()
    res = {"fused": (o.float().cpu().numpy(), lse.cpu().numpy()),
           "chunked": (o2.float().cpu().numpy(), lse2.cpu().numpy())}
    del qd, kd, vd, o, lse, o2, lse2
    return w, res, tuple(si.as_f64(x, "bf16") for x in (q, k, v))


@pytest.mark.parametrize("form", ["fused", "chunked"])
def test_ring8_rank3_32k_workload_sampled(ring32k, form):
    w, res, (q64, k64, v64) = ring32k
    _sampled_check(w, *res[form], q64, k64, v64, form)


@pytest.mark.parametrize("form", ["fused", "chunked"])
@pytest.mark.parametrize("h", [0, 18, 31])
def test_ring8_rank3_32k_workload_whole_head(ring32k, form, h):
    w, res, (q64, k64, v64) = ring32k
    _whole_head_check(w, *res[form], q64, k64, v64, h, form)


@pytest.fixture(scope="module")
def qwen32k():
    """Permute the sequence-sharded sources of rank 0 (bit-exact), then causal GQA
    attention over the whole 32K head shard."""
    w = si.WORKLOADS["qwen7b_ulysses4_rank0_32k"]
    say(f"workload {w.name}")
    qs, ks, vs = si.draw_ulysses_sources(w.seed)
    P, r = w.ulysses_P, w.ulysses_rank
    heads = []
    for src in (qs, ks, vs):
        d = ra.ulysses_permute(to_dev(src, "bf16"), P, r, 0)
        ref = oracle.seq_to_head(src, P, r)
        got = d.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), "permute not bit-exact"
        heads.append((d.unsqueeze(0), ref[None]))
    (qd, q_ref), (kd, k_ref), (vd, v_ref) = heads
    assert tuple(qd.shape) == w.q_shape and tuple(kd.shape) == w.kv_shape
    o = torch.full(qd.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ra.attn_fwd(qd, kd, vd, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    res = (w, o.float().cpu().numpy(), lse.cpu().numpy(),
           *(si.as_f64(x, "bf16") for x in (q_ref, k_ref, v_ref)))
    del qd, kd, vd, o, lse, heads
    return res


def test_qwen_ulysses_32k_workload_sampled(qwen32k):
    w, o_np, l_np, q64, k64, v64 = qwen32k
    _sampled_check(w, o_np, l_np, q64, k64, v64, w.name, per_head=12)


@pytest.mark.parametrize("h", range(7))
def test_qwen_ulysses_32k_workload_whole_head(qwen32k, h):
    """All 7 query heads of the headline, every row (each one query tile set of the
    work-counter launch)."""
    w, o_np, l_np, q64, k64, v64 = qwen32k
    _whole_head_check(w, o_np, l_np, q64, k64, v64, h, w.name)


def _counter(q):
    ra._sched_counter(q)
    return ra._SCHED[(q.device.index, torch.cuda.current_stream(q.device).cuda_stream)]


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 7, 1, 1000, 128), (3, 2, 1, 777, 64),
                                          (1, 28, 4, 700, 128)])
def test_work_counter_changes_order_not_results(B, Hq, Hkv, S, D):
    """With the work counter (B*Hq not a multiple of 8) workgroups take query tiles in
    start order; the outputs are bitwise those of the fixed order, also when the counter
    holds an arbitrary value (the order rotates), and every call leaves it as it was."""
    say(f"work counter B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}")
    q, k, v = si.draw_qkv(11, (B, Hq, S, D), (B, Hkv, S, D), "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o0, l0 = ra.attn_fwd(qd, kd, vd, causal=True, sched=False)
    ctr = _counter(qd)
    for start in (0, 0, 12345, 2**40 + 3):
        ctr.fill_(start)
        o1, l1 = ra.attn_fwd(qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), start
        assert torch.equal(l1.view(torch.int32), l0.view(torch.int32)), start
        assert int(ctr.item()) == start
    ctr.zero_()
    # packed documents use the same kernel and counter
    cu = torch.tensor([0, S // 3, S // 3 + 5, S], dtype=torch.int32, device="cuda")
    o2, l2 = ra.attn_fwd_varlen(qd, kd, vd, cu, causal=True, sched=False)
    o3, l3 = ra.attn_fwd_varlen(qd, kd, vd, cu, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l2.view(torch.int32))
    assert int(ctr.item()) == 0
