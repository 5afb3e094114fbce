"""GPU parity of ra_attn_bwd (dq, dk, dv) against the oracle's fp64 gradients.

The GPU forward supplies o and lse to the GPU backward (the product path); the oracle
recomputes everything from q, k, v, dO on its own.

Tolerance for bf16 gradients (none is stated for gradients, so it is derived from the
arithmetic): each output is rounded to bf16 once (<= 2^-9 |g|) and P and dS are rounded
to bf16 before their matrix products (aggregate <= 2^-9 |g| more), so element-wise
|err| <= 2e-2 + 2^-8 |ref|; besides, mean abs err <= 2e-3 and L2 error <= 1e-2 of the
reference's L2 norm, or the mean bound's floor (2e-3 RMS) where that is larger: for a gradient that vanishes
exactly: a row that sees a single key has P = 1 and dP = D, so its dS is 0.  With
grouped heads dK and dV sum over the group and reach |g| of several units, where the
output rounding alone exceeds a flat 2e-2.
"""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import check_grad, require_gpu, say, to_dev, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(B, Hq, Hkv, Sq, Skv, D, causal, P=1, start=0, q_off=0, kv_off=0, seed=0):
    say(f"bwd D={D} causal={causal} B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Skv={Skv} P={P} "
        f"start={start} q_off={q_off} kv_off={kv_off}")
    q, k, v, do = si.draw_qkv(seed, (B, Hq, Sq, D), (B, Hkv, Skv, D), "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    kw = dict(causal=causal, num_chunks=P, start_chunk=start, q_offset=q_off, kv_offset=kv_off)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ra.attn_bwd(qd, kd, vd, o, dod, lse, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(*(si.as_f64(x, "bf16") for x in (q, k, v, do)), causal=causal,
                               q_offset=q_off, kv_offset=kv_off)
    for got, r, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(to_np64(got), r, name)


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off
    (1, 2, 2, 300, 300, 128, True, 1, 0, 0, 0),
    (2, 4, 2, 200, 300, 64, False, 3, 1, 0, 0),
    (1, 4, 1, 256, 256, 128, True, 4, 1, 0, 0),
    (1, 2, 2, 130, 390, 128, True, 3, 2, 260, 0),
    (1, 2, 2, 200, 200, 128, True, 1, 0, 0, 100),
    (1, 7, 1, 333, 333, 128, True, 1, 0, 0, 0),
    (1, 2, 2, 1, 1, 64, True, 1, 0, 0, 0),
    (1, 3, 3, 700, 700, 64, True, 1, 0, 0, 0),     # 64-dim heads: several tiles, ragged tail
    (1, 6, 2, 523, 523, 64, True, 1, 0, 0, 0),     # 64-dim grouped heads (partials)
    (1, 2, 2, 300, 900, 64, True, 3, 2, 600, 0),   # 64-dim causal ring share
    (2, 4, 1, 300, 300, 128, True, 1, 0, 0, 0),    # two batches of grouped heads (partials)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_small_bwd(case):
    B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off = case
    _run(B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off,
         seed=sum(map(ord, str(case))) % 991)


@pytest.mark.parametrize("Hkv", [4, 1])
def test_bwd_deterministic(Hkv):
    """Bitwise the same gradients on repeated calls: one key/value head per query head,
    and grouped heads (per-query-head partials summed in head order; the workspace is
    filled with garbage first, so nothing may depend on its old contents)."""
    say(f"bwd determinism Hkv={Hkv}")
    q, do = (torch.randn(1, 4, 400, 128, device="cuda").bfloat16() for _ in range(2))
    k, v = (torch.randn(1, Hkv, 400, 128, device="cuda").bfloat16() for _ in range(2))
    o, lse = ra.attn_fwd(q, k, v, causal=True)
    need = ra.attn_bwd_workspace_size(q, k, causal=True)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    a = ra.attn_bwd(q, k, v, o, do, lse, causal=True, workspace=ws)
    b = ra.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_qwen_gqa_causal_bwd_8k_whole_kv_head():
    """Grouped heads at full width (Qwen2.5-7B heads, 28 query over 4 key/value heads,
    8K causal): the workspace path (per-query-head dK/dV partials and their group sum).
    Every element of one key/value head's dK, dV and of its 7 query heads' dQ is checked."""
    q_shape, kv_shape = (1, 28, 8192, 128), (1, 4, 8192, 128)
    say(f"gqa bwd 8k q {q_shape} kv {kv_shape}")
    q, k, v, do = si.draw_qkv(1011, q_shape, kv_shape, "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True)
    assert ra.attn_bwd_workspace_size(qd, kd, causal=True) > ra.attn_bwd_workspace_size(
        qd, qd, causal=True)  # the partials are in use
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    g = 2
    q64, k64, v64, do64 = (si.as_f64(x, "bf16") for x in (q, k, v, do))
    ref = oracle.attention_bwd_heads(q64, k64, v64, do64, [(0, g)], causal=True, row_block=512)
    rq, rk, rv = ref[(0, g)]
    dq_n, dk_n, dv_n = (to_np64(t) for t in (dq, dk, dv))
    check_grad(dq_n[0, 7 * g:7 * g + 7], rq, "dq heads 14-20")
    check_grad(dk_n[0, g], rk, f"dk head {g}")
    check_grad(dv_n[0, g], rv, f"dv head {g}")


def test_llama_causal_bwd_16k_workload_sampled_heads():
    """Full-size backward; every element of three whole heads checked against the oracle."""
    w = si.WORKLOADS["llama7b_causal_bwd_16k"]
    say(f"workload {w.name}")
    q, k, v, do = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    heads = [(0, 0), (0, 17), (0, 31)]
    q64, k64, v64, do64 = (si.as_f64(x, "bf16") for x in (q, k, v, do))
    ref = oracle.attention_bwd_heads(q64, k64, v64, do64, heads, causal=True, row_block=512)
    dq_n, dk_n, dv_n = (to_np64(t) for t in (dq, dk, dv))
    for (b, g), (rq, rk, rv) in ref.items():
        check_grad(dq_n[b, g:g + 1], rq, f"dq head {g}")
        check_grad(dk_n[b, g], rk, f"dk head {g}")
        check_grad(dv_n[b, g], rv, f"dv head {g}")


def test_d64_causal_bwd_16k_whole_head():
    """64-dim heads at full size (32 heads, 16K causal: the dK/dV kernel's two-waves-per-
    SIMD form): every element of one head's dq, dk and dv against the oracle."""
    q_shape = (1, 32, 16384, 64)
    say(f"d64 bwd 16k {q_shape}")
    q, k, v, do = si.draw_qkv(1012, q_shape, q_shape, "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    g = 21
    q64, k64, v64, do64 = (si.as_f64(x, "bf16") for x in (q, k, v, do))
    rq, rk, rv = oracle.attention_bwd_heads(q64, k64, v64, do64, [(0, g)], causal=True,
                                            row_block=512)[(0, g)]
    dq_n, dk_n, dv_n = (to_np64(t) for t in (dq, dk, dv))
    check_grad(dq_n[0, g:g + 1], rq, f"dq head {g}")
    check_grad(dk_n[0, g], rk, f"dk head {g}")
    check_grad(dv_n[0, g], rv, f"dv head {g}")
