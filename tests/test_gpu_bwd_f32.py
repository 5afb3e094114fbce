"""GPU parity of the fp32 backward (ra_attn_bwd, ra_attn_bwd_accum and ra_attn_bwd_noalloc
with fp32 inputs) against the oracle's fp64 gradients.

The GPU fp32 forward supplies o and lse; the oracle recomputes everything from q, k, v,
dO.  Tolerance (none is stated for fp32 gradients; derived from the arithmetic, as the
forward's fp32 bound of 1e-5 max abs): inputs are exact, every product and sum is an
fp32 operation, so scores carry a relative error of a few 2^-24 per term over D terms,
exp2 of an argument up to ~|s| c adds ~|s| c 2^-24, and dS = P (dP - D) and the
gradient sums over up to a few hundred rows inherit that: element-wise
|err| <= 1e-5 + 2^-16 |ref| (the forward's absolute bound, plus a relative term for
the group-summed dK, dV that reach several units), and L2 error <= 1e-5 ||ref|| (or a
1e-6 RMS floor where the reference vanishes).
"""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import require_gpu, say, to_dev, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check_grad_f32(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = np.abs(got - ref)
    mx = float(err.max(initial=0.0))
    l2 = float(np.linalg.norm(got - ref))
    nref = float(np.linalg.norm(ref))
    print(f"[parity] {what}: max|err|={mx:.3e} relL2={l2 / max(nref, 1e-30):.3e} "
          f"max|ref|={float(np.abs(ref).max(initial=0.0)):.3e}", flush=True)
    excess = float((err - (1e-5 + 2.0 ** -16 * np.abs(ref))).max(initial=-1.0))
    assert excess <= 0.0, f"{what}: element error over 1e-5 + 2^-16|ref| by {excess}"
    # relative L2, with a 1e-6 RMS floor for gradients that vanish (dS of a row that sees
    # a single key is 0 up to the fp32 rounding of P = 1)
    assert l2 <= max(1e-5 * nref, 1e-6 * np.sqrt(err.size)), f"{what}: L2 {l2}"


def _draw(B, Hq, Hkv, Sq, Skv, D, seed):
    q, k, v, do = si.draw_qkv(seed, (B, Hq, Sq, D), (B, Hkv, Skv, D), "f32", with_dout=True)
    return tuple(to_dev(x, "f32") for x in (q, k, v, do)), \
        tuple(si.as_f64(x, "f32") for x in (q, k, v, do))


def test_ring_tiny_f32_workload_backward():
    """The tiny ring simulation's shape (fp32 [1, 2, 256, 64], 4 chunks from chunk 1,
    non-causal): the fused backward against the full-attention gradient and against the
    oracle's chunk-by-chunk ring backward, and the per-chunk accumulating steps."""
    w = si.WORKLOADS["ring_tiny_f32"]
    say(f"bwd f32 workload {w.name}")
    B, Hq, Sq, D = w.q_shape
    (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, w.kv_shape[1], Sq, w.kv_shape[2], D,
                                             w.seed)
    kw = dict(causal=w.causal, num_chunks=w.num_chunks, start_chunk=w.start_chunk)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = ra.attn_bwd(qd, kd, vd, o, dod, lse, **kw)
    acc = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    full = oracle.attention_bwd(q, k, v, do, causal=w.causal)
    ring = oracle.ring_attention_bwd(q, k, v, do, **kw)
    for got, r_full, r_ring, name in zip((dq, dk, dv), full, ring, ("dq", "dk", "dv")):
        check_grad_f32(to_np64(got), r_full, f"{name} vs full attention")
        check_grad_f32(to_np64(got), r_ring, f"{name} vs naive ring")
    for got, r_ring, name in zip(acc, ring, ("dq", "dk", "dv")):
        check_grad_f32(to_np64(got), r_ring, f"{name} chunk by chunk")


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off
    (1, 2, 2, 300, 300, 128, True, 1, 0, 0, 0),
    (2, 4, 2, 200, 300, 64, False, 3, 1, 0, 0),
    (1, 4, 1, 256, 256, 128, True, 4, 1, 0, 0),
    (1, 2, 2, 130, 390, 128, True, 3, 2, 260, 0),
    (1, 2, 2, 200, 200, 64, True, 1, 0, 0, 100),     # rows with no visible key
    (1, 7, 1, 333, 333, 128, True, 1, 0, 0, 0),      # GQA 7:1
    (1, 2, 2, 1, 1, 64, True, 1, 0, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_small_bwd_f32(case):
    B, Hq, Hkv, Sq, Skv, D, causal, P, start, q_off, kv_off = case
    say(f"bwd f32 {case}")
    (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, Hkv, Sq, Skv, D,
                                             sum(map(ord, str(case))) % 983)
    kw = dict(causal=causal, num_chunks=P, start_chunk=start, q_offset=q_off, kv_offset=kv_off)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    outs = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
    ra.attn_bwd(qd, kd, vd, o, dod, lse, dq=outs[0], dk=outs[1], dv=outs[2], **kw)
    na = ra.attn_bwd_noalloc(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, do, causal=causal, q_offset=q_off, kv_offset=kv_off)
    for got, r, other, name in zip(outs, ref, na, ("dq", "dk", "dv")):
        check_grad_f32(to_np64(got), r, name)
        assert torch.equal(got, other), f"{name}: noalloc differs"


def test_accum_steps_f32_ring_share():
    """One device of a 4-way causal ring (fp32): one accumulating step per visible chunk
    into fp32 accumulators, against the oracle's ring backward."""
    B, Hq, Hkv, L, P, r, D = 1, 4, 2, 96, 4, 2, 128
    say("bwd f32 ring steps")
    (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, Hkv, L, P * L, D, 321)
    kw = dict(num_chunks=P, start_chunk=r, causal=True, q_offset=r * L)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.ring_attention_bwd(q, k, v, do, **kw)
    for got, rr, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad_f32(to_np64(got), rr, name)
    assert not dk[:, :, (r + 1) * L:].any() and not dv[:, :, (r + 1) * L:].any()


def test_bwd_f32_deterministic():
    say("bwd f32 determinism")
    q, k, v, do = (torch.randn(1, 4, 300, 128, device="cuda") for _ in range(4))
    o, lse = ra.attn_fwd(q, k, v, causal=True)
    a = ra.attn_bwd(q, k, v, o, do, lse, causal=True)
    b = ra.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
