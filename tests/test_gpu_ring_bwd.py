"""GPU parity of the chunk-by-chunk ring backward (ra_attn_bwd_accum) against the oracle.

Each case plays one device of a ring: its query block of L rows at global position r L,
the key/value sequence as P chunks of L in one buffer, (o, lse) from the GPU's ring
forward, then one accumulating call per visible chunk in ring order into fp32
accumulators.  The oracle walks the same chunks in fp64.  Tolerance: the bf16 gradient
bound of test_gpu_bwd.py (element-wise 2e-2 + 2^-8 |ref|, mean 2e-3, L2 1e-2 of the
reference plus a 2e-3 RMS floor);
the fp32 accumulators add no output rounding, so the bound holds with margin.
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


def _draw(B, Hq, Hkv, Sq, Skv, D, seed):
    q, k, v, do = si.draw_qkv(seed, (B, Hq, Sq, D), (B, Hkv, Skv, D), "bf16", with_dout=True)
    return (q, k, v, do), tuple(to_dev(x, "bf16") for x in (q, k, v, do)), \
        tuple(si.as_f64(x, "bf16") for x in (q, k, v, do))


CASES = [
    # B, Hq, Hkv, L, P, r, D, causal
    (1, 4, 2, 96, 4, 2, 128, True),
    (2, 2, 2, 100, 3, 1, 64, False),
    (1, 7, 1, 130, 4, 3, 128, True),
    (1, 2, 2, 64, 2, 0, 128, True),
    (1, 4, 4, 200, 2, 1, 64, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_device_step(case):
    B, Hq, Hkv, L, P, r, D, causal = case
    say(f"ring bwd step B={B} Hq={Hq} Hkv={Hkv} L={L} P={P} r={r} D={D} causal={causal}")
    _, (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, Hkv, L, P * L, D,
                                                sum(map(ord, str(case))) % 997)
    kw = dict(num_chunks=P, start_chunk=r, causal=causal, q_offset=r * L)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.ring_attention_bwd(q, k, v, do, **kw)
    for got, rr, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(to_np64(got), rr, name)
    if causal:  # chunks after the block are skipped: their accumulators stay exactly 0
        assert not dk[:, :, (r + 1) * L:].any() and not dv[:, :, (r + 1) * L:].any()


def test_whole_ring_on_one_gpu():
    """Every device's block in turn, adding into shared dK/dV accumulators as the ring
    would: the result is the whole-sequence gradient."""
    B, Hq, Hkv, L, P, D = 1, 4, 2, 80, 3, 128
    say(f"whole ring P={P} L={L}")
    _, (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, Hkv, P * L, P * L, D, 77)
    dq = torch.zeros(qd.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(kd.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    for r in range(P):
        rows = slice(r * L, (r + 1) * L)
        kw = dict(num_chunks=P, start_chunk=r, causal=True, q_offset=r * L)
        qr, dor = qd[:, :, rows], dod[:, :, rows]
        o, lse = ra.attn_fwd(qr, kd, vd, **kw)
        ra.ring_attn_bwd_chunked(qr, kd, vd, o, dor, lse, dq_acc=dq[:, :, rows], dk_acc=dk,
                                 dv_acc=dv, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, do, causal=True)
    for got, rr, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(to_np64(got), rr, name)


def test_accumulates_onto_existing_values():
    """acc_in + step == the step from zero added to acc_in, and a causal chunk wholly
    after the block leaves the accumulators untouched.  dv is one fp32 add (bitwise);
    dq and dk may fuse their scale into that add (one rounding apart)."""
    B, Hq, Hkv, L, D = 1, 2, 1, 96, 128
    say("ring bwd accumulate semantics")
    _, (qd, kd, vd, dod), _ = _draw(B, Hq, Hkv, L, 2 * L, D, 5)
    kw = dict(num_chunks=2, start_chunk=0, causal=True, q_offset=L)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    k0, v0 = kd[:, :, :L], vd[:, :, :L]
    zero = lambda t: torch.zeros(t.shape, dtype=torch.float32, device="cuda")
    base = ra.attn_bwd_accum(qd, k0, v0, o, dod, lse, zero(qd), zero(k0), zero(v0), causal=True,
                             q_offset=L, kv_offset=0)
    g = torch.Generator(device="cuda").manual_seed(3)
    start = [torch.randn(t.shape, device="cuda", generator=g) for t in (qd, k0, v0)]
    accs = [s.clone() for s in start]
    ra.attn_bwd_accum(qd, k0, v0, o, dod, lse, *accs, causal=True, q_offset=L, kv_offset=0)
    # a chunk at keys 2L.. follows every query (last query L + L - 1): nothing is added
    ra.attn_bwd_accum(qd, k0, v0, o, dod, lse, *accs, causal=True, q_offset=L, kv_offset=2 * L)
    torch.cuda.synchronize()
    for a, s, b, name in zip(accs, start, base, ("dq", "dk", "dv")):
        if name == "dv":
            assert torch.equal(a, s + b)
        else:
            torch.testing.assert_close(a, s + b, rtol=1e-6, atol=1e-6)
        assert not torch.equal(a, s)  # something was added


def test_chunked_matches_fused_ring_backward():
    """The per-chunk steps and the fused ra_attn_bwd over the same ring agree (both
    against the oracle; the fused one rounds its outputs to bf16)."""
    B, Hq, Hkv, L, P, r, D = 1, 4, 1, 128, 4, 1, 128
    say("chunked vs fused ring backward")
    _, (qd, kd, vd, dod), (q, k, v, do) = _draw(B, Hq, Hkv, L, P * L, D, 9)
    kw = dict(num_chunks=P, start_chunk=r, causal=True, q_offset=r * L)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    fused = ra.attn_bwd(qd, kd, vd, o, dod, lse, **kw)
    chunked = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    again = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.ring_attention_bwd(q, k, v, do, **kw)
    for f, c, a, rr, name in zip(fused, chunked, again, ref, ("dq", "dk", "dv")):
        assert torch.equal(c, a), f"{name}: chunked backward not deterministic"
        check_grad(to_np64(f), rr, f"fused {name}")
        check_grad(to_np64(c), rr, f"chunked {name}")


def test_ring8_rank3_bwd_32k_workload_sampled_heads():
    """Full-size rank-3-of-8 ring backward (q 4096 rows at 12288, k/v 8 chunks of 4096):
    every element of three key/value heads checked against the oracle."""
    w = si.WORKLOADS["ring8_rank3_bwd_32k"]
    say(f"workload {w.name}")
    q, k, v, do = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    kw = dict(num_chunks=w.num_chunks, start_chunk=w.start_chunk, causal=True,
              q_offset=w.q_offset)
    o, lse = ra.attn_fwd(qd, kd, vd, **kw)
    dq, dk, dv = ra.ring_attn_bwd_chunked(qd, kd, vd, o, dod, lse, **kw)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    L = w.kv_shape[2] // w.num_chunks
    last = w.q_offset + w.q_shape[2]  # keys at or after this position are never visible
    assert not dk[:, :, last:].any() and not dv[:, :, last:].any()
    heads = [(0, 0), (0, 13), (0, 31)]
    q64, k64, v64, do64 = (si.as_f64(x, "bf16") for x in (q, k, v, do))
    ref = oracle.attention_bwd_heads(q64, k64[:, :, :last], v64[:, :, :last], do64, heads,
                                     causal=True, q_offset=w.q_offset, row_block=512)
    dq_n, dk_n, dv_n = (to_np64(t) for t in (dq, dk, dv))
    assert last == (w.start_chunk + 1) * L
    for (b, g), (rq, rk, rv) in ref.items():
        check_grad(dq_n[b, g:g + 1], rq, f"dq head {g}")
        check_grad(dk_n[b, g, :last], rk, f"dk head {g}")
        check_grad(dv_n[b, g, :last], rv, f"dv head {g}")
