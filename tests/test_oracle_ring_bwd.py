"""Pins of the oracle's chunk-by-chunk ring backward (one device's query block).

Pinned against finite differences of that device's loss, against the whole-sequence
gradient (the sum over every device's block), and against the chunk skip rule.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _setup(B, Hq, Hkv, Sq, Skv, D, seed):
    return (_rand((B, Hq, Sq, D), seed), _rand((B, Hkv, Skv, D), seed + 1),
            _rand((B, Hkv, Skv, D), seed + 2), _rand((B, Hq, Sq, D), seed + 3))


@pytest.mark.parametrize("causal,P,start,q_off", [(True, 3, 1, 4), (False, 6, 2, 0),
                                                   (True, 2, 0, 0)])
def test_finite_differences_of_the_block_loss(causal, P, start, q_off):
    """d/dx of L = sum(dO * o) for one device's block, o from the full definition."""
    q, k, v, do = _setup(1, 4, 2, 3, 6, 3, 11)
    kw = dict(causal=causal, scale=0.8, q_offset=q_off)
    dq, dk, dv = oracle.ring_attention_bwd(q, k, v, do, num_chunks=P, start_chunk=start, **kw)

    def loss(q_, k_, v_):
        o, _ = oracle.full_attention(q_, k_, v_, **kw)
        return float((do * o).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P", [1, 2, 4])
def test_sum_over_devices_is_the_whole_gradient(causal, P):
    """Device r holds queries [r L, (r+1) L) and starts its walk at chunk r; the sum of
    every device's dK/dV, and the concatenation of their dQ, is the gradient of
    attention over the whole sequence."""
    L = 5
    S = P * L
    q, k, v, do = _setup(2, 4, 2, S, S, 8, 21)
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd(q, k, v, do, causal=causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(P):
        rows = slice(r * L, (r + 1) * L)
        gq, gk, gv = oracle.ring_attention_bwd(q[:, :, rows], k, v, do[:, :, rows], num_chunks=P,
                                               start_chunk=r, causal=causal, q_offset=r * L)
        dq[:, :, rows] = gq
        dk += gk
        dv += gv
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_block_equals_the_unchunked_block_gradient():
    """Chunking the keys does not change one block's gradients (any start)."""
    q, k, v, do = _setup(1, 6, 2, 7, 24, 5, 31)
    ref = oracle.attention_bwd(q, k, v, do, causal=True, q_offset=10, kv_offset=0)
    for P in (1, 3, 8):
        for start in range(P):
            got = oracle.ring_attention_bwd(q, k, v, do, num_chunks=P, start_chunk=start,
                                            causal=True, q_offset=10)
            for g, r in zip(got, ref):
                np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_future_chunks_get_exact_zeros():
    """Causal: chunks whose first key follows the block's last query add nothing."""
    q, k, v, do = _setup(1, 2, 1, 4, 16, 4, 41)
    dq, dk, dv = oracle.ring_attention_bwd(q, k, v, do, num_chunks=4, start_chunk=1,
                                           causal=True, q_offset=4)
    assert not dk[:, :, 8:].any() and not dv[:, :, 8:].any()
    assert np.abs(dk[:, :, :8]).min() > 0 and np.abs(dv[:, :, :8]).min() > 0
    assert np.isfinite(dq).all()


def test_rows_with_no_visible_key_have_zero_gradient():
    """kv_offset past every query: each row is empty (o = 0, lse = -inf), all zeros."""
    q, k, v, do = _setup(1, 2, 2, 3, 6, 4, 51)
    dq, dk, dv = oracle.ring_attention_bwd(q, k, v, do, num_chunks=2, causal=True,
                                           kv_offset=3)
    assert not dq.any() and not dk.any() and not dv.any()
