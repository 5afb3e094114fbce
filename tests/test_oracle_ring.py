"""Pins of the oracle's chunked (ring) path and of both LSE merges.

The pages claim the ring result is mathematically the full-attention result; the
checks below hold the naive chunk-by-chunk fold and the n-way merge to that, to
order invariance, and to algebraic identities of the merge.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.attention import ring_order


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(seed, B=1, Hq=4, Hkv=2, Sq=24, Skv=32, D=8):
    return (_rand((B, Hq, Sq, D), seed), _rand((B, Hkv, Skv, D), seed + 1),
            _rand((B, Hkv, Skv, D), seed + 2))


def test_ring_order_increasing():
    assert ring_order(8, 3) == [3, 4, 5, 6, 7, 0, 1, 2]
    assert ring_order(4, 1) == [1, 2, 3, 0]


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("causal,q_offset", [(False, 0), (True, 8), (True, 0)])
def test_chunked_equals_unchunked(P, causal, q_offset):
    q, k, v = _qkv(100 + P)
    o, lse = oracle.full_attention(q, k, v, causal=causal, q_offset=q_offset)
    for start in range(P):
        oc, lc = oracle.ring_attention(q, k, v, num_chunks=P, start_chunk=start, causal=causal,
                                       q_offset=q_offset)
        assert np.array_equal(np.isinf(lc), np.isinf(lse))
        fin = np.isfinite(lse)
        assert np.max(np.abs(lc[fin] - lse[fin])) <= 1e-12
        assert np.max(np.abs(oc - o)) <= 1e-12


def test_noncausal_order_invariance():
    q, k, v = _qkv(200, Skv=64)
    res = [oracle.ring_attention(q, k, v, num_chunks=8, start_chunk=s) for s in range(8)]
    for oc, lc in res[1:]:
        assert np.max(np.abs(oc - res[0][0])) <= 1e-12
        assert np.max(np.abs(lc - res[0][1])) <= 1e-12


def test_ring_rank_share_equals_full_rows():
    """One rank's share of a causal ring: its Q rows at a global offset, all chunks."""
    S, P, rank = 64, 8, 3
    L = S // P
    qfull, k, v = _rand((1, 2, S, 8), 300), _rand((1, 2, S, 8), 301), _rand((1, 2, S, 8), 302)
    o, lse = oracle.full_attention(qfull, k, v, causal=True)
    q = qfull[:, :, rank * L:(rank + 1) * L]
    oc, lc = oracle.ring_attention(q, k, v, num_chunks=P, start_chunk=rank, causal=True,
                                   q_offset=rank * L)
    assert np.max(np.abs(oc - o[:, :, rank * L:(rank + 1) * L])) <= 1e-12
    assert np.max(np.abs(lc - lse[:, :, rank * L:(rank + 1) * L])) <= 1e-12
    # chunks after the rank's own are entirely in the future: empty partials
    for c in range(rank + 1, P):
        pc, pl = oracle.chunk_partial(q, k, v, c, P, causal=True, q_offset=rank * L)
        assert np.all(pc == 0.0) and np.all(np.isneginf(pl))


def _parts(seed, n, shape=(1, 2, 5, 4)):
    rng = np.random.default_rng(seed)
    os_ = [rng.standard_normal(shape) for _ in range(n)]
    ls = [rng.standard_normal(shape[:-1]) * 3 for _ in range(n)]
    return os_, ls


def test_merge_with_empty_partial_is_identity():
    (o,), (l,) = _parts(400, 1)
    empty = (np.zeros_like(o), np.full_like(l, -np.inf))
    for got in (oracle.fold_pair((o, l), empty), oracle.fold_pair(empty, (o, l)),
                oracle.lse_merge([o, empty[0]], [l, empty[1]])):
        assert np.max(np.abs(got[0] - o)) <= 1e-15
        assert np.max(np.abs(got[1] - l)) <= 1e-15


def test_merge_self_adds_ln2():
    (o,), (l,) = _parts(401, 1)
    for got in (oracle.fold_pair((o, l), (o, l)), oracle.lse_merge([o, o], [l, l])):
        assert np.max(np.abs(got[0] - o)) <= 1e-15
        assert np.max(np.abs(got[1] - (l + math.log(2)))) <= 1e-15


def test_merge_all_empty():
    o = np.full((1, 1, 3, 4), 0.0)
    l = np.full((1, 1, 3), -np.inf)
    for got in (oracle.fold_pair((o, l), (o, l)), oracle.lse_merge([o, o, o], [l, l, l])):
        assert np.all(got[0] == 0.0) and np.all(np.isneginf(got[1]))


def test_merge_commutative_and_nway_equals_pairwise():
    os_, ls = _parts(402, 5)
    a = oracle.fold_pair((os_[0], ls[0]), (os_[1], ls[1]))
    b = oracle.fold_pair((os_[1], ls[1]), (os_[0], ls[0]))
    assert np.max(np.abs(a[0] - b[0])) <= 1e-14 and np.max(np.abs(a[1] - b[1])) <= 1e-14
    acc = (np.zeros_like(os_[0]), np.full_like(ls[0], -np.inf))
    for o, l in zip(os_, ls):
        acc = oracle.fold_pair(acc, (o, l))
    n = oracle.lse_merge(os_, ls)
    assert np.max(np.abs(acc[0] - n[0])) <= 1e-13
    assert np.max(np.abs(acc[1] - n[1])) <= 1e-13
    assert np.max(np.abs(n[1] - scipy.special.logsumexp(np.stack(ls), axis=0))) <= 1e-13


def test_merge_of_chunk_partials_matches_page1_statistics():
    """Global max of local maxima and Z from raw scores, computed without lse."""
    q, k, v = _qkv(500, Hq=2, Hkv=2, Sq=6, Skv=24)
    P = 4
    parts = [oracle.chunk_partial(q, k, v, c, P) for c in range(P)]
    o, lse = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(8)
    L = 24 // P
    m_i = np.stack([s[..., c * L:(c + 1) * L].max(-1) for c in range(P)])
    m_g = m_i.max(0)
    Z = np.exp(s - m_g[..., None]).sum(-1)
    assert np.max(np.abs(lse - (m_g + np.log(Z)))) <= 1e-13
    w = np.exp(s - m_g[..., None]) / Z[..., None]
    assert np.max(np.abs(o - np.einsum("bhij,bhjd->bhid", w, v))) <= 1e-13
