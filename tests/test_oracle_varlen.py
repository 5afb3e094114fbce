"""Pins of the oracle's packed-document attention against things other than itself.

A query sees only the keys of its own document (at or before it when causal).  The
brute force below decides visibility token by token from the document index of each
position (not by slicing), so an off-by-one in the document bounds, a mask that leaks
across a boundary, or positions counted globally instead of per document fails it.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _doc_of(cu, t):
    for d in range(len(cu) - 1):
        if cu[d] <= t < cu[d + 1]:
            return d
    return None


def _brute(q, k, v, cu, causal, scale):
    """Pure-Python loops, math.exp / math.fsum only."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    o = np.zeros((B, Hq, T, D))
    lse = np.full((B, Hq, T), -math.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(T):
                di = _doc_of(cu, i)
                vis = [j for j in range(T) if di is not None and _doc_of(cu, j) == di
                       and (not causal or j <= i)]
                if not vis:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, d]) * float(k[b, g, j, d])
                                          for d in range(D)) for j in vis}
                m = max(s.values())
                l = m + math.log(math.fsum(math.exp(s[j] - m) for j in vis))
                lse[b, h, i] = l
                for d in range(D):
                    o[b, h, i, d] = math.fsum(math.exp(s[j] - l) * float(v[b, g, j, d])
                                              for j in vis)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cu", [[0, 3, 3, 7, 8, 12], [0, 1, 2, 12], [0, 12], [0, 5, 9]])
def test_brute_force_tiny(causal, cu):
    # cu [0, 3, 3, ...]: an empty document; [0, 5, 9]: tokens 9..11 in no document
    q, k, v = _rand((1, 4, 12, 5), 21), _rand((1, 2, 12, 5), 22), _rand((1, 2, 12, 5), 23)
    o, lse = oracle.varlen_attention(q, k, v, cu, causal=causal, scale=0.41)
    bo, bl = _brute(q, k, v, cu, causal, 0.41)
    assert np.array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    assert np.max(np.abs(lse[fin] - bl[fin])) <= 1e-13
    assert np.max(np.abs(o - bo)) <= 1e-13


def test_one_document_is_full_attention():
    q, k, v = _rand((2, 2, 40, 8), 31), _rand((2, 1, 40, 8), 32), _rand((2, 1, 40, 8), 33)
    for causal in (False, True):
        o, lse = oracle.varlen_attention(q, k, v, [0, 40], causal=causal)
        fo, fl = oracle.full_attention(q, k, v, causal=causal)
        assert np.array_equal(o, fo) and np.array_equal(lse, fl)


def test_other_documents_do_not_leak():
    """Changing k, v of every other document leaves a document's rows bit-identical."""
    cu = [0, 17, 30, 64]
    q, k, v = _rand((1, 2, 64, 8), 41), _rand((1, 2, 64, 8), 42), _rand((1, 2, 64, 8), 43)
    o, lse = oracle.varlen_attention(q, k, v, cu, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :17] += 5.0
    k2[:, :, 30:] -= 3.0
    v2[:, :, :17] *= -2.0
    v2[:, :, 30:] += 1.0
    o2, lse2 = oracle.varlen_attention(q, k2, v2, cu, causal=True)
    assert np.array_equal(o[:, :, 17:30], o2[:, :, 17:30])
    assert np.array_equal(lse[:, :, 17:30], lse2[:, :, 17:30])
    assert not np.array_equal(o[:, :, :17], o2[:, :, :17])


def test_first_token_of_each_document():
    """Causal: a document's first token sees only itself: o = v, lse = its own score."""
    cu = [0, 6, 11, 20]
    q, k, v = _rand((1, 1, 20, 4), 51), _rand((1, 1, 20, 4), 52), _rand((1, 1, 20, 4), 53)
    o, lse = oracle.varlen_attention(q, k, v, cu, causal=True, scale=0.5)
    for a in cu[:-1]:
        assert np.allclose(o[0, 0, a], v[0, 0, a], atol=1e-15, rtol=0)
        assert abs(lse[0, 0, a] - 0.5 * float(q[0, 0, a] @ k[0, 0, a])) <= 1e-14


def test_bad_offsets_rejected():
    q = _rand((1, 1, 8, 4), 61)
    for cu in ([1, 8], [0, 5, 3], [0, 9], []):
        with pytest.raises(ValueError):
            oracle.varlen_attention(q, q, q, cu)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Gradients of L = sum(dO * o) against central differences of the packed forward
    (itself pinned by the brute force above); cu has an empty document and tokens past
    the last one (their gradients must be 0)."""
    cu = [0, 3, 3, 7, 8]
    T = 10
    q, k, v = _rand((1, 2, T, 3), 71), _rand((1, 1, T, 3), 72), _rand((1, 1, T, 3), 73)
    do = _rand((1, 2, T, 3), 74)
    dq, dk, dv = oracle.varlen_attention_bwd(q, k, v, do, cu, causal=causal, scale=0.6)

    def loss(qq, kk, vv):
        o, _ = oracle.varlen_attention(qq, kk, vv, cu, causal=causal, scale=0.6)
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
        assert np.all(g[:, :, 8:] == 0.0), name  # tokens in no document


def test_backward_one_document_is_attention_bwd():
    q, k, v, do = (_rand((1, 2, 30, 4), s) for s in (81, 82, 83, 84))
    a = oracle.varlen_attention_bwd(q, k, v, do, [0, 30], causal=True)
    b = oracle.attention_bwd(q, k, v, do, causal=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
