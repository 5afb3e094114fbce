"""Pins of the oracle's gradients: finite differences, closed form, invariants."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, **kw):
    o, _ = oracle.full_attention(q, k, v, **kw)
    return float((do * o).sum())


@pytest.mark.parametrize("causal,q_offset,kv_offset", [(False, 0, 0), (True, 0, 0), (True, 3, 1)])
def test_finite_differences(causal, q_offset, kv_offset):
    B, Hq, Hkv, S, D = 1, 4, 2, 6, 3
    q, k, v = _rand((B, Hq, S, D), 1), _rand((B, Hkv, S, D), 2), _rand((B, Hkv, S, D), 3)
    do = _rand((B, Hq, S, D), 4)
    kw = dict(causal=causal, scale=0.7, q_offset=q_offset, kv_offset=kv_offset)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, **kw)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, **kw)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-30)
        assert err <= 1e-6, (name, err)


def _golden(x):
    if isinstance(x, list):
        return [_golden(y) for y in x]
    if isinstance(x, str):
        return {"ln3": math.log(3), "ln4": math.log(4),
                "0.75ln3": 0.75 * math.log(3), "-0.75ln3": -0.75 * math.log(3)}[x]
    return float(x)


@pytest.mark.parametrize("mode", ["noncausal", "causal"])
def test_golden_closed_form(mode):
    g = json.load(open(os.path.join(GOLDEN, "two_key_closed_form.json")))
    arr = lambda key: np.array(_golden(g[key]))[None, None]
    dq, dk, dv = oracle.attention_bwd(arr("q"), arr("k"), arr("v"), arr("dout"),
                                      causal=(mode == "causal"), scale=g["scale"])
    for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert np.max(np.abs(got[0, 0] - np.array(_golden(g[mode][key])))) <= 1e-15, key


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, Hq, Hkv, S, D = 2, 4, 2, 40, 8
    q, k, v = _rand((B, Hq, S, D), 5), _rand((B, Hkv, S, D), 6), _rand((B, Hkv, S, D), 7)
    do = _rand((B, Hq, S, D), 8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=causal, row_block=7)
    # sum over keys of dK vanishes (each row of dS sums to zero)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    # sum over keys of dV equals the sum of dO over the query heads of the group
    group = Hq // Hkv
    sdo = do.reshape(B, Hkv, group, S, D).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - sdo)) <= 1e-12


def test_sampled_heads_match_full():
    B, Hq, Hkv, S, D = 1, 4, 2, 20, 8
    q, k, v = _rand((B, Hq, S, D), 9), _rand((B, Hkv, S, D), 10), _rand((B, Hkv, S, D), 11)
    do = _rand((B, Hq, S, D), 12)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True)
    part = oracle.attention_bwd_heads(q, k, v, do, [(0, 1)], causal=True, row_block=6)
    pq, pk, pv = part[(0, 1)]
    assert np.max(np.abs(pq - dq[0, 2:4])) <= 1e-13
    assert np.max(np.abs(pk - dk[0, 1])) <= 1e-13
    assert np.max(np.abs(pv - dv[0, 1])) <= 1e-13
