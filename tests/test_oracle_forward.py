"""Pins of the oracle's forward definition against things other than itself.

Each check is chosen so a plausible slip in ``oracle.full_attention`` (a dropped
scale, a transposed operand, a wrong head mapping, an off-by-one in the causal
mask, a wrong log base) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.attention import chunk_bounds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, causal, scale, q_offset, kv_offset):
    """Pure-Python loops over the definition, math.exp / math.fsum only."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    o = [[[[0.0] * D for _ in range(Sq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[-math.inf] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Sq):
                vis = [j for j in range(Skv) if (not causal) or kv_offset + j <= q_offset + i]
                if not vis:
                    continue
                s = {j: scale * math.fsum(float(q[b, h, i, d]) * float(k[b, g, j, d])
                                          for d in range(D)) for j in vis}
                m = max(s.values())
                z = math.fsum(math.exp(s[j] - m) for j in vis)
                l = m + math.log(z)
                lse[b][h][i] = l
                for d in range(D):
                    o[b][h][i][d] = math.fsum(math.exp(s[j] - l) * float(v[b, g, j, d])
                                              for j in vis)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal,q_offset,kv_offset", [
    (False, 0, 0), (True, 0, 0), (True, 5, 0), (True, 0, 3), (True, 2, 9)])
def test_brute_force_tiny(causal, q_offset, kv_offset):
    q = _rand((2, 4, 7, 5), 1)
    k = _rand((2, 2, 9, 5), 2)
    v = _rand((2, 2, 9, 5), 3)
    scale = 0.37
    o, lse = oracle.full_attention(q, k, v, causal=causal, scale=scale,
                                   q_offset=q_offset, kv_offset=kv_offset, row_block=3)
    ob, lb = _brute(q, k, v, causal, scale, q_offset, kv_offset)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) <= 1e-13
    assert np.max(np.abs(o - ob)) <= 1e-13


def test_matches_torch_sdpa_fp64():
    """A different library's attention routine, fp64 on the CPU, with an explicit mask."""
    B, Hq, Hkv, Sq, Skv, D = 2, 6, 3, 33, 47, 16
    q, k, v = _rand((B, Hq, Sq, D), 4), _rand((B, Hkv, Skv, D), 5), _rand((B, Hkv, Skv, D), 6)
    q_offset, kv_offset = 20, 0
    o, lse = oracle.full_attention(q, k, v, causal=True, q_offset=q_offset, kv_offset=kv_offset)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    qt = torch.from_numpy(q)
    mask = (torch.arange(Skv)[None, :] + kv_offset) <= (torch.arange(Sq)[:, None] + q_offset)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.max(np.abs(o - ref.numpy())) <= 1e-12
    s = torch.einsum("bhid,bhjd->bhij", qt, kt) / math.sqrt(D)
    s = s.masked_fill(~mask, float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


def test_scipy_softmax_and_logsumexp():
    q, k = _rand((1, 2, 12, 8), 7), _rand((1, 2, 30, 8), 8)
    P = oracle.attention_probs(q, k, scale=0.5)
    s = 0.5 * np.einsum("bhid,bhjd->bhij", q, k)
    assert np.max(np.abs(P - scipy.special.softmax(s, axis=-1))) <= 1e-14
    _, lse = oracle.full_attention(q, k, k, scale=0.5)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=-1))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    q, k = _rand((1, 3, 40, 8), 9), _rand((1, 3, 40, 8), 10)
    P = oracle.attention_probs(q, k, causal=causal)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-14
    if causal:
        assert np.all(np.triu(P[0, 0], 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    q, k = _rand((1, 2, 20, 8), 11), _rand((1, 1, 20, 8), 12)
    v = np.full((1, 1, 20, 8), -2.75)
    o, _ = oracle.full_attention(q, k, v, causal=causal, q_offset=3)
    assert np.max(np.abs(o + 2.75)) <= 8 * np.finfo(float).eps * 2.75


def test_single_visible_key():
    q, k, v = _rand((1, 2, 5, 8), 13), _rand((1, 2, 5, 8), 14), _rand((1, 2, 5, 8), 15)
    o, lse = oracle.full_attention(q, k, v, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    s00 = (q[:, :, 0] * k[:, :, 0]).sum(-1) / math.sqrt(8)
    assert np.max(np.abs(lse[:, :, 0] - s00)) <= 1e-15


def test_zero_q_uniform_weights():
    k, v = _rand((1, 1, 16, 4), 16), _rand((1, 1, 16, 4), 17)
    q = np.zeros((1, 1, 16, 4))
    o, lse = oracle.full_attention(q, k, v, causal=True)
    for i in range(16):
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, :i + 1].mean(0))) <= 1e-15
        assert abs(lse[0, 0, i] - math.log(i + 1)) <= 1e-15


def test_empty_rows():
    """Queries that see no key (q_offset < kv_offset) give o = 0, lse = -inf, no NaN."""
    q, k, v = _rand((1, 1, 6, 4), 18), _rand((1, 1, 6, 4), 19), _rand((1, 1, 6, 4), 20)
    o, lse = oracle.full_attention(q, k, v, causal=True, q_offset=0, kv_offset=3)
    assert np.all(np.isneginf(lse[0, 0, :3])) and np.all(o[0, 0, :3] == 0.0)
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    assert not np.isnan(o).any()


def test_causal_future_perturbation():
    q, k, v = _rand((1, 2, 24, 8), 21), _rand((1, 2, 24, 8), 22), _rand((1, 2, 24, 8), 23)
    o, lse = oracle.full_attention(q, k, v, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 10:] += 5.0 * _rand((1, 2, 14, 8), 24)
    v2[:, :, 10:] -= 3.0
    o2, lse2 = oracle.full_attention(q, k2, v2, causal=True)
    assert np.array_equal(o[:, :, :10], o2[:, :, :10])
    assert np.array_equal(lse[:, :, :10], lse2[:, :, :10])
    assert not np.allclose(o[:, :, 10:], o2[:, :, 10:])


def test_gqa_mapping_contiguous_groups():
    """Query heads 0..g-1 read kv head 0: moving kv head 1 must not change them."""
    q, k, v = _rand((1, 4, 10, 8), 25), _rand((1, 2, 10, 8), 26), _rand((1, 2, 10, 8), 27)
    o, _ = oracle.full_attention(q, k, v)
    v2 = v.copy()
    v2[:, 1] += 1.0
    o2, _ = oracle.full_attention(q, k, v2)
    assert np.array_equal(o[:, :2], o2[:, :2])
    assert np.allclose(o2[:, 2:], o[:, 2:] + 1.0, atol=1e-14)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = _rand((1, 1, 9, 16), 28), _rand((1, 1, 9, 16), 29), _rand((1, 1, 9, 16), 30)
    a = oracle.full_attention(q, k, v)
    b = oracle.full_attention(q, k, v, scale=0.25)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_attention_rows_matches_full():
    q, k, v = _rand((2, 4, 30, 8), 31), _rand((2, 2, 50, 8), 32), _rand((2, 2, 50, 8), 33)
    o, lse = oracle.full_attention(q, k, v, causal=True, q_offset=20)
    idx = [(0, 0, 0), (1, 3, 29), (0, 2, 7), (1, 1, 15)]
    orow, lrow = oracle.attention_rows(q, k, v, idx, causal=True, q_offset=20)
    for n, (b, h, i) in enumerate(idx):
        assert np.max(np.abs(orow[n] - o[b, h, i])) <= 1e-15
        assert abs(lrow[n] - lse[b, h, i]) <= 1e-15


def _golden(x):
    if isinstance(x, list):
        return [_golden(y) for y in x]
    if isinstance(x, str):
        return {"ln3": math.log(3), "ln4": math.log(4),
                "0.75ln3": 0.75 * math.log(3), "-0.75ln3": -0.75 * math.log(3)}[x]
    return float(x)


@pytest.mark.parametrize("mode", ["noncausal", "causal"])
def test_golden_two_key_closed_form(mode):
    g = json.load(open(os.path.join(GOLDEN, "two_key_closed_form.json")))
    q = np.array(_golden(g["q"]))[None, None]
    k = np.array(_golden(g["k"]))[None, None]
    v = np.array(_golden(g["v"]))[None, None]
    o, lse = oracle.full_attention(q, k, v, causal=(mode == "causal"), scale=g["scale"])
    assert np.max(np.abs(o[0, 0] - np.array(_golden(g[mode]["o"])))) <= 1e-15
    assert np.max(np.abs(lse[0, 0] - np.array(_golden(g[mode]["lse"])))) <= 1e-15


def test_chunk_bounds_equal_contiguous():
    assert [chunk_bounds(256, 4, c) for c in range(4)] == [(0, 64), (64, 128), (128, 192),
                                                           (192, 256)]
    with pytest.raises(ValueError):
        chunk_bounds(250, 4, 0)
