"""Pins of the oracle's FP8 pieces: the e4m3 code, the per-head scaling rule, attention
over dequantized inputs and the derived bound on rounding the attention weights.

The code is pinned against torch's float8_e4m3fn conversion (a library routine) and the
format's defining values; the bound against an exact simulation of the rounding,
including a case built to sit near the bound, which a smaller constant would fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_decode_matches_torch_and_the_definition():
    codes = np.arange(256, dtype=np.uint8)
    dec = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    same = (dec == ref) | (np.isnan(dec) & np.isnan(ref))
    assert same.all()
    # defining values: 1.0, the largest finite value, smallest normal and subnormal, NaN
    assert dec[0x38] == 1.0 and dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert dec[0x08] == 2.0 ** -6 and dec[0x01] == 2.0 ** -9 and dec[0x07] == 7 * 2.0 ** -9
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert dec[0x80] == 0.0 and math.copysign(1.0, dec[0x80]) == -1.0


def test_encode_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000) * s for s in (1e-3, 1e-1, 1.0, 30.0, 200.0)]
    finite = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448
    mids = (finite[1:] + finite[:-1]) / 2
    eps = np.float32(1 + 2.0 ** -20)
    x = np.concatenate(vals + [finite, mids, mids * eps, mids / eps, -mids,
                               [450.0, 463.0, 464.0, -464.0]]).astype(np.float32)
    got = fp8.e4m3_encode(x)
    want = _torch_encode(x)
    assert np.array_equal(got, want)


def test_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def test_quantize_heads_rule():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((2, 3, 40, 16)) * [[[[1.0]], [[7.0]], [[0.01]]]]).astype(np.float32)
    x[1, 2] = 0.0  # an all-zero head
    codes, desc = fp8.quantize_heads(x)
    for b in range(2):
        for h in range(3):
            xh = x[b, h]
            amax = np.float32(np.abs(xh).max())
            if amax == 0:
                assert desc[b, h] == 1.0 and not codes[b, h].any()
                continue
            assert desc[b, h] == np.float32(amax / np.float32(448))
            # the largest magnitude maps to +-448 exactly
            i = np.unravel_index(np.argmax(np.abs(xh)), xh.shape)
            assert codes[b, h][i] in (0x7E, 0xFE)
            # the same pipeline through torch's conversion
            r = np.float32(np.float32(448) / amax)
            y = np.clip(xh * r, -448, 448).astype(np.float32)
            assert np.array_equal(codes[b, h], _torch_encode(y))
            # dequantized values are within half a quantum of x
            deq = fp8.dequantize(codes[b:b + 1, h:h + 1], desc[b:b + 1, h:h + 1])[0, 0]
            err = np.abs(deq - xh)
            assert (err <= np.maximum(2.0 ** -4 * np.abs(xh), 2.0 ** -10 * amax / 448) * 1.001
                    + 1e-30).all()


def test_transpose_codes_layout():
    codes = np.random.default_rng(3).integers(0, 0x7E, size=(1, 2, 37, 8), dtype=np.uint8)
    t = fp8.transpose_codes(codes)
    assert t.shape == (1, 2, 8, 48)
    assert np.array_equal(t[:, :, :, :37], codes.transpose(0, 1, 3, 2))
    assert not t[:, :, :, 37:].any()


def test_fp8_attention_is_attention_of_the_dequantized_inputs():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 4, 33, 16)).astype(np.float32) for _ in range(3))
    k, v = k[:, :2], v[:, :2]
    (qc, qd), (kc, kd), (vc, vd) = (fp8.quantize_heads(t) for t in (q, k, v))
    o, lse = fp8.fp8_attention(qc, kc, vc, qd, kd, vd, causal=True)
    ot, lt = fp8.fp8_attention(qc, kc, fp8.transpose_codes(vc), qd, kd, vd, causal=True,
                               v_transposed=True)
    np.testing.assert_allclose(ot, o, rtol=0, atol=1e-13)  # same values, another memory order
    np.testing.assert_allclose(lt, lse, rtol=0, atol=1e-13)
    ref_o, ref_l = oracle.full_attention(fp8.dequantize(qc, qd), fp8.dequantize(kc, kd),
                                         fp8.dequantize(vc, vd), causal=True)
    assert np.array_equal(o, ref_o) and np.array_equal(lse, ref_l)
    # quantization error of the inputs is real but small against the bf16-free result
    o32, _ = oracle.full_attention(q, k, v, causal=True)
    assert np.abs(o - o32).max() < 0.25


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("delta", [0.0, 1.0, 2.0])
@pytest.mark.parametrize("spread", [1.0, 6.0])
def test_bound_holds_for_simulated_rounding(causal, delta, spread):
    """Rounding P' = 2^(6+delta) exp(s - m) to e4m3 (numerator only) stays within the
    bound, for score spreads that do and do not reach the subnormal range."""
    rng = np.random.default_rng(int(10 * delta + spread))
    q = rng.standard_normal((1, 2, 48, 8)) * spread
    k = rng.standard_normal((1, 2, 64, 8))
    v = rng.standard_normal((1, 2, 64, 8))
    o_ref, _ = oracle.full_attention(q, k, v, causal=causal)
    o_sim = fp8.simulate_p_rounding(q, k, v, causal=causal, delta=delta)
    rows = [(0, h, i) for h in range(2) for i in range(48)]
    bound = fp8.p_rounding_bound(q, k, v, rows, causal=causal)
    err = np.stack([np.abs(o_sim[b, h, i] - o_ref[b, h, i]) for (b, h, i) in rows])
    assert (err <= bound * (1 + 1e-9) + 1e-15).all()
    assert err.max() > 0  # the rounding is real


def test_bound_constant_is_tight():
    """Keys whose P' = 34 (a tie, rounded to 32: 5.9 % low) with v = 1 beside a max key
    with v = 0: the error is 2/34 of sum p|v|, above 2^-5, within 2^-4."""
    n = 5
    s = np.array([0.0] + [math.log(34 / 64)] * n)  # scores relative to the max key
    q = np.array([[[[1.0]]]])
    k = s[None, None, :, None]
    v = np.array([0.0] + [1.0] * n)[None, None, :, None]
    o_ref, _ = oracle.full_attention(q, k, v, scale=1.0)
    o_sim = fp8.simulate_p_rounding(q, k, v, scale=1.0)
    A = (n * 34 / (64 + 34 * n))
    err = abs(o_sim[0, 0, 0, 0] - o_ref[0, 0, 0, 0])
    assert err == pytest.approx(2 / 34 * A, rel=1e-12)
    assert err > 2.0 ** -5 * A
    bound = fp8.p_rounding_bound(q, k, v, [(0, 0, 0)], scale=1.0)[0, 0]
    assert err <= bound


@pytest.mark.parametrize("causal,q_off,kv_off", [(False, 0, 0), (True, 0, 0), (True, 30, 0),
                                                 (True, 0, 20), (True, 5, 70)])
def test_head_bound_matches_row_bound_and_holds(causal, q_off, kv_off):
    """The whole-head form of the bound is the per-row bound for every row (including
    rows with no visible key), with several row blocks and a ragged last block, and the
    simulated e4m3 rounding of P' stays within it."""
    rng = np.random.default_rng(7 + q_off + kv_off)
    q = rng.standard_normal((1, 4, 70, 8)) * 4.0
    k = rng.standard_normal((1, 2, 64, 8))
    v = rng.standard_normal((1, 2, 64, 8))
    kw = dict(causal=causal, q_offset=q_off, kv_offset=kv_off)
    for h in range(4):
        head = fp8.p_rounding_bound_head(q, k, v, 0, h, row_block=32, **kw)
        rows = fp8.p_rounding_bound(q, k, v, [(0, h, i) for i in range(70)], **kw)
        np.testing.assert_allclose(head, rows, rtol=1e-12, atol=1e-300)
    if q_off == 0 and kv_off == 0:
        o_ref, _ = oracle.full_attention(q, k, v, causal=causal)
        o_sim = fp8.simulate_p_rounding(q, k, v, causal=causal, delta=1.0)
        for h in range(4):
            bound = fp8.p_rounding_bound_head(q, k, v, 0, h, causal=causal)
            assert (np.abs(o_sim[0, h] - o_ref[0, h]) <= bound * (1 + 1e-9) + 1e-15).all()
