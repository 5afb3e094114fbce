"""Oracle: FP8 (e4m3) inputs for the attention forward -- TEST INFRASTRUCTURE ONLY.

See ``oracle/__init__.py`` for who may import it.

The pages say only that FlashAttention-3 supports the FP8 data type, which halves
the traffic of the key/value cache ([P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效",
section "那么，FlashAttention-2 和 -3 又改进了什么？", its FlashAttention-3 list), and that
sequence parallelism combines with FP8 training ([P2] "Ulysses与Ring-Attention序列并行技术详解",
the list of engineering considerations near its end).  Everything else here is a
reading, stated once:

* Format: e4m3 as defined by the OCP 8-bit floating-point specification -- 1 sign,
  4 exponent (bias 7) and 3 mantissa bits; exponent 0 holds the subnormals M * 2^-9;
  no infinities; S.1111.111 is NaN, so the largest finite value is 1.75 * 2^8 = 448.
  Conversion rounds to nearest, ties to even mantissa; a magnitude that rounds past
  448 is NaN.
* Scaling rule: one scale per (batch, head) of each of q, k, v.  With a = max |x| over
  the head (fp32), the codes are e4m3(clamp(x * r, -448, 448)) where r = 448 / a and
  every product is an fp32 operation rounded to nearest even; the stored descale is
  a / 448 (fp32), and the value a code stands for is decode(code) * descale.  An all-
  zero head has r = descale = 1.
* Attention over fp8 inputs is exact softmax attention (the definition, as
  ``attention.full_attention``) of the dequantized q, k, v: the oracle never rounds,
  so input quantization is not counted as error -- only what the GPU rounds after it.
* Layouts: q and k codes are [B, H, S, D]; v codes may be stored transposed,
  [B, H, D, S_pad] with S_pad = S rounded up to a multiple of 16 and zero codes in
  the padding.

Error bound (derived, used by the parity tests).  The GPU rounds the exponentials
P' = 2^(6 + delta) * exp(s - m) (m = the row max, 0 <= delta <= 2 the lag of its
running max) to e4m3 before the P V product while the normaliser sums the unrounded
fp32 values.  A normal e4m3 value is within 2^-4 of relative error; P' < 2^-6 is
subnormal, within 2^-10 absolute, and needs exp(s - m) < 2^-12; the normaliser is at
least 2^6.  Hence, element-wise,

    |o - o_exact| <= 2^-4 * sum_j p_j |v_j|  +  2^-16 * n_sub * max_j |v_j|

with p the exact softmax weights and n_sub the number of visible keys with
exp(s - m) < 2^-12.  ``p_rounding_bound`` computes the right-hand side for listed rows,
``p_rounding_bound_head`` for every row of one head.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .attention import _as64, _default_scale, _masked_scores, full_attention

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6      # smallest normal: 2^-6
_SUB_QUANTUM = 2.0 ** -9  # subnormal spacing


def e4m3_decode(codes) -> np.ndarray:
    """Value (fp64) of each e4m3 code; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * _SUB_QUANTUM, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest e4m3 code (ties to even mantissa)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    # the quantum of the binade a falls in (subnormals share the 2^-6 binade's quantum)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, _MIN_NORMAL_EXP)
    # floor(log2) can be off by one right at a power of two; fix it exactly
    e = np.where(a >= np.exp2(e + 1), e + 1, e)
    e = np.where((a < np.exp2(e)) & (e > _MIN_NORMAL_EXP), e - 1, e)
    quantum = np.exp2(e - 3)
    n = np.rint(a / quantum)  # a / quantum is exact; rint rounds half to even
    v = n * quantum           # the rounded magnitude (may step up into the next binade)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = v < 2.0 ** _MIN_NORMAL_EXP
    codes = np.where(sub, np.rint(v / _SUB_QUANTUM).astype(np.int64), codes)
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(sub, 1.0, v)))
    mant = np.rint(np.where(sub, 0.0, v / np.exp2(ev) * 8.0 - 8.0)).astype(np.int64)
    codes = np.where(sub, codes, ((ev.astype(np.int64) + 7) << 3) | mant)
    codes = np.where((v > E4M3_MAX) | np.isnan(a), 0x7F, codes)
    return (codes | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_heads(x) -> Tuple[np.ndarray, np.ndarray]:
    """Codes [B, H, S, D] and descales [B, H] (fp32) of x by the per-head rule above.

    x is read as fp32 (bf16 inputs are exact in it); every step is an fp32 operation,
    so the rounding decisions are the ones an fp32 implementation takes.
    """
    x = np.asarray(x, dtype=np.float32)
    B, H = x.shape[:2]
    codes = np.zeros(x.shape, dtype=np.uint8)
    descale = np.ones((B, H), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    for b in range(B):
        for h in range(H):
            amax = np.float32(np.max(np.abs(x[b, h]), initial=np.float32(0)))
            if amax > 0:
                r = np.float32(f448 / amax)
                descale[b, h] = np.float32(amax / f448)
            else:
                r = np.float32(1.0)
            y = np.clip((x[b, h] * r).astype(np.float32), -f448, f448)
            codes[b, h] = e4m3_encode(y)
    return codes, descale


def transpose_codes(codes: np.ndarray) -> np.ndarray:
    """[B, H, S, D] codes -> [B, H, D, S_pad] (S_pad = S rounded up to 16, zero codes)."""
    B, H, S, D = codes.shape
    S_pad = (S + 15) // 16 * 16
    out = np.zeros((B, H, D, S_pad), dtype=np.uint8)
    out[:, :, :, :S] = codes.transpose(0, 1, 3, 2)
    return out


def dequantize(codes, descale) -> np.ndarray:
    """decode(code) * descale[b, h], fp64."""
    return e4m3_decode(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]


def fp8_attention(q_codes, k_codes, v_codes, q_descale, k_descale, v_descale, *,
                  causal: bool = False, scale: Optional[float] = None, q_offset: int = 0,
                  kv_offset: int = 0, v_transposed: bool = False):
    """(o, lse) of exact attention over the dequantized fp8 inputs (fp64).

    Ring chunking does not change the exact result, so no chunk parameters appear.
    """
    q = dequantize(q_codes, q_descale)
    k = dequantize(k_codes, k_descale)
    if v_transposed:
        Skv = k.shape[2]
        v = dequantize(np.asarray(v_codes)[:, :, :, :Skv].transpose(0, 1, 3, 2), v_descale)
    else:
        v = dequantize(v_codes, v_descale)
    return full_attention(q, k, v, causal=causal, scale=scale, q_offset=q_offset,
                          kv_offset=kv_offset)


def p_rounding_bound(q, k, v, rows: Iterable[Tuple[int, int, int]], *, causal: bool = False,
                     scale: Optional[float] = None, q_offset: int = 0,
                     kv_offset: int = 0) -> np.ndarray:
    """The derived element-wise bound (module docstring) for the given (b, h, i) rows.

    q, k, v are the dequantized fp64 inputs; returns [len(rows), D].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Hq, Hkv, D = q.shape[1], k.shape[1], q.shape[3]
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    kpos = kv_offset + np.arange(k.shape[2])
    out = []
    for (b, h, i) in rows:
        g = h // group
        s = _masked_scores(q[b, h, i:i + 1], k[b, g], scale,
                           np.array([q_offset + i]), kpos, causal)[0]
        vis = np.isfinite(s)
        if not vis.any():
            out.append(np.zeros(D))
            continue
        pt = np.exp(s[vis] - s[vis].max())
        p = pt / pt.sum()
        va = np.abs(v[b, g][vis])
        n_sub = int(np.count_nonzero(pt < 2.0 ** -12))
        out.append(2.0 ** -4 * (p @ va) + 2.0 ** -16 * n_sub * va.max(axis=0))
    return np.stack(out)


def p_rounding_bound_head(q, k, v, b: int, h: int, *, causal: bool = False,
                          scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0,
                          row_block: int = 256) -> np.ndarray:
    """``p_rounding_bound`` for every row of head (b, h) at once -> [Sq, D].

    The same right-hand side, row block by row block: the visible keys of a row are a
    prefix of the key axis (all keys without the mask, those at or before the row's
    position with it), so max_j |v_j| over them is a running maximum along the keys.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    Hq, Hkv, Sq, D = q.shape[1], k.shape[1], q.shape[2], q.shape[3]
    Skv = k.shape[2]
    scale = _default_scale(scale, D)
    g = h // (Hq // Hkv)
    kpos = kv_offset + np.arange(Skv)
    va = np.abs(v[b, g])
    va_prefix_max = np.maximum.accumulate(va, axis=0) if Skv else va
    out = np.zeros((Sq, D))
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        qpos = q_offset + np.arange(r0, r1)
        s = _masked_scores(q[b, h, r0:r1], k[b, g], scale, qpos, kpos, causal)
        vis = np.isfinite(s)
        n_vis = vis.sum(axis=1)
        m = np.where(n_vis > 0, s.max(axis=1, initial=-np.inf), 0.0)
        pt = np.where(vis, np.exp(s - m[:, None]), 0.0)
        tot = pt.sum(axis=1)
        p = pt / np.where(tot > 0, tot, 1.0)[:, None]
        n_sub = np.count_nonzero(vis & (pt < 2.0 ** -12), axis=1)
        last = np.clip(n_vis - 1, 0, max(Skv - 1, 0))
        vmax = va_prefix_max[last] if Skv else np.zeros((r1 - r0, D))
        blk = 2.0 ** -4 * (p @ va) + 2.0 ** -16 * n_sub[:, None] * vmax
        out[r0:r1] = np.where((n_vis > 0)[:, None], blk, 0.0)
    return out


def simulate_p_rounding(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                        delta: float = 0.0):
    """o with P' = 2^(6 + delta) exp(s - m) rounded to e4m3 in the numerator only
    (fp64 otherwise): the arithmetic the bound above describes, for pinning it."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    o = np.zeros_like(q)
    pos = np.arange(Sq)
    kpos = np.arange(k.shape[2])
    for b in range(B):
        for h in range(Hq):
            s = _masked_scores(q[b, h], k[b, h // group], scale, pos, kpos, causal)
            m = np.max(s, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            with np.errstate(invalid="ignore"):
                pp = np.exp2(6.0 + delta) * np.exp(s - m)
            pp = np.where(np.isfinite(s), pp, 0.0)
            l = pp.sum(axis=1, keepdims=True)
            num = e4m3_decode(e4m3_encode(pp)) @ v[b, h // group]
            o[b, h] = np.where(l > 0, num / np.where(l > 0, l, 1.0), 0.0)
    return o


__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_heads", "transpose_codes",
           "dequantize", "fp8_attention", "p_rounding_bound", "p_rounding_bound_head",
           "simulate_p_rounding"]
