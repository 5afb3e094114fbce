"""Oracle: gradients of softmax attention (fp64, no autograd).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import it.

The pages say only that the backward pass works from the forward's saved
statistics and recomputes the attention weights rather than storing them
([P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效", section
"为什么传统注意力这么“吃”显存？"), and that gradients travel back along the same
path ([P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用", section
"Ring-Attention：面向大规模部署的工程利器").  The formulas themselves are the
textbook softmax-attention gradient, written here for L = sum(dO * O):

    P    = softmax of the masked scores (the oracle's own forward)
    O    = P V,            D_i = sum_d dO_id O_id
    dV   = P^T dO
    dP   = dO V^T
    dS   = P o (dP - D)    (0 where masked)
    dQ   = scale * dS K
    dK   = scale * dS^T Q

With grouped heads, dK and dV of key/value head g sum over the query heads of
its group.  Pinned in ``tests/`` by central finite differences of L and by
invariants (sum_j dS_ij = 0, sum_j dK_j = 0, sum_j dV_j = sum_i dO_i).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .attention import (_as64, _default_scale, _masked_scores, _row_softmax, _shapes,
                        chunk_bounds, ring_attention, ring_order)


def _bwd_group(q, k, v, do, b, g, group, scale, qpos, kpos, causal, row_block):
    """Gradients of one key/value head g (and its query heads) in batch b."""
    Sq, D = q.shape[2], q.shape[3]
    dk_g = np.zeros((k.shape[2], D))
    dv_g = np.zeros((k.shape[2], D))
    dq_heads = {}
    for h in range(g * group, (g + 1) * group):
        dq_h = np.zeros((Sq, D))
        for r0 in range(0, Sq, row_block):
            r1 = min(Sq, r0 + row_block)
            s = _masked_scores(q[b, h, r0:r1], k[b, g], scale, qpos[r0:r1], kpos, causal)
            p, _ = _row_softmax(s)
            o = p @ v[b, g]
            dO = do[b, h, r0:r1]
            Di = (dO * o).sum(axis=1)
            dv_g += p.T @ dO
            dp = dO @ v[b, g].T
            ds = p * (dp - Di[:, None])
            dq_h[r0:r1] = scale * (ds @ k[b, g])
            dk_g += scale * (ds.T @ q[b, h, r0:r1])
        dq_heads[h] = dq_h
    return dq_heads, dk_g, dv_g


def attention_bwd(q, k, v, do, *, causal: bool = False, scale: Optional[float] = None,
                  q_offset: int = 0, kv_offset: int = 0, row_block: int = 256):
    """(dq, dk, dv) of L = sum(dO * attention(q, k, v)), all fp64."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must be shaped like q")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    group = Hq // Hkv
    qpos = q_offset + np.arange(Sq)
    kpos = kv_offset + np.arange(Skv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for g in range(Hkv):
            dq_heads, dk[b, g], dv[b, g] = _bwd_group(q, k, v, do, b, g, group, scale,
                                                      qpos, kpos, causal, row_block)
            for h, val in dq_heads.items():
                dq[b, h] = val
    return dq, dk, dv


def attention_bwd_heads(q, k, v, do, kv_heads: Iterable[Tuple[int, int]], *,
                        causal: bool = False, scale: Optional[float] = None,
                        q_offset: int = 0, kv_offset: int = 0, row_block: int = 256):
    """Gradients for selected (b, g) key/value heads only (large problems, sampled).

    Returns {(b, g): (dq [group, Sq, D], dk [Skv, D], dv [Skv, D])}; dq rows are the
    query heads g*group .. (g+1)*group-1 of batch b.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    group = Hq // Hkv
    qpos = q_offset + np.arange(Sq)
    kpos = kv_offset + np.arange(Skv)
    out = {}
    for (b, g) in kv_heads:
        dq_heads, dk_g, dv_g = _bwd_group(q, k, v, do, b, g, group, scale, qpos, kpos,
                                          causal, row_block)
        out[(b, g)] = (np.stack([dq_heads[h] for h in sorted(dq_heads)]), dk_g, dv_g)
    return out


def varlen_attention_bwd(q, k, v, do, cu_seqlens: Sequence[int], *, causal: bool = False,
                         scale: Optional[float] = None):
    """(dq, dk, dv) of L = sum(dO * varlen_attention(q, k, v, cu_seqlens)), fp64.

    Each packed document is its own attention problem (the reading of the pages'
    packing taken in ``attention.varlen_attention``), so its gradients are
    ``attention_bwd`` of its own slice; tokens in no document get zero gradients.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, T, D, Hkv, Tk = _shapes(q, k, v)
    if Tk != T or do.shape != q.shape:
        raise ValueError("packed q, k, v, dO must hold the same tokens")
    cu = [int(x) for x in cu_seqlens]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])) or cu[-1] > T:
        raise ValueError("cu_seqlens must start at 0, not decrease and stay within T")
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for a, b in zip(cu, cu[1:]):
        if b > a:
            dq[:, :, a:b], dk[:, :, a:b], dv[:, :, a:b] = attention_bwd(
                q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], do[:, :, a:b], causal=causal,
                scale=scale)
    return dq, dk, dv


def ring_attention_bwd(q, k, v, do, *, num_chunks: int, start_chunk: int = 0,
                       causal: bool = False, scale: Optional[float] = None,
                       q_offset: int = 0, kv_offset: int = 0):
    """One device's ring backward, chunk by chunk; returns (dq, dk, dv), fp64.

    The device holds the query block q (and dO) and sees the key/value sequence as
    ``num_chunks`` equal chunks, visited in the forward's ring order
    (start_chunk + t) mod P ([P2] ``ring_attention_forward`` listing; [P1]
    "Ring-Attention：面向大规模部署的工程利器": gradients travel back along the
    ring).  The forward's merged (o, lse) over every chunk come first (the
    oracle's own ``ring_attention``); then, per visited chunk c,

        P_c = exp(s_c - lse)  (0 where masked),  D = rowsum(dO * o)
        dV_c = P_c^T dO,  dS_c = P_c o (dO V_c^T - D)
        dQ  += scale dS_c K_c,  dK_c = scale dS_c^T q

    so dQ is a sum over chunks and dK/dV of chunk c hold this device's share only
    (the sum over every device's query block is the full gradient).  A causal chunk
    whose first key lies after the block's last query is skipped (it adds 0).
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must be shaped like q")
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    o, lse = ring_attention(q, k, v, num_chunks=num_chunks, start_chunk=start_chunk,
                            causal=causal, scale=scale, q_offset=q_offset,
                            kv_offset=kv_offset)
    delta = (do * o).sum(axis=3)
    qpos = q_offset + np.arange(Sq)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for c in ring_order(num_chunks, start_chunk):
        lo, hi = chunk_bounds(Skv, num_chunks, c)
        if hi == lo or (causal and kv_offset + lo > q_offset + Sq - 1):
            continue
        kpos = kv_offset + np.arange(lo, hi)
        for b in range(B):
            for h in range(Hq):
                g = h // group
                kc, vc = k[b, g, lo:hi], v[b, g, lo:hi]
                s = _masked_scores(q[b, h], kc, scale, qpos, kpos, causal)
                with np.errstate(invalid="ignore"):
                    p = np.exp(s - lse[b, h][:, None])
                p[~np.isfinite(s)] = 0.0
                dO = do[b, h]
                dv[b, g, lo:hi] += p.T @ dO
                ds = p * (dO @ vc.T - delta[b, h][:, None])
                dq[b, h] += scale * (ds @ kc)
                dk[b, g, lo:hi] += scale * (ds.T @ q[b, h])
    return dq, dk, dv
