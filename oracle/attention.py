"""Oracle: full softmax attention, chunk partials and the two LSE merges (fp64).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import it.

Page legend (title, host):
  [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn)
  [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com)
  [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn)

Conventions (readings where the pages are silent, each listed in the design doc):

* Layout [B, H, L, D] with the key/value sequence on axis 2, as in the
  ``ulysses_attention_forward`` listing of [P2].
* Scores are ``scale * q . k`` with ``scale = 1/sqrt(D)`` by default, the
  divisor both listings of [P2] use.
* The pages never mention masking.  ``causal`` means: key j (global position
  kv_offset + j) is visible to query i (global position q_offset + i) iff
  kv_offset + j <= q_offset + i.
* Grouped heads (also not on the pages): query head h reads key/value head
  h // (Hq // Hkv).
* lse is the natural log of the sum of exp(score) over visible keys, the
  quantity the ``ring_attention_forward`` listing of [P2] carries with
  ``torch.log``.  A row with no visible key has o = 0 and lse = -inf.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError("k and v must be [B, Hkv, Skv, D] matching q")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Sq, D, Hkv, Skv


def _default_scale(scale: Optional[float], D: int) -> float:
    # [P2], both listings: scores are divided by the square root of the head dim.
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _masked_scores(qrows: np.ndarray, kmat: np.ndarray, scale: float,
                   qpos: np.ndarray, kpos: np.ndarray, causal: bool) -> np.ndarray:
    """s_ij = scale * q_i . k_j, with -inf where key j is not visible to row i."""
    s = scale * (qrows @ kmat.T)
    if causal:
        s = np.where(kpos[None, :] <= qpos[:, None], s, NEG_INF)
    return s


def _row_softmax(s: np.ndarray):
    """Row statistics of masked scores, as [P1] defines them for one chunk.

    m_i = max_j s_ij, z_i = sum_j exp(s_ij - m_i), lse_i = m_i + ln z_i,
    P_ij = exp(s_ij - lse_i).  Rows with no visible key: P = 0, lse = -inf.
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    nonempty = np.isfinite(m)
    m_safe = np.where(nonempty, m, 0.0)
    z = np.exp(s - m_safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(nonempty, m_safe + np.log(np.where(nonempty, z, 1.0)), NEG_INF)
    lse_safe = np.where(nonempty, lse, 0.0)
    p = np.exp(s - lse_safe[:, None])
    p[~nonempty, :] = 0.0
    return p, lse


def full_attention(q, k, v, *, causal: bool = False, scale: Optional[float] = None,
                   q_offset: int = 0, kv_offset: int = 0, row_block: int = 256):
    """Full softmax(scale * Q K^T) V over every key at once -> (o, lse), fp64.

    The definition the method must reproduce exactly: [P2] ``ulysses_attention_forward``
    (softmax over the whole key axis, then multiply by V); [P4] "那么，FlashAttention-2 和
    -3 又改进了什么？" states that the tiled kernels keep this same result.  Rows are processed in
    blocks of ``row_block`` only to bound memory; each row still gets its whole softmax.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, v)
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    o = np.zeros((B, Hq, Sq, D))
    lse = np.full((B, Hq, Sq), NEG_INF)
    qpos_all = q_offset + np.arange(Sq)
    kpos = kv_offset + np.arange(Skv)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, Sq, row_block):
                r1 = min(Sq, r0 + row_block)
                s = _masked_scores(q[b, h, r0:r1], k[b, g], scale,
                                   qpos_all[r0:r1], kpos, causal)
                p, lse_rows = _row_softmax(s)
                o[b, h, r0:r1] = p @ v[b, g]
                lse[b, h, r0:r1] = lse_rows
    return o, lse


def attention_rows(q, k, v, index: Iterable[Tuple[int, int, int]], *, causal: bool = False,
                   scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0):
    """The same definition as ``full_attention`` for selected (b, h, i) rows only.

    Used to check large problems at sampled outputs.  Returns (o [n, D], lse [n]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, v)
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    kpos = kv_offset + np.arange(Skv)
    index = list(index)
    o = np.zeros((len(index), D))
    lse = np.full(len(index), NEG_INF)
    for n, (b, h, i) in enumerate(index):
        g = h // group
        s = _masked_scores(q[b, h, i:i + 1], k[b, g], scale,
                           np.array([q_offset + i]), kpos, causal)
        p, l = _row_softmax(s)
        o[n] = (p @ v[b, g])[0]
        lse[n] = l[0]
    return o, lse


def attention_probs(q, k, *, causal: bool = False, scale: Optional[float] = None,
                    q_offset: int = 0, kv_offset: int = 0) -> np.ndarray:
    """The attention weights P [B, Hq, Sq, Skv] (small problems only)."""
    q, k = _as64(q), _as64(k)
    B, Hq, Sq, D, Hkv, Skv = _shapes(q, k, k)
    scale = _default_scale(scale, D)
    group = Hq // Hkv
    out = np.zeros((B, Hq, Sq, Skv))
    qpos = q_offset + np.arange(Sq)
    kpos = kv_offset + np.arange(Skv)
    for b in range(B):
        for h in range(Hq):
            s = _masked_scores(q[b, h], k[b, h // group], scale, qpos, kpos, causal)
            out[b, h], _ = _row_softmax(s)
    return out


def chunk_bounds(Skv: int, num_chunks: int, c: int) -> Tuple[int, int]:
    """Chunk c of P equal contiguous chunks of the key axis ([P1]: the sequence is
    split into P chunks, one per device)."""
    if num_chunks <= 0 or Skv % num_chunks:
        raise ValueError("Skv must split into num_chunks equal chunks")
    L = Skv // num_chunks
    return c * L, (c + 1) * L


def chunk_partial(q, k, v, c: int, num_chunks: int, *, causal: bool = False,
                  scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0):
    """Partial (o_c, lse_c) of the local queries against key chunk c alone.

    One step of the ring ([P2] ``ring_attention_forward``: the local Q against the
    K/V block currently held).  A chunk with no visible key gives (0, -inf).
    """
    k, v = _as64(k), _as64(v)
    lo, hi = chunk_bounds(k.shape[2], num_chunks, c)
    return full_attention(q, k[:, :, lo:hi], v[:, :, lo:hi], causal=causal, scale=scale,
                          q_offset=q_offset, kv_offset=kv_offset + lo)


def fold_pair(acc, part):
    """One ring step's update: fold a chunk partial into the running (o, lse).

    [P2] ``ring_attention_forward`` carries a running log-sum-exp and replaces the
    running output by the average of the old output and the step's output, weighted
    by their exponentiated log-sum-exps.  Written out with the listing's
    bookkeeping faults removed (the running lse starts at -inf, not 0; the max is
    per row, not over the query axis):

        lse' = log(exp(lse) + exp(lse_c))
        o'   = exp(lse - lse') * o + exp(lse_c - lse') * o_c

    A partial with lse = -inf carries zero weight.
    """
    o_a, lse_a = acc
    o_c, lse_c = part
    m = np.maximum(lse_a, lse_c)
    fin = np.isfinite(m)
    m_safe = np.where(fin, m, 0.0)
    with np.errstate(divide="ignore"):
        lse_new = np.where(fin, m_safe + np.log(np.exp(lse_a - m_safe) + np.exp(lse_c - m_safe)),
                           NEG_INF)
    ref = np.where(fin, lse_new, 0.0)
    w_a = np.where(fin, np.exp(lse_a - ref), 0.0)
    w_c = np.where(fin, np.exp(lse_c - ref), 0.0)
    o_new = w_a[..., None] * o_a + w_c[..., None] * o_c
    return o_new, lse_new


def ring_order(num_chunks: int, start_chunk: int) -> List[int]:
    """Chunk visiting order (start + t) mod P, t = 0 .. P-1 (increasing)."""
    return [(start_chunk + t) % num_chunks for t in range(num_chunks)]


def ring_attention(q, k, v, *, num_chunks: int, start_chunk: int = 0, causal: bool = False,
                   scale: Optional[float] = None, q_offset: int = 0, kv_offset: int = 0):
    """Naive chunk-by-chunk ring attention: one partial per chunk, folded in ring order.

    Every chunk is computed, including ones with no visible key (their (0, -inf)
    partial folds in with zero weight); nothing is skipped or fused.
    """
    q = _as64(q)
    B, Hq, Sq, D = q.shape
    acc = (np.zeros((B, Hq, Sq, D)), np.full((B, Hq, Sq), NEG_INF))
    for c in ring_order(num_chunks, start_chunk):
        part = chunk_partial(q, k, v, c, num_chunks, causal=causal, scale=scale,
                             q_offset=q_offset, kv_offset=kv_offset)
        acc = fold_pair(acc, part)
    return acc


def lse_merge(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """n-way merge of partial (o_i, lse_i) with [P1]'s global statistics.

    [P1] "Ring-Attention：面向大规模部署的工程利器": the global max is the max of the
    local maxima, and the global normaliser Z sums every exponential after shifting
    by that global max.  For partials already normalised by their own lse:

        m_g = max_i lse_i,  Z = sum_i exp(lse_i - m_g),  lse = m_g + ln Z,
        o   = sum_i exp(lse_i - lse) * o_i.

    All partials empty (lse = -inf everywhere) gives (0, -inf).
    """
    if len(o_parts) == 0 or len(o_parts) != len(lse_parts):
        raise ValueError("need matching, non-empty lists of partials")
    L = np.stack([_as64(x) for x in lse_parts])
    O = np.stack([_as64(x) for x in o_parts])
    m_g = L.max(axis=0)
    fin = np.isfinite(m_g)
    m_safe = np.where(fin, m_g, 0.0)
    Z = np.exp(L - m_safe[None]).sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(fin, m_safe + np.log(np.where(fin, Z, 1.0)), NEG_INF)
    ref = np.where(fin, lse, 0.0)
    w = np.where(fin[None], np.exp(L - ref[None]), 0.0)
    o = (w[..., None] * O).sum(axis=0)
    return o, lse


def varlen_attention(q, k, v, cu_seqlens: Sequence[int], *, causal: bool = False,
                     scale: Optional[float] = None):
    """Attention over packed documents -> (o, lse), fp64.

    [P3] "ms-swift长文本训练秘诀：Ulysses并行技术解析", section "5. 实战案例": several short
    samples are packed into one 32K sequence; [P4] section "工程实践中的真实收益" packs
    mixed sequences the same way.  The pages do not state the mask; the reading taken
    here is that every packed sample is its own attention problem: q, k, v are
    [B, H, T, D] token streams, document d holds tokens cu_seqlens[d] .. cu_seqlens[d+1]-1,
    and a query sees exactly the keys of its own document (the ones at or before it when
    ``causal``).  Each document is therefore ``full_attention`` of its own slice, with
    positions counted from the document's first token.  Tokens past the last document see
    no key: o = 0, lse = -inf.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, T, D, Hkv, Tk = _shapes(q, k, v)
    if Tk != T:
        raise ValueError("packed q and k/v must hold the same tokens")
    cu = [int(x) for x in cu_seqlens]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])) or cu[-1] > T:
        raise ValueError("cu_seqlens must start at 0, not decrease and stay within T")
    o = np.zeros((B, Hq, T, D))
    lse = np.full((B, Hq, T), NEG_INF)
    for a, b in zip(cu, cu[1:]):
        if b > a:
            o[:, :, a:b], lse[:, :, a:b] = full_attention(
                q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], causal=causal, scale=scale)
    return o, lse
