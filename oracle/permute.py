"""Oracle: the Ulysses layout step, sequence shards <-> head shards (bit-exact).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import it.

[P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效", section "Ulysses：强互联下的高速通路":
the input sequence is cut into N per-device shards [B, S_local]; an all-to-all runs
before attention so each device can attend over the whole sequence, and a second
all-to-all after attention restores the sequence order of the output.  The pages
do not say which axis the all-to-all trades the sequence for; the reading taken
(listed in the design doc) is the head axis: a device gives up its sequence shard of
every head and receives the full sequence of H/P heads.  [P2] "Ulysses与Ring-Attention
序列并行技术详解" mentions splitting attention heads across devices when combined
with tensor parallelism, which is the same axis.

Layouts:

* sequence-sharded source: ``src[s, t, h, d]`` = token t of shard s (global token
  s * S_local + t), head h -- shape [P, S/P, H, D];
* head-sharded destination of rank r: ``dst[h', j, d]`` = head r * H/P + h', global
  token j -- shape [H/P, S, D].  All ranks at once: [P, H/P, S, D].

Both directions are pure element moves; the arrays may be any dtype (tests use
uint16 bit patterns, so equality is bitwise).
"""
from __future__ import annotations

import numpy as np


def seq_to_head(src: np.ndarray, P: int, rank: int) -> np.ndarray:
    """[P, S/P, H, D] -> [H/P, S, D] for ``rank``, or [P, H/P, S, D] for rank = -1."""
    if src.ndim != 4 or src.shape[0] != P:
        raise ValueError("src must be [P, S/P, H, D]")
    _, Sl, H, D = src.shape
    if H % P:
        raise ValueError("H must be a multiple of P")
    Hl = H // P
    if rank == -1:
        return np.stack([seq_to_head(src, P, r) for r in range(P)])
    if not 0 <= rank < P:
        raise ValueError("rank out of range")
    heads = src[:, :, rank * Hl:(rank + 1) * Hl, :]          # [P, Sl, Hl, D]
    # token order: shard-major then position within the shard
    return np.ascontiguousarray(heads.transpose(2, 0, 1, 3).reshape(Hl, P * Sl, D))


def head_to_seq(src: np.ndarray, P: int, rank: int, out: np.ndarray) -> np.ndarray:
    """Inverse of ``seq_to_head``: write a head shard back into ``out`` [P, S/P, H, D].

    ``src`` is [H/P, S, D] for one rank, or [P, H/P, S, D] for rank = -1.  Only the
    head slice of ``rank`` is written; the rest of ``out`` is left as it was.
    """
    if out.ndim != 4 or out.shape[0] != P:
        raise ValueError("out must be [P, S/P, H, D]")
    _, Sl, H, D = out.shape
    Hl = H // P
    if rank == -1:
        for r in range(P):
            head_to_seq(src[r], P, r, out)
        return out
    if src.shape != (Hl, P * Sl, D):
        raise ValueError("src must be [H/P, S, D]")
    out[:, :, rank * Hl:(rank + 1) * Hl, :] = src.reshape(Hl, P, Sl, D).transpose(1, 2, 0, 3)
    return out
