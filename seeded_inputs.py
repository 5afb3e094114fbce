"""Seeded synthetic inputs, shared by the oracle-side and the GPU-side checks.

This module holds no attention arithmetic.  It only draws N(0, 1) tensors from
a named seed and rounds them to bfloat16 bit patterns, so that the CPU oracle
and the HIP path can be fed byte-identical inputs.  Neither side imports the
other; both import this.

Recipe (stated once, used everywhere):

* generator: ``numpy.random.Generator(PCG64(seed))``;
* draws: ``standard_normal(shape, dtype=float32)`` for q, k, v, then dO, in
  that order, from one generator;
* bf16 workloads: every float32 draw is rounded to bfloat16 with
  round-to-nearest-even on the bit pattern.  The oracle reads those rounded
  values exactly (bf16 -> fp64 is exact), so input rounding is never counted
  as kernel error.

The workload table describes the shapes of the attention problems measured
and checked (head shapes of a Llama-7B-like model, 32 x 128, and a
Qwen2.5-7B-like GQA model, 28 query / 4 key-value heads x 128, at 8K-32K
context).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "draw",
    "draw_qkv",
    "bf16_bits",
    "bf16_bits_to_f32",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) -> uint16 bits.

    NaN handling is not needed (inputs are finite normal draws).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = u + np.uint64(0x7FFF) + lsb
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """One N(0,1) tensor.  dtype 'f32' -> float32 array; 'bf16' -> uint16 bits."""
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_qkv(seed: int, q_shape, kv_shape, dtype: str, with_dout: bool = False):
    """q, k, v (and dO shaped like q) drawn in that order from one generator."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = draw(rng, q_shape, dtype)
    k = draw(rng, kv_shape, dtype)
    v = draw(rng, kv_shape, dtype)
    if with_dout:
        do = draw(rng, q_shape, dtype)
        return q, k, v, do
    return q, k, v


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact fp64 value of a drawn tensor ('bf16' arrays are bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype and the ring/causal parameters."""

    name: str
    dtype: str                      # 'f32' or 'bf16'
    q_shape: Tuple[int, int, int, int]   # [B, Hq, Sq, D]
    kv_shape: Tuple[int, int, int, int]  # [B, Hkv, Skv, D]
    causal: bool
    num_chunks: int = 1
    start_chunk: int = 0
    q_offset: int = 0
    kv_offset: int = 0
    scale: Optional[float] = None   # None -> 1/sqrt(D)
    seed: int = 0
    # Ulysses layout step (sequence-sharded <-> head-sharded), if any
    ulysses_P: int = 0
    ulysses_rank: int = 0
    backward: bool = False
    # packed documents (cu_seqlens drawn by draw_doc_offsets from this workload's seed)
    packed_docs: bool = False
    # inputs quantized to e4m3 with one scale per (batch, head) before the attention
    fp8: bool = False


def draw_doc_offsets(seed: int, total: int, median: int = 2048, sigma: float = 1.0,
                     lo: int = 64, hi: int = 16384) -> list:
    """Document boundaries of a packed token stream: lengths log-normal around `median`
    (clipped to [lo, hi]) drawn until `total` tokens are covered, the last one cut to
    fit.  Returns cu_seqlens = [0, end_0, end_1, ..., total]."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    cu = [0]
    while cu[-1] < total:
        n = int(np.clip(round(float(rng.lognormal(np.log(median), sigma))), lo, hi))
        cu.append(min(total, cu[-1] + n))
    return cu


# The workloads.  Seeds are 1000 + workload number.
WORKLOADS: Dict[str, Workload] = {
    "ring_tiny_f32": Workload(
        name="ring_tiny_f32", dtype="f32",
        q_shape=(1, 2, 256, 64), kv_shape=(1, 2, 256, 64),
        causal=False, num_chunks=4, start_chunk=1, seed=1001),
    "llama7b_causal_8k": Workload(
        name="llama7b_causal_8k", dtype="bf16",
        q_shape=(1, 32, 8192, 128), kv_shape=(1, 32, 8192, 128),
        causal=True, seed=1002),
    "ring8_rank3_32k": Workload(
        name="ring8_rank3_32k", dtype="bf16",
        q_shape=(1, 32, 4096, 128), kv_shape=(1, 32, 32768, 128),
        causal=True, num_chunks=8, start_chunk=3, q_offset=3 * 4096, seed=1003),
    "qwen7b_ulysses4_rank0_32k": Workload(
        name="qwen7b_ulysses4_rank0_32k", dtype="bf16",
        q_shape=(1, 7, 32768, 128), kv_shape=(1, 1, 32768, 128),
        causal=True, seed=1004, ulysses_P=4, ulysses_rank=0),
    "qwen7b_packed_32k": Workload(
        name="qwen7b_packed_32k", dtype="bf16",
        q_shape=(1, 28, 32768, 128), kv_shape=(1, 4, 32768, 128),
        causal=True, seed=1006, packed_docs=True),
    "qwen7b_packed_bwd_32k": Workload(
        name="qwen7b_packed_bwd_32k", dtype="bf16",
        q_shape=(1, 28, 32768, 128), kv_shape=(1, 4, 32768, 128),
        causal=True, seed=1006, packed_docs=True, backward=True),
    "ring8_rank3_bwd_32k": Workload(
        name="ring8_rank3_bwd_32k", dtype="bf16",
        q_shape=(1, 32, 4096, 128), kv_shape=(1, 32, 32768, 128),
        causal=True, num_chunks=8, start_chunk=3, q_offset=3 * 4096, seed=1007, backward=True),
    "qwen7b_gqa_32k_fp8": Workload(
        name="qwen7b_gqa_32k_fp8", dtype="bf16",
        q_shape=(1, 7, 32768, 128), kv_shape=(1, 1, 32768, 128),
        causal=True, seed=1008, fp8=True),
    "llama7b_causal_bwd_16k": Workload(
        name="llama7b_causal_bwd_16k", dtype="bf16",
        q_shape=(1, 32, 16384, 128), kv_shape=(1, 32, 16384, 128),
        causal=True, seed=1005, backward=True),
}

# Ulysses source layout of the GQA workload: 4 sequence shards of 8192 tokens,
# [P, S/P, H, D] with 28 query heads and 4 key-value heads.
ULYSSES_SRC = {
    "q": (4, 8192, 28, 128),
    "kv": (4, 8192, 4, 128),
}


def draw_ulysses_sources(seed: int):
    """Sequence-sharded q, k, v sources ([P, S/P, H, D] bf16 bits), in order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = draw(rng, ULYSSES_SRC["q"], "bf16")
    k = draw(rng, ULYSSES_SRC["kv"], "bf16")
    v = draw(rng, ULYSSES_SRC["kv"], "bf16")
    return q, k, v
