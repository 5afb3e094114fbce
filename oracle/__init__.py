"""CPU oracle for exact blockwise (ring) softmax attention -- TEST INFRASTRUCTURE.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The GPU path (``long_context_exact_tiled_amd``) never imports it,
and it never imports the GPU path: the two share no code.  The only shared
module is ``seeded_inputs``, which draws inputs and holds no attention
arithmetic.

Everything is plain NumPy in float64, computed from the definitions the pages
give, in the order they give them.  Sources (page title, then the section):

* [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn),
  section "Ring-Attention：面向大规模部署的工程利器" -- the per-chunk local max
  m_i, local exponential sum z_i, the global max and the global normaliser Z.
* [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com) -- the
  ``ulysses_attention_forward`` listing (local Q against the gathered K/V,
  softmax then matmul, scale 1/sqrt(head dim), K/V concatenated on the
  sequence axis of [B, H, L, D]) and the ``ring_attention_forward`` listing
  (per-step log-sum-exp carry and a weighted average of the running output
  with the step's output).
* [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn),
  sections "FlashAttention 如何破局？不只是融合内核" (tiling with an online
  running max and normaliser, only the output written back), "那么，
  FlashAttention-2 和 -3 又改进了什么？" (the speed-ups keep the results
  numerically identical to plain attention) and
  "Ulysses：强互联下的高速通路" (sequence shards [B, S_local] x N, an
  all-to-all before attention and one after that restores the order), and
  "工程实践中的真实收益" (packing mixed sequences into one).
* [P3] "ms-swift长文本训练秘诀：Ulysses并行技术解析" (bxzpzcl.cn), section
  "5. 实战案例" -- short samples packed into a single 32K sequence.

Module map:

* ``attention``  -- full softmax attention (the definition), per-chunk
  partials, the pairwise ring fold, the n-way LSE merge, and attention over
  packed documents (each document its own problem).
* ``permute``    -- the Ulysses sequence-shard <-> head-shard layout step.
* ``backward``   -- the textbook softmax-attention gradient (the pages only
  say the backward recomputes from saved statistics; the formulas are not on
  them), whole or chunk by chunk in ring order for one device's query block,
  and over packed documents.  Pinned by finite differences in ``tests/``.
* ``fp8``        -- the e4m3 code (OCP definition), the per-head scaling rule,
  attention over dequantized fp8 inputs, and the derived bound on the error of
  rounding the attention weights to e4m3.  Pinned against torch's float8_e4m3fn
  conversion, the format's defining values and a simulation of the rounding.

Parity status: every function here is pinned by ``-m "not gpu"`` tests
(brute force, closed forms, invariants, a library routine, finite
differences); none is "parity unpinned".
"""
from .attention import (  # noqa: F401
    full_attention,
    attention_rows,
    attention_probs,
    chunk_partial,
    ring_attention,
    fold_pair,
    lse_merge,
    varlen_attention,
)
from .permute import seq_to_head, head_to_seq  # noqa: F401
from .backward import (  # noqa: F401
    attention_bwd,
    attention_bwd_heads,
    ring_attention_bwd,
    varlen_attention_bwd,
)
from . import fp8  # noqa: F401,E402
