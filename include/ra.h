/*
 * ra.h -- C ABI of libra: exact blockwise (ring) softmax attention on MI355X (gfx950).
 *
 * Sources (page title, host), cited by section below:
 *   [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn)
 *   [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com)
 *   [P3] "ms-swift长文本训练秘诀：Ulysses并行技术解析" (bxzpzcl.cn)
 *   [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn)
 *
 * General rules for every entry point
 * -----------------------------------
 * - Tensors are described by ra_tensor: a device pointer, a dtype, a rank and
 *   per-axis shape and stride counted in ELEMENTS.  The innermost stride must be 1.
 *   Every data pointer must be 16-byte aligned and every outer stride must be a
 *   whole number of 16-byte units (rows are moved with 16-byte vector accesses).
 * - Token strides of attention operands ([B, H, S, D] tensors of the attention entry
 *   points): the kernels move tiles of up to 128 tokens and form a byte offset within
 *   a tile in 32 bits, so (min(128, S) - 1) * stride[2] + D, in bytes, must stay below
 *   2^31 (about 8.4 M bf16 elements of token stride); otherwise RA_ERR_SHAPE.  Batch
 *   and head strides are not limited.
 * - The caller owns and allocates every buffer (inputs, outputs, workspace).  The
 *   library allocates nothing, keeps no global state and never synchronises; the one
 *   exception is ra_attn_bwd_noalloc, whose workspace is a fixed array of the loaded
 *   module (see there).
 * - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).  Outputs
 *   are valid once the stream's work has completed.  Inputs must stay alive and
 *   unmodified until then.  Calls are thread-safe.
 * - The return value is a ra_status.  Argument errors (negative codes other than
 *   RA_ERR_HIP) are detected on the host before anything is enqueued, so nothing is
 *   written on error.  RA_ERR_HIP reports a failed kernel launch.  No C++ exception
 *   crosses this boundary.
 * - The *_validate functions run the same host-side checks without touching the
 *   device, so they can be called on a machine with no GPU.
 */
#ifndef RA_H_
#define RA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_VERSION 100 /* 0.1.0 */
#define RA_MAX_MERGE_PARTS 64
#define RA_MAX_PERMUTE_TENSORS 4
#define RA_MAX_QUANT_TENSORS 4
#define RA_MAX_DOCS (1 << 24)

typedef enum {
  RA_OK = 0,
  RA_ERR_NULL = -1,        /* a required pointer is NULL */
  RA_ERR_DTYPE = -2,       /* dtype not allowed for this argument or mismatched */
  RA_ERR_SHAPE = -3,       /* ranks or extents inconsistent */
  RA_ERR_STRIDE = -4,      /* innermost stride != 1, negative/overlapping strides */
  RA_ERR_ALIGN = -5,       /* pointer or stride not a multiple of 16 bytes */
  RA_ERR_RANGE = -6,       /* a scalar parameter out of range */
  RA_ERR_UNSUPPORTED = -7, /* valid request this build does not implement */
  RA_ERR_HIP = -8,         /* kernel launch failed */
  RA_ERR_WORKSPACE = -9,   /* workspace missing or smaller than required */
  RA_ERR_SCRATCH = -10     /* needs more than ra_attn_bwd_noalloc's fixed scratch */
} ra_status;

typedef enum { RA_F32 = 0, RA_BF16 = 1, RA_FP8_E4M3 = 2 /* OCP e4m3, 1 byte */ } ra_dtype;

typedef struct {
  void *data;        /* device pointer, 16-byte aligned */
  int32_t dtype;     /* ra_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];  /* extents of the first ndim axes */
  int64_t stride[4]; /* element strides; stride[ndim-1] must be 1 */
} ra_tensor;

typedef struct {
  uint32_t struct_size; /* sizeof(ra_attn_params); lets the struct grow */
  int32_t causal;       /* 0: every key visible; 1: key j visible to query i iff
                           kv_offset + j <= q_offset + i (global positions) */
  int32_t num_chunks;   /* P >= 1: the key axis is split into P equal chunks */
  int32_t start_chunk;  /* first chunk visited; order (start + t) mod P */
  int64_t q_offset;     /* global position of query row 0 (>= 0) */
  int64_t kv_offset;    /* global position of key row 0 (>= 0) */
  float scale;          /* score scale; <= 0 selects 1/sqrt(D) */
  /* Optional (present when struct_size >= RA_ATTN_PARAMS_SIZE_V2): DEVICE pointer to a
   * uint64 work counter, 8-byte aligned and zero before its first use, or NULL.  The
   * forward kernels (ra_attn_fwd and ra_attn_fwd_varlen on bf16, ra_attn_fwd_fp8) use it
   * when B * Hq is not a multiple of 8: each workgroup then takes the next query tile from the counter when
   * it starts, heaviest first, so XCDs that run faster take more tiles (the launch
   * places workgroups on XCDs in a fixed round-robin order, and XCD speeds differ).
   * Every call leaves the counter as it found it.  Results never depend on the
   * counter's value; the tile order does (zero gives heaviest first).  Calls that share
   * a counter must not overlap in time: use one counter per stream.  Other entry points,
   * and shapes with B * Hq a multiple of 8, do not touch it; every call that takes
   * ra_attn_params rejects a non-NULL counter that is not 8-byte aligned
   * (RA_ERR_ALIGN).  NULL: the fixed order. */
  uint64_t *sched;
} ra_attn_params;

/* struct_size of ra_attn_params without / with the sched field; both are accepted. */
#define RA_ATTN_PARAMS_SIZE_V1 40
#define RA_ATTN_PARAMS_SIZE_V2 48

typedef void *ra_stream; /* a hipStream_t */

/*
 * ra_attn_fwd -- exact softmax attention of a local query block over P key/value
 * chunks visited in ring order, carrying the running row max and exponential sum
 * (log-sum-exp) from chunk to chunk.
 *
 * Defines: o = softmax(scale * q k^T) v over the visible keys, lse = natural log of
 * the row's sum of exp(scale * q k^T).  [P2] listing ulysses_attention_forward (the
 * full softmax of a local Q against every key, scale 1/sqrt(head dim), [B,H,L,D]
 * layout); [P2] listing ring_attention_forward and [P1] section
 * "Ring-Attention：面向大规模部署的工程利器" (a device holds one chunk at a time,
 * visits all P chunks and folds each into log-space running statistics); [P4]
 * section "FlashAttention 如何破局？不只是融合内核" (tiles on chip, online max and
 * normaliser, only the output written back).  Causal masking and grouped heads are
 * not on the pages; their meaning is fixed by ra_attn_params above and the mapping
 * below.
 *
 * q   [B, Hq, Sq, D]   RA_F32 or RA_BF16
 * k,v [B, Hkv, Skv, D] same dtype as q; Hq % Hkv == 0; query head h reads
 *                      key/value head h / (Hq / Hkv); Skv % num_chunks == 0
 * o   [B, Hq, Sq, D]   dtype of q, or RA_F32 (e.g. partials for ra_lse_merge)
 * lse [B, Hq, Sq]      RA_F32
 * D must be 64 or 128 (else RA_ERR_UNSUPPORTED).  A row with no visible key gets
 * o = 0 and lse = -inf.  Sq == 0 or B*Hq == 0 is a no-op.  o must not overlap q, k, v.
 * Chunks with no visible key (causal) are skipped; skipping is exact.
 * Deterministic: the same inputs give bitwise the same outputs.
 */
int ra_attn_fwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                const ra_attn_params *p, ra_tensor *o, ra_tensor *lse, ra_stream stream);
int ra_attn_fwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         const ra_attn_params *p, const ra_tensor *o, const ra_tensor *lse);

/*
 * ra_attn_fwd_varlen -- ra_attn_fwd over packed documents: several sequences laid end
 * to end in one token stream, each its own attention problem.
 *
 * [P3] "ms-swift长文本训练秘诀：Ulysses并行技术解析", section "5. 实战案例" (short samples
 * packed into one 32K sequence) and [P4] section "工程实践中的真实收益" (mixed sequences
 * packed the same way).  The pages do not state the mask; here a query sees exactly the
 * keys of its own document (with p->causal, those at or before it).
 *
 * q   [B, Hq, T, D]  RA_BF16; k, v [B, Hkv, T, D] (the same T tokens); D 64 or 128
 * cu_seqlens  DEVICE pointer to n_docs + 1 int32 (4-byte aligned), read by the kernel:
 *             document d holds tokens cu_seqlens[d] .. cu_seqlens[d+1] - 1; the same
 *             packing for every batch entry.  Must start at 0, not decrease and not
 *             exceed T; tokens at or past cu_seqlens[n_docs] see no key (o = 0,
 *             lse = -inf).  Values breaking these rules give unspecified results but
 *             no access outside q, k, v, o, lse and the n_docs + 1 entries.
 * 1 <= n_docs <= RA_MAX_DOCS.  p: causal and scale apply; num_chunks must be 1 and
 * start_chunk, q_offset, kv_offset 0 (else RA_ERR_RANGE).  o: bf16 or RA_F32; lse fp32.
 * The caller owns every buffer; nothing is allocated; work is enqueued on `stream`.
 */
int ra_attn_fwd_varlen(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                       const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                       ra_tensor *o, ra_tensor *lse, ra_stream stream);
int ra_attn_fwd_varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                const int32_t *cu_seqlens, int32_t n_docs,
                                const ra_attn_params *p, const ra_tensor *o,
                                const ra_tensor *lse);

/*
 * ra_lse_merge -- combine n partial results (o_i, lse_i) of the same queries over
 * disjoint key sets into the result over their union.
 *
 * Defines ([P1] section "Ring-Attention：面向大规模部署的工程利器": global max of the
 * local maxima, then the global normaliser Z of all exponentials shifted by it):
 *   m = max_i lse_i, lse = m + ln sum_i exp(lse_i - m), o = sum_i exp(lse_i - lse) o_i.
 * A partial with lse = -inf has weight 0; if all are -inf the row gets o = 0,
 * lse = -inf.
 *
 * o_parts   array of n tensors [B, H, S, D], RA_F32 or RA_BF16, all the same shape,
 *           dtype and strides
 * lse_parts array of n tensors [B, H, S], RA_F32, all the same strides
 * o         [B, H, S, D] RA_F32 or RA_BF16;  lse [B, H, S] RA_F32
 * 1 <= n <= RA_MAX_MERGE_PARTS.  o (lse) may be the very same view as one of the
 * o_parts (lse_parts) -- in place; any other overlap is undefined.  D: any multiple of
 * 8 up to 256.
 */
int ra_lse_merge(int32_t n, const ra_tensor *o_parts, const ra_tensor *lse_parts, ra_tensor *o,
                 ra_tensor *lse, ra_stream stream);
int ra_lse_merge_validate(int32_t n, const ra_tensor *o_parts, const ra_tensor *lse_parts,
                          const ra_tensor *o, const ra_tensor *lse);

/*
 * ra_ulysses_permute -- the local layout step of Ulysses sequence parallelism:
 * sequence shards <-> head shards (a pure element move, bit-exact).
 *
 * [P4] section "Ulysses：强互联下的高速通路": the sequence is cut into per-device
 * shards [B, S_local] x N; an all-to-all before attention gives each device the
 * whole sequence, another after it restores the output's sequence order.  Which
 * axis is traded is not on the pages; here it is the head axis.
 *
 * dir = 0 (sequence -> head):
 *   src [P, S/P, H, D]  (shard s, token t of the shard, head, dim)
 *   dst [H/P, S, D]     heads rank*H/P .. of the whole sequence, tokens in shard
 *                       order: dst[h', s*(S/P) + t, :] = src[s, t, rank*H/P + h', :]
 *   rank = -1 does every rank at once: dst [P, H/P, S, D].
 * dir = 1 (head -> sequence): the inverse; src is [H/P, S, D] (or [P, H/P, S, D] with
 *   rank = -1) and only the head slice of `rank` in dst [P, S/P, H, D] is written.
 * H % P == 0; src and dst have the same dtype (RA_F32 or RA_BF16) and must not
 * overlap; D * element size must be a multiple of 16 bytes.
 */
int ra_ulysses_permute(const ra_tensor *src, ra_tensor *dst, int32_t P, int32_t rank, int32_t dir,
                       ra_stream stream);
int ra_ulysses_permute_validate(const ra_tensor *src, const ra_tensor *dst, int32_t P, int32_t rank,
                                int32_t dir);

/*
 * ra_ulysses_permute_n -- ra_ulysses_permute of n (src, dst) pairs in one launch, e.g. the
 * q, k and v of one layer before attention (the same section of [P4]: one all-to-all
 * carries all of a layer's inputs; here one kernel packs them).
 *
 * srcs, dsts: arrays of n descriptors; pair i is exactly ra_ulysses_permute(&srcs[i],
 * &dsts[i], P, rank, dir) and is validated as such (pairs may differ in head count, e.g.
 * 28 query and 4 key/value heads, in dtype and in head dim).  No destination may overlap
 * any source or another destination.  1 <= n <= RA_MAX_PERMUTE_TENSORS (else
 * RA_ERR_RANGE).  Pairs whose rows (D * element size) are all 128, 256 or 512 bytes of
 * one size move in a single launch; otherwise pair by pair.  Bit-exact.
 */
int ra_ulysses_permute_n(int32_t n, const ra_tensor *srcs, ra_tensor *dsts, int32_t P, int32_t rank,
                         int32_t dir, ra_stream stream);
int ra_ulysses_permute_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts,
                                  int32_t P, int32_t rank, int32_t dir);

/*
 * ra_attn_bwd -- gradients dq, dk, dv of L = sum(dout * o) for the attention of
 * ra_attn_fwd, recomputing the attention weights from the saved lse instead of
 * storing them ([P4] section "为什么传统注意力这么“吃”显存？": the backward pass either
 * keeps the intermediates or recomputes them).  The gradient formulas are the
 * textbook ones (not on the pages): P = exp(scale q k^T - lse), D_i = rowsum(dout*o),
 * dv = P^T dout, dS = P * (dout v^T - D), dq = scale dS k, dk = scale dS^T q; with
 * grouped heads dk, dv sum over the query heads of a group.
 *
 * q, o, dout [B, Hq, Sq, D]; k, v [B, Hkv, Skv, D]; all RA_BF16 or all RA_F32 (fp32
 * inputs run fp32 MFMAs throughout); D 64 or 128; lse [B, Hq, Sq] RA_F32 from
 * ra_attn_fwd with the same p.  dq like q, dk and dv like k, same dtype as q.  The ring parameters
 * fix the order in which dq accumulates over chunks.  Outputs must not overlap the
 * inputs.  workspace: device memory of at least ra_attn_bwd_workspace_size bytes,
 * 256-byte aligned, overwritten: the D_i rows (B * Hq * Sq fp32), and with bf16 grouped
 * heads (Hq > Hkv) also one fp32 dk and dv partial per query head (2 * B * Hq * Skv * D
 * fp32), summed over each group in head order after the per-head passes.
 * Deterministic.
 */
int ra_attn_bwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, const ra_tensor *o,
                const ra_tensor *dout, const ra_tensor *lse, const ra_attn_params *p,
                ra_tensor *dq, ra_tensor *dk, ra_tensor *dv, void *workspace,
                size_t workspace_bytes, ra_stream stream);
int ra_attn_bwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                         const ra_attn_params *p, const ra_tensor *dq, const ra_tensor *dk,
                         const ra_tensor *dv);
/* Bytes of workspace ra_attn_bwd needs for these shapes and dtype (0 if the shapes are
 * invalid): see ra_attn_bwd's workspace. */
size_t ra_attn_bwd_workspace_size(const ra_tensor *q, const ra_tensor *k, const ra_attn_params *p);

/*
 * ra_attn_bwd_noalloc -- ra_attn_bwd without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc).
 *
 * Same arguments (minus workspace), checks and errors as ra_attn_bwd, and the same
 * results, except that with bf16 grouped heads dk and dv are summed over the group
 * inside each workgroup (ra_attn_bwd sums per-head partials from its workspace): the
 * same sums in another fp32 order, not bitwise equal.  It runs on the CURRENT device
 * (the stream must belong to it).  Its workspace is a fixed device array inside the
 * library, RA_NOALLOC_SCRATCH_BYTES per GPU, held from library load until the process
 * ends; a problem whose D_i rows (B * Hq * Sq fp32) exceed it returns RA_ERR_SCRATCH
 * with nothing enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined gradients; calls in one stream's order are safe.
 * No hipMalloc, hipFree or allocating library routine is called (the first call on a
 * device looks up the array's device address once).
 */
#define RA_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB: B * Hq * Sq up to 8 M query rows */
int ra_attn_bwd_noalloc(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                        const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                        const ra_attn_params *p, ra_tensor *dq, ra_tensor *dk, ra_tensor *dv,
                        ra_stream stream);
/* RA_NOALLOC_SCRATCH_BYTES of the loaded library. */
size_t ra_noalloc_scratch_bytes(void);

/*
 * ra_attn_bwd_varlen -- ra_attn_bwd over packed documents (the gradients of
 * ra_attn_fwd_varlen): each document's queries, keys and values get the gradients of
 * that document's own attention problem; tokens in no document get zero gradients.
 *
 * Same sources and reading as ra_attn_fwd_varlen ([P3] section "5. 实战案例", [P4]
 * section "工程实践中的真实收益"; the backward formulas are the textbook softmax
 * gradient, recomputing P from lse).  Tensors, dtypes, workspace and errors as for
 * ra_attn_bwd (bf16 only, like the packed forward; D 64 or 128, workspace from ra_attn_bwd_workspace_size with
 * num_chunks = 1); q, k, v, o, dout hold the same T tokens; cu_seqlens, n_docs and the
 * params restrictions as for ra_attn_fwd_varlen; o and lse must come from
 * ra_attn_fwd_varlen with the same cu_seqlens.
 */
int ra_attn_bwd_varlen(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                       const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                       const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                       ra_tensor *dq, ra_tensor *dk, ra_tensor *dv, void *workspace,
                       size_t workspace_bytes, ra_stream stream);
int ra_attn_bwd_varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                                const int32_t *cu_seqlens, int32_t n_docs,
                                const ra_attn_params *p, const ra_tensor *dq, const ra_tensor *dk,
                                const ra_tensor *dv);

/*
 * ra_attn_bwd_accum -- one device's step of the ring backward: the gradient
 * contributions of its query block against one key/value chunk, ADDED to fp32
 * accumulators.
 *
 * [P1] section "Ring-Attention：面向大规模部署的工程利器": gradients travel back
 * along the ring the way the blocks came.  Reading taken: at every step the device
 * recomputes P = exp(scale q k_c^T - lse) against the chunk it holds, with lse (and o)
 * the forward's result merged over every chunk; its dq accumulator stays with it and
 * sums over the chunks; the chunk's dk/dv accumulators travel with the chunk and sum
 * over the devices.  Formulas as for ra_attn_bwd, restricted to the chunk.
 *
 * q, o, dout [B, Hq, Sq, D]; k, v [B, Hkv, Skv, D], the chunk only; all RA_BF16 or all
 * RA_F32; lse [B, Hq, Sq] RA_F32, the merged forward lse of this block; D 64 or 128.
 * dq_acc [B, Hq, Sq, D], dk_acc and dv_acc [B, Hkv, Skv, D]: RA_F32, read and
 * updated in place (acc += contribution); the caller zeroes them before the first
 * step.  p: causal, scale and the global positions q_offset (first query) and
 * kv_offset (first key of the chunk); num_chunks must be 1 and start_chunk 0
 * (RA_ERR_RANGE otherwise).  A causal chunk whose first key follows the block's last
 * query adds nothing and returns RA_OK with no work enqueued.  workspace as for
 * ra_attn_bwd (D_i is recomputed on every call).  Accumulators must not overlap each
 * other or the inputs; steps on one stream accumulate in stream order
 * (deterministic, no atomics).
 */
int ra_attn_bwd_accum(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                      const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                      const ra_attn_params *p, ra_tensor *dq_acc, ra_tensor *dk_acc,
                      ra_tensor *dv_acc, void *workspace, size_t workspace_bytes,
                      ra_stream stream);
int ra_attn_bwd_accum_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                               const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                               const ra_attn_params *p, const ra_tensor *dq_acc,
                               const ra_tensor *dk_acc, const ra_tensor *dv_acc);

/*
 * ra_fp8_quantize -- bf16 -> e4m3 codes with one fp32 scale per (batch, head), the
 * input of ra_attn_fwd_fp8.
 *
 * [P4] section "那么，FlashAttention-2 和 -3 又改进了什么？": FlashAttention-3 supports
 * the FP8 data type, halving key/value traffic.  The scaling rule is a reading (the pages
 * give none): with a = max |x| over the head, code = e4m3(clamp(x * (448 / a), -448,
 * 448)), an fp32 multiply and a round-to-nearest-even conversion to OCP e4m3;
 * descale = a / 448 (fp32); an all-zero head gets descale 1 and zero codes.  The value
 * of a code is decode(code) * descale.
 *
 * src     [B, H, S, D] RA_BF16, D a multiple of 16 and at most 256
 * dst     RA_FP8_E4M3: [B, H, S, D] (transpose = 0), or [B, H, D, S_pad] with
 *         S_pad = S rounded up to 16 (transpose = 1: tokens contiguous, the layout of
 *         ra_attn_fwd_fp8's vt; tokens S .. S_pad-1 get code 0)
 * descale [B, H] RA_F32, written
 * workspace: device memory of at least ra_fp8_quantize_workspace_size bytes, 256-byte
 * aligned, overwritten.  Non-finite inputs give unspecified codes.  Deterministic.
 */
int ra_fp8_quantize(const ra_tensor *src, ra_tensor *dst, ra_tensor *descale, int32_t transpose,
                    void *workspace, size_t workspace_bytes, ra_stream stream);
int ra_fp8_quantize_validate(const ra_tensor *src, const ra_tensor *dst,
                             const ra_tensor *descale, int32_t transpose);
/* Bytes of workspace ra_fp8_quantize needs for src (0 if src is invalid). */
size_t ra_fp8_quantize_workspace_size(const ra_tensor *src);

/*
 * ra_fp8_quantize_n -- ra_fp8_quantize of n tensors (1 <= n <= RA_MAX_QUANT_TENSORS; q, k
 * and v of a layer, each with its own transpose flag) in two launches instead of 2n.
 * Each tensor's codes and descales are those ra_fp8_quantize gives it.  srcs, dsts,
 * descales: arrays of n descriptors; transpose: n flags.  No destination (codes or
 * descales) may overlap a source or another destination (RA_ERR_STRIDE).  workspace:
 * at least ra_fp8_quantize_n_workspace_size bytes, 256-byte aligned, overwritten.
 * Errors as for ra_fp8_quantize, and RA_ERR_RANGE for n outside 1..4.
 */
int ra_fp8_quantize_n(int32_t n, const ra_tensor *srcs, ra_tensor *dsts, ra_tensor *descales,
                      const int32_t *transpose, void *workspace, size_t workspace_bytes,
                      ra_stream stream);
int ra_fp8_quantize_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts,
                               const ra_tensor *descales, const int32_t *transpose);
/* Bytes of workspace ra_fp8_quantize_n needs for these sources (0 if any is invalid). */
size_t ra_fp8_quantize_n_workspace_size(int32_t n, const ra_tensor *srcs);

/*
 * ra_attn_fwd_fp8 -- ra_attn_fwd over e4m3 inputs: exact softmax attention of the
 * dequantized q, k, v (value = decode(code) * descale of its (batch, head)), the same
 * ring walk, causal mask and outputs.
 *
 * [P4] sections "那么，FlashAttention-2 和 -3 又改进了什么？" (FlashAttention-3's FP8
 * support) and "FlashAttention 如何破局？不只是融合内核" (tiling and the online
 * softmax); ring and merge sources as ra_attn_fwd.  The attention
 * weights are rounded to e4m3 for the P V product (after scaling by 2^6); the row sums
 * and lse use the unrounded fp32 weights.
 *
 * q   [B, Hq, Sq, D] RA_FP8_E4M3;  k [B, Hkv, Skv, D] RA_FP8_E4M3;  D 64 or 128
 * vt  [B, Hkv, D, S_pad] RA_FP8_E4M3, V transposed (tokens contiguous), S_pad = Skv
 *     rounded up to 16, rows 16-byte aligned; columns Skv .. S_pad-1 are read and must
 *     hold finite codes (ra_fp8_quantize writes 0 there)
 * q_descale [B, Hq], k_descale and v_descale [B, Hkv]: RA_F32, finite and > 0
 * p   as for ra_attn_fwd;  o [B, Hq, Sq, D] RA_BF16 or RA_F32;  lse [B, Hq, Sq] RA_F32
 *     With num_chunks > 1 the chunk length Skv / num_chunks must be a multiple of 16
 *     keys (RA_ERR_ALIGN otherwise): key tiles then start on 16-byte boundaries of vt's
 *     rows, as a chunk-by-chunk call's vt view must (its data pointer is 16-byte aligned).
 * Errors as for ra_attn_fwd; RA_ERR_SHAPE also when one head's byte offsets exceed
 * 2^31.  Outputs must not overlap the inputs.
 */
int ra_attn_fwd_fp8(const ra_tensor *q, const ra_tensor *k, const ra_tensor *vt,
                    const ra_tensor *q_descale, const ra_tensor *k_descale,
                    const ra_tensor *v_descale, const ra_attn_params *p, ra_tensor *o,
                    ra_tensor *lse, ra_stream stream);
int ra_attn_fwd_fp8_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *vt,
                             const ra_tensor *q_descale, const ra_tensor *k_descale,
                             const ra_tensor *v_descale, const ra_attn_params *p,
                             const ra_tensor *o, const ra_tensor *lse);

/* Static message for a status code (never NULL). */
const char *ra_status_string(int status);
/* RA_VERSION of the loaded library. */
int ra_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RA_H_ */
