// Internal (non-exported) interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

constexpr float kLog2eHost = 1.4426950408889634f;

// Kernels that move [rows, D] tiles straight from global memory into LDS form each
// lane's byte offset within a tile in 32 bits.  No tile has more rows than this, so the
// host accepts a token stride only if (min(kMaxTileRows, S) - 1) * stride + D elements
// stay below 2^31 bytes.
constexpr int kMaxTileRows = 128;

// Forward attention problem after validation: raw pointers and element strides.
struct FwdArgs {
  const void *q;
  const void *k;
  const void *v;
  void *o;
  float *lse;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t l_sb, l_sh;
  int32_t B, Hq, Hkv, Sq, Skv;
  int32_t group;        // Hq / Hkv
  int32_t num_chunks;   // P
  int32_t start_chunk;
  int32_t chunk_len;    // Skv / P
  int32_t num_q_tiles;
  int64_t q_offset, kv_offset;
  float scale_log2;     // scale * log2(e)
  int32_t o_is_f32;     // output dtype: 1 = fp32, 0 = same as inputs (bf16 path)
  // packed documents (attn_fwd_varlen only): document d holds tokens cu[d] .. cu[d+1]-1
  const int32_t *cu;
  int32_t n_docs;
  // work counter (bf16 direct kernel, B*Hq not a multiple of 8): NULL = fixed tile order
  uint64_t *sched;
};

int launch_attn_fwd(const FwdArgs &a, int dtype, int D, int causal, hipStream_t stream);
int launch_attn_fwd_varlen(const FwdArgs &a, int D, int causal, hipStream_t stream);

struct MergeArgs {
  const void *o_parts[RA_MAX_MERGE_PARTS];
  const float *lse_parts[RA_MAX_MERGE_PARTS];
  void *o;
  float *lse;
  int64_t p_sb, p_sh, p_ss;   // strides of every o part
  int64_t pl_sb, pl_sh;       // strides of every lse part (seq stride 1)
  int64_t o_sb, o_sh, o_ss;
  int64_t l_sb, l_sh;
  int32_t n, B, H, S, D;
  int32_t parts_f32, out_f32;
};

int launch_lse_merge(const MergeArgs &a, hipStream_t stream);

struct PermuteArgs {
  const void *src;
  void *dst;
  // Sequence-sharded side [P, S/P, H, D] and head-sharded side [R, H/P, S, D] (R = 1 or P).
  int64_t seq_s0, seq_s1, seq_s2;       // strides of the shard, token, head axes
  int64_t head_s0, head_s1, head_s2;    // strides of the rank, head, token axes
  int32_t P, Sl, H, Hl, row_bytes, elem_bytes;
  int32_t rank0, nranks;                // ranks rank0 .. rank0 + nranks - 1
  int32_t dir;                          // 0: seq -> head, 1: head -> seq
};

int launch_ulysses_permute(const PermuteArgs &a, hipStream_t stream);
// Several (src, dst) pairs with the same P, rank and direction in one launch.
int launch_ulysses_permute_n(const PermuteArgs *a, int n, hipStream_t stream);

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *delta;  // workspace: D_i = rowsum(dout * o), [B, Hq, Sq] contiguous
  // workspace, or null: with grouped heads, per-query-head fp32 partials of dK and dV
  // ([2][B, Hq, Skv, D] contiguous, unscaled), summed over the group afterwards
  float *kv_part;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t l_sb, l_sh;
  int64_t dq_sb, dq_sh, dq_ss;
  int64_t dk_sb, dk_sh, dk_ss;
  int64_t dv_sb, dv_sh, dv_ss;
  int32_t B, Hq, Hkv, Sq, Skv, group;
  int32_t num_chunks, start_chunk, chunk_len;
  int64_t q_offset, kv_offset;
  float scale, scale_log2;
  // packed documents (attn_bwd_varlen only): document d holds tokens cu[d] .. cu[d+1]-1
  const int32_t *cu;
  int32_t n_docs;
};

// Attention over e4m3 inputs: the FwdArgs problem (q, k codes; v holds V^T codes
// [B, Hkv, D, vt_cols] with f.v_sb, f.v_sh its batch/head strides and f.v_ss the stride
// between its head-dim rows, all in bytes) plus one fp32 descale per (batch, head).
struct Fp8Args {
  FwdArgs f;
  const float *q_desc, *k_desc, *v_desc;
  int64_t qd_sb, qd_sh, kd_sb, kd_sh, vd_sb, vd_sh;
  int32_t vt_cols;  // stored keys per V^T row (Skv rounded up to 16)
};

int launch_attn_fwd_fp8(const Fp8Args &a, int D, int causal, hipStream_t stream);

// Per-head e4m3 quantization of a bf16 tensor [B, H, S, D]: partial maxima, then codes.
struct QuantArgs {
  const uint16_t *src;
  uint8_t *dst;
  float *descale;
  float *partial;            // workspace: B*H*nsplit partial maxima
  int64_t s_sb, s_sh, s_ss;  // src strides (elements)
  int64_t d_sb, d_sh, d_s2;  // dst strides (bytes); d_s2: token stride, or head-dim row stride (transposed)
  int64_t ds_sb, ds_sh;      // descale strides
  int32_t B, H, S, D, S_pad, nsplit, rows_per_split, transpose;
};

void quant_split(int64_t S, int64_t D, int32_t &nsplit, int32_t &rows_per_split);
int launch_fp8_quantize(const QuantArgs &a, hipStream_t stream);
// Several tensors (each with its own workspace partials) in one max launch and one
// conversion launch.
int launch_fp8_quantize_n(const QuantArgs *a, int n, hipStream_t stream);

size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq);
// Bytes of the grouped-head dK/dV partials (0 without grouped heads); they follow the
// D_i rows in the bf16 backward's workspace.
size_t bwd_kv_part_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D);
int launch_attn_bwd(const BwdArgs &a, int D, int causal, hipStream_t stream);
int launch_attn_bwd_varlen(const BwdArgs &a, int D, int causal, hipStream_t stream);
// One ring step: dq, dk, dv point at fp32 accumulators that receive += contributions.
int launch_attn_bwd_accum(const BwdArgs &a, int D, int causal, hipStream_t stream);
// fp32 inputs: dq, dk, dv are fp32; acc = true adds to them (the ring step).
int launch_attn_bwd_f32(const BwdArgs &a, int D, int causal, bool acc, hipStream_t stream);

}  // namespace ra
