// The exported C ABI of libra (declared in include/ra.h): host-side argument
// validation, then dispatch to the kernel launchers.  Validation touches no device
// state, so the *_validate entry points run on machines without a GPU.
#include <math.h>
#include <stddef.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

namespace ra {
namespace {

int64_t esize(int32_t dtype) {
  return dtype == RA_F32 ? 4 : (dtype == RA_BF16 ? 2 : (dtype == RA_FP8_E4M3 ? 1 : 0));
}

bool known_dtype(int32_t dtype) {
  return dtype == RA_F32 || dtype == RA_BF16 || dtype == RA_FP8_E4M3;
}

int64_t numel(const ra_tensor *t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// Rank, extents, innermost stride, non-negative strides and (for outputs) a layout in
// which no two elements share an address.  `vec_align`: the data pointer and outer
// strides must be multiples of this many bytes.
int check_tensor(const ra_tensor *t, int ndim, int64_t vec_align, bool is_output) {
  if (!t) return RA_ERR_NULL;
  if (!known_dtype(t->dtype)) return RA_ERR_DTYPE;
  if (t->ndim != ndim) return RA_ERR_SHAPE;
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0 || t->shape[i] > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  const int64_t n = numel(t);
  if (n == 0) return RA_OK;
  if (!t->data) return RA_ERR_NULL;
  for (int i = 0; i < ndim; ++i)
    if (t->stride[i] < 0) return RA_ERR_STRIDE;
  if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1) return RA_ERR_STRIDE;
  const int64_t es = esize(t->dtype);
  if (((uintptr_t)t->data) % (uintptr_t)vec_align) return RA_ERR_ALIGN;
  for (int i = 0; i < ndim - 1; ++i)
    if (t->shape[i] > 1 && (t->stride[i] * es) % vec_align) return RA_ERR_ALIGN;
  if (is_output) {
    // sufficient non-overlap test: visiting axes by increasing stride, each stride
    // exceeds the span of the axes already visited.
    int order[4] = {0, 1, 2, 3};
    std::sort(order, order + ndim, [&](int x, int y) { return t->stride[x] < t->stride[y]; });
    int64_t span = 0;
    for (int j = 0; j < ndim; ++j) {
      const int ax = order[j];
      if (t->shape[ax] <= 1) continue;
      if (t->stride[ax] <= span) return RA_ERR_STRIDE;
      span += (t->shape[ax] - 1) * t->stride[ax];
    }
  }
  return RA_OK;
}

bool same_shape(const ra_tensor *a, const ra_tensor *b) {
  if (a->ndim != b->ndim) return false;
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

bool same_strides(const ra_tensor *a, const ra_tensor *b) {
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] > 1 && a->stride[i] != b->stride[i]) return false;
  return true;
}

#define RA_TRY(expr)             \
  do {                           \
    int rc_ = (expr);            \
    if (rc_ != RA_OK) return rc_; \
  } while (0)

static_assert(offsetof(ra_attn_params, sched) == RA_ATTN_PARAMS_SIZE_V1 &&
                  sizeof(ra_attn_params) == RA_ATTN_PARAMS_SIZE_V2,
              "ra_attn_params layout");

// The work counter of a version-2 parameter block, NULL for a version-1 one.
uint64_t *sched_of(const ra_attn_params *p) {
  return p->struct_size >= RA_ATTN_PARAMS_SIZE_V2 ? p->sched : nullptr;
}

int check_params(const ra_attn_params *p, int64_t Skv) {
  if (!p) return RA_ERR_NULL;
  if (p->struct_size < RA_ATTN_PARAMS_SIZE_V1) return RA_ERR_RANGE;
  if (p->causal != 0 && p->causal != 1) return RA_ERR_RANGE;
  if (p->num_chunks < 1) return RA_ERR_RANGE;
  if (p->start_chunk < 0 || p->start_chunk >= p->num_chunks) return RA_ERR_RANGE;
  if (p->q_offset < 0 || p->kv_offset < 0) return RA_ERR_RANGE;
  if (p->q_offset > ((int64_t)1 << 40) || p->kv_offset > ((int64_t)1 << 40)) return RA_ERR_RANGE;
  if (!isfinite(p->scale)) return RA_ERR_RANGE;
  if (Skv % p->num_chunks) return RA_ERR_SHAPE;
  if (sched_of(p) && ((uintptr_t)sched_of(p)) % 8) return RA_ERR_ALIGN;
  return RA_OK;
}

float effective_scale(const ra_attn_params *p, int64_t D) {
  return p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)D));
}

// q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]; returns the shared checks of fwd and bwd.
int check_qkv(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v) {
  if (!q || !k || !v) return RA_ERR_NULL;
  RA_TRY(check_tensor(q, 4, 16, false));
  RA_TRY(check_tensor(k, 4, 16, false));
  RA_TRY(check_tensor(v, 4, 16, false));
  if (k->dtype != q->dtype || v->dtype != q->dtype) return RA_ERR_DTYPE;
  if (q->dtype == RA_FP8_E4M3) return RA_ERR_DTYPE;  // fp8 inputs: ra_attn_fwd_fp8
  if (!same_shape(k, v)) return RA_ERR_SHAPE;
  if (k->shape[0] != q->shape[0] || k->shape[3] != q->shape[3]) return RA_ERR_SHAPE;
  const int64_t Hq = q->shape[1], Hkv = k->shape[1];
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv)) return RA_ERR_SHAPE;
  return RA_OK;
}

int check_lse(const ra_tensor *lse, const ra_tensor *q, bool is_output) {
  if (!lse) return RA_ERR_NULL;
  RA_TRY(check_tensor(lse, 3, 4, is_output));
  if (lse->dtype != RA_F32) return RA_ERR_DTYPE;
  for (int i = 0; i < 3; ++i)
    if (lse->shape[i] != q->shape[i]) return RA_ERR_SHAPE;
  return RA_OK;
}

// A [B, H, S, D] operand read in tiles of up to kMaxTileRows tokens: a lane's byte offset
// within a tile, (rows - 1) * token stride + row bytes, must fit in 31 bits.
int check_tile_span(const ra_tensor *t) {
  if (!t || t->ndim != 4) return RA_OK;
  const int64_t rows = std::min<int64_t>(kMaxTileRows, t->shape[2]);
  if (rows <= 1 || t->shape[3] == 0) return RA_OK;
  const int64_t es = esize(t->dtype);
  if ((rows - 1) * t->stride[2] * es + t->shape[3] * es > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  return RA_OK;
}

int check_grid(const ra_tensor *q) {
  const int64_t tiles = (q->shape[2] + 127) / 128;
  if (tiles * q->shape[1] * q->shape[0] > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  return RA_OK;
}

int fwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                 const ra_attn_params *p, const ra_tensor *o, const ra_tensor *lse) {
  if (!o || !lse || !p) return RA_ERR_NULL;
  RA_TRY(check_qkv(q, k, v));
  RA_TRY(check_params(p, k->shape[2]));
  RA_TRY(check_tensor(o, 4, 16, true));
  if (o->dtype != q->dtype && o->dtype != RA_F32) return RA_ERR_DTYPE;
  if (!same_shape(o, q)) return RA_ERR_SHAPE;
  RA_TRY(check_lse(lse, q, true));
  RA_TRY(check_grid(q));
  for (const ra_tensor *t : {q, k, v, o}) RA_TRY(check_tile_span(t));
  const int64_t D = q->shape[3];
  if (D != 64 && D != 128) return RA_ERR_UNSUPPORTED;
  return RA_OK;
}

int merge_validate(int32_t n, const ra_tensor *o_parts, const ra_tensor *lse_parts,
                   const ra_tensor *o, const ra_tensor *lse) {
  if (!o_parts || !lse_parts || !o || !lse) return RA_ERR_NULL;
  if (n < 1 || n > RA_MAX_MERGE_PARTS) return RA_ERR_RANGE;
  RA_TRY(check_tensor(o, 4, 16, true));
  if (o->dtype == RA_FP8_E4M3) return RA_ERR_DTYPE;
  RA_TRY(check_lse(lse, o, true));
  for (int i = 0; i < n; ++i) {
    RA_TRY(check_tensor(&o_parts[i], 4, 16, false));
    RA_TRY(check_tensor(&lse_parts[i], 3, 4, false));
    if (o_parts[i].dtype != o_parts[0].dtype) return RA_ERR_DTYPE;
    if (o_parts[i].dtype == RA_FP8_E4M3) return RA_ERR_DTYPE;
    if (lse_parts[i].dtype != RA_F32) return RA_ERR_DTYPE;
    if (!same_shape(&o_parts[i], o)) return RA_ERR_SHAPE;
    for (int d = 0; d < 3; ++d)
      if (lse_parts[i].shape[d] != o->shape[d]) return RA_ERR_SHAPE;
    if (!same_strides(&o_parts[i], &o_parts[0])) return RA_ERR_STRIDE;
    if (!same_strides(&lse_parts[i], &lse_parts[0])) return RA_ERR_STRIDE;
  }
  const int64_t D = o->shape[3];
  if (D % 8 || D > 256) return RA_ERR_UNSUPPORTED;
  return RA_OK;
}

int permute_validate(const ra_tensor *src, const ra_tensor *dst, int32_t P, int32_t rank,
                     int32_t dir) {
  if (!src || !dst) return RA_ERR_NULL;
  if (dir != 0 && dir != 1) return RA_ERR_RANGE;
  if (P < 1) return RA_ERR_RANGE;
  if (rank < -1 || rank >= P) return RA_ERR_RANGE;
  const ra_tensor *seq = dir == 0 ? src : dst;
  const ra_tensor *head = dir == 0 ? dst : src;
  const int head_nd = rank == -1 ? 4 : 3;
  RA_TRY(check_tensor(seq, 4, 16, dir == 1));
  RA_TRY(check_tensor(head, head_nd, 16, dir == 0));
  if (src->dtype != dst->dtype) return RA_ERR_DTYPE;
  if (seq->shape[0] != P) return RA_ERR_SHAPE;
  const int64_t Sl = seq->shape[1], H = seq->shape[2], D = seq->shape[3];
  if (H % P) return RA_ERR_SHAPE;
  const int64_t hs[3] = {H / P, P * Sl, D};
  const int off = head_nd - 3;
  if (rank == -1 && head->shape[0] != P) return RA_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (head->shape[off + i] != hs[i]) return RA_ERR_SHAPE;
  if ((D * esize(src->dtype)) % 16) return RA_ERR_ALIGN;
  if (P * Sl > (int64_t)INT32_MAX) return RA_ERR_SHAPE;
  return RA_OK;
}

// grad_f32: dq, dk, dv are fp32 accumulators (the ring step) rather than q's dtype.
int bwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, const ra_tensor *o,
                 const ra_tensor *dout, const ra_tensor *lse, const ra_attn_params *p,
                 const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv,
                 bool grad_f32 = false) {
  if (!o || !dout || !lse || !p || !dq || !dk || !dv) return RA_ERR_NULL;
  RA_TRY(check_qkv(q, k, v));
  RA_TRY(check_params(p, k->shape[2]));
  RA_TRY(check_tensor(o, 4, 16, false));
  RA_TRY(check_tensor(dout, 4, 16, false));
  RA_TRY(check_tensor(dq, 4, 16, true));
  RA_TRY(check_tensor(dk, 4, 16, true));
  RA_TRY(check_tensor(dv, 4, 16, true));
  for (const ra_tensor *t : {o, dout})
    if (t->dtype != q->dtype) return RA_ERR_DTYPE;
  for (const ra_tensor *t : {dq, dk, dv})
    if (t->dtype != (grad_f32 ? RA_F32 : q->dtype)) return RA_ERR_DTYPE;
  if (!same_shape(o, q) || !same_shape(dout, q) || !same_shape(dq, q)) return RA_ERR_SHAPE;
  if (!same_shape(dk, k) || !same_shape(dv, k)) return RA_ERR_SHAPE;
  RA_TRY(check_lse(lse, q, false));
  RA_TRY(check_grid(q));
  RA_TRY(check_grid(k));
  for (const ra_tensor *t : {q, k, v, o, dout, dq, dk, dv}) RA_TRY(check_tile_span(t));
  const int64_t D = q->shape[3];
  if (D != 64 && D != 128) return RA_ERR_UNSUPPORTED;
  return RA_OK;
}

// Backward over packed documents: the ra_attn_bwd checks plus those of the packed forward.
int bwd_varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                        const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                        const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                        const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv) {
  RA_TRY(bwd_validate(q, k, v, o, dout, lse, p, dq, dk, dv));
  if (q->dtype != RA_BF16) return RA_ERR_UNSUPPORTED;  // the packed forward is bf16 only
  if (q->shape[2] != k->shape[2]) return RA_ERR_SHAPE;
  if (p->num_chunks != 1 || p->start_chunk != 0 || p->q_offset != 0 || p->kv_offset != 0)
    return RA_ERR_RANGE;
  if (n_docs < 1 || n_docs > RA_MAX_DOCS) return RA_ERR_RANGE;
  if (!cu_seqlens) return RA_ERR_NULL;
  if (((uintptr_t)cu_seqlens) % 4) return RA_ERR_ALIGN;
  return RA_OK;
}

// One device's ring-backward step: the ra_attn_bwd checks with fp32 accumulators, and
// the key/value block is a single chunk.
int bwd_accum_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                       const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                       const ra_attn_params *p, const ra_tensor *dq, const ra_tensor *dk,
                       const ra_tensor *dv) {
  RA_TRY(bwd_validate(q, k, v, o, dout, lse, p, dq, dk, dv, true));
  if (p->num_chunks != 1 || p->start_chunk != 0) return RA_ERR_RANGE;
  return RA_OK;
}

// One fp32 scale per (batch, head): a [B, H] tensor.
int check_descale(const ra_tensor *t, int64_t B, int64_t H, bool is_output) {
  if (!t) return RA_ERR_NULL;
  RA_TRY(check_tensor(t, 2, 4, is_output));
  if (t->dtype != RA_F32) return RA_ERR_DTYPE;
  if (t->shape[0] != B || t->shape[1] != H) return RA_ERR_SHAPE;
  return RA_OK;
}

// fp8 forward: q, k codes [B, H, S, D]; vt codes [B, Hkv, D, S_pad] (S_pad = Skv rounded
// up to 16, tokens contiguous, rows 16-byte aligned); descales; o bf16 or fp32.
int fp8_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *vt,
                 const ra_tensor *qd, const ra_tensor *kd, const ra_tensor *vd,
                 const ra_attn_params *p, const ra_tensor *o, const ra_tensor *lse) {
  if (!q || !k || !vt || !o || !lse || !p) return RA_ERR_NULL;
  RA_TRY(check_tensor(q, 4, 16, false));
  RA_TRY(check_tensor(k, 4, 16, false));
  RA_TRY(check_tensor(vt, 4, 16, false));
  for (const ra_tensor *t : {q, k, vt})
    if (t->dtype != RA_FP8_E4M3) return RA_ERR_DTYPE;
  const int64_t B = q->shape[0], Hq = q->shape[1], Sq = q->shape[2], D = q->shape[3];
  const int64_t Hkv = k->shape[1], Skv = k->shape[2];
  if (k->shape[0] != B || k->shape[3] != D) return RA_ERR_SHAPE;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv)) return RA_ERR_SHAPE;
  const int64_t S_pad = (Skv + 15) / 16 * 16;
  if (vt->shape[0] != B || vt->shape[1] != Hkv || vt->shape[2] != D || vt->shape[3] != S_pad)
    return RA_ERR_SHAPE;
  RA_TRY(check_params(p, Skv));
  // key tiles start at chunk starts plus multiples of 64: 16-key chunks keep every V^T
  // tile load on a 16-byte boundary of its row, so the last tile's clamped columns
  // never hold a visible key
  if (p->num_chunks > 1 && (Skv / p->num_chunks) % 16 != 0) return RA_ERR_ALIGN;
  RA_TRY(check_tensor(o, 4, 16, true));
  if (o->dtype != RA_BF16 && o->dtype != RA_F32) return RA_ERR_DTYPE;
  if (!same_shape(o, q)) return RA_ERR_SHAPE;
  RA_TRY(check_lse(lse, q, true));
  RA_TRY(check_grid(q));
  RA_TRY(check_descale(qd, B, Hq, false));
  RA_TRY(check_descale(kd, B, Hkv, false));
  RA_TRY(check_descale(vd, B, Hkv, false));
  if (D != 64 && D != 128) return RA_ERR_UNSUPPORTED;
  // the kernel forms byte offsets within one head in 32 bits
  if (Skv > 0 && ((Skv - 1) * k->stride[2] + D > (int64_t)INT32_MAX ||
                  (D - 1) * vt->stride[2] + S_pad > (int64_t)INT32_MAX))
    return RA_ERR_SHAPE;
  return RA_OK;
}

// Quantizer: src bf16 [B, H, S, D] (D a multiple of 16, at most 256); dst codes of the
// same shape, or [B, H, D, S_pad] when transposed; descale [B, H] fp32.
int quant_validate(const ra_tensor *src, const ra_tensor *dst, const ra_tensor *descale,
                   int32_t transpose) {
  if (!src || !dst || !descale) return RA_ERR_NULL;
  if (transpose != 0 && transpose != 1) return RA_ERR_RANGE;
  RA_TRY(check_tensor(src, 4, 16, false));
  RA_TRY(check_tensor(dst, 4, 16, true));
  if (src->dtype != RA_BF16 || dst->dtype != RA_FP8_E4M3) return RA_ERR_DTYPE;
  const int64_t B = src->shape[0], H = src->shape[1], S = src->shape[2], D = src->shape[3];
  if (D % 16 || D > 256) return RA_ERR_UNSUPPORTED;
  if (transpose) {
    const int64_t S_pad = (S + 15) / 16 * 16;
    if (dst->shape[0] != B || dst->shape[1] != H || dst->shape[2] != D || dst->shape[3] != S_pad)
      return RA_ERR_SHAPE;
  } else if (!same_shape(src, dst)) {
    return RA_ERR_SHAPE;
  }
  RA_TRY(check_descale(descale, B, H, true));
  if (B * H > (int64_t)INT32_MAX / 1024 || B * H * ((S + 63) / 64 + 1) > (int64_t)INT32_MAX)
    return RA_ERR_SHAPE;
  return RA_OK;
}

size_t quant_workspace_bytes(const ra_tensor *src) {
  int32_t nsplit, rps;
  quant_split(src->shape[2], src->shape[3], nsplit, rps);
  const size_t n = (size_t)(src->shape[0] * src->shape[1]) * (size_t)nsplit * sizeof(float);
  return (n + 255) / 256 * 256;
}

QuantArgs quant_args(const ra_tensor *src, ra_tensor *dst, ra_tensor *descale, int32_t transpose,
                     void *workspace) {
  QuantArgs a{};
  a.src = (const uint16_t *)src->data;
  a.dst = (uint8_t *)dst->data;
  a.descale = (float *)descale->data;
  a.partial = (float *)workspace;
  a.s_sb = src->stride[0]; a.s_sh = src->stride[1]; a.s_ss = src->stride[2];
  a.d_sb = dst->stride[0]; a.d_sh = dst->stride[1]; a.d_s2 = dst->stride[2];
  a.ds_sb = descale->stride[0]; a.ds_sh = descale->stride[1];
  a.B = (int32_t)src->shape[0]; a.H = (int32_t)src->shape[1];
  a.S = (int32_t)src->shape[2]; a.D = (int32_t)src->shape[3];
  a.S_pad = (a.S + 15) / 16 * 16;
  a.transpose = transpose;
  quant_split(a.S, a.D, a.nsplit, a.rows_per_split);
  return a;
}

BwdArgs bwd_args(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, const ra_tensor *o,
                 const ra_tensor *dout, const ra_tensor *lse, const ra_attn_params *p,
                 ra_tensor *dq, ra_tensor *dk, ra_tensor *dv, void *workspace) {
  BwdArgs a{};
  a.q = q->data; a.k = k->data; a.v = v->data; a.o = o->data; a.dout = dout->data;
  a.lse = (const float *)lse->data;
  a.dq = dq->data; a.dk = dk->data; a.dv = dv->data;
  a.delta = (float *)workspace;
  a.q_sb = q->stride[0]; a.q_sh = q->stride[1]; a.q_ss = q->stride[2];
  a.k_sb = k->stride[0]; a.k_sh = k->stride[1]; a.k_ss = k->stride[2];
  a.v_sb = v->stride[0]; a.v_sh = v->stride[1]; a.v_ss = v->stride[2];
  a.o_sb = o->stride[0]; a.o_sh = o->stride[1]; a.o_ss = o->stride[2];
  a.do_sb = dout->stride[0]; a.do_sh = dout->stride[1]; a.do_ss = dout->stride[2];
  a.l_sb = lse->stride[0]; a.l_sh = lse->stride[1];
  a.dq_sb = dq->stride[0]; a.dq_sh = dq->stride[1]; a.dq_ss = dq->stride[2];
  a.dk_sb = dk->stride[0]; a.dk_sh = dk->stride[1]; a.dk_ss = dk->stride[2];
  a.dv_sb = dv->stride[0]; a.dv_sh = dv->stride[1]; a.dv_ss = dv->stride[2];
  a.B = (int32_t)q->shape[0]; a.Hq = (int32_t)q->shape[1]; a.Sq = (int32_t)q->shape[2];
  a.Hkv = (int32_t)k->shape[1]; a.Skv = (int32_t)k->shape[2];
  a.group = a.Hkv ? a.Hq / a.Hkv : 1;
  a.num_chunks = p->num_chunks; a.start_chunk = p->start_chunk;
  a.chunk_len = a.Skv / a.num_chunks;
  a.q_offset = p->q_offset; a.kv_offset = p->kv_offset;
  a.scale = effective_scale(p, q->shape[3]);
  a.scale_log2 = a.scale * kLog2eHost;
  return a;
}

// Workspace of the bf16/fp32 backward: the D_i rows, then (bf16 with grouped heads) the
// per-query-head dK/dV partials.
size_t bwd_need_bytes(const ra_tensor *q, const ra_tensor *k) {
  const size_t delta = bwd_workspace_bytes(q->shape[0], q->shape[1], q->shape[2]);
  if (q->dtype != RA_BF16) return delta;
  return delta + bwd_kv_part_bytes(q->shape[0], q->shape[1], k->shape[1], k->shape[2],
                                   q->shape[3]);
}

// Points a.kv_part at the partials that follow the D_i rows, when there are any.
void bwd_set_parts(BwdArgs &a, const ra_tensor *q, const ra_tensor *k, void *workspace) {
  if (q->dtype != RA_BF16 ||
      bwd_kv_part_bytes(q->shape[0], q->shape[1], k->shape[1], k->shape[2], q->shape[3]) == 0)
    return;
  a.kv_part = (float *)((char *)workspace +
                        bwd_workspace_bytes(q->shape[0], q->shape[1], q->shape[2]));
}

}  // namespace
}  // namespace ra

using namespace ra;

extern "C" {

int ra_version(void) { return RA_VERSION; }

const char *ra_status_string(int status) {
  switch (status) {
    case RA_OK: return "RA_OK: success";
    case RA_ERR_NULL: return "RA_ERR_NULL: a required pointer is NULL";
    case RA_ERR_DTYPE: return "RA_ERR_DTYPE: dtype not allowed or mismatched";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE: ranks or extents are inconsistent";
    case RA_ERR_STRIDE: return "RA_ERR_STRIDE: innermost stride must be 1, strides non-negative, outputs non-overlapping";
    case RA_ERR_ALIGN: return "RA_ERR_ALIGN: pointer or row stride not a multiple of 16 bytes";
    case RA_ERR_RANGE: return "RA_ERR_RANGE: a scalar parameter is out of range";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED: valid request not implemented (head dim or dtype)";
    case RA_ERR_HIP: return "RA_ERR_HIP: kernel launch failed";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case RA_ERR_SCRATCH: return "RA_ERR_SCRATCH: the problem needs more workspace than the no-allocation entry point's fixed scratch holds (use ra_attn_bwd with a workspace)";
    default: return "unknown ra_status";
  }
}

int ra_attn_fwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         const ra_attn_params *p, const ra_tensor *o, const ra_tensor *lse) {
  return fwd_validate(q, k, v, p, o, lse);
}

int ra_attn_fwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                const ra_attn_params *p, ra_tensor *o, ra_tensor *lse, ra_stream stream) {
  RA_TRY(fwd_validate(q, k, v, p, o, lse));
  if (numel(q) == 0) return RA_OK;
  FwdArgs a{};
  a.q = q->data; a.k = k->data; a.v = v->data; a.o = o->data; a.lse = (float *)lse->data;
  a.q_sb = q->stride[0]; a.q_sh = q->stride[1]; a.q_ss = q->stride[2];
  a.k_sb = k->stride[0]; a.k_sh = k->stride[1]; a.k_ss = k->stride[2];
  a.v_sb = v->stride[0]; a.v_sh = v->stride[1]; a.v_ss = v->stride[2];
  a.o_sb = o->stride[0]; a.o_sh = o->stride[1]; a.o_ss = o->stride[2];
  a.l_sb = lse->stride[0]; a.l_sh = lse->stride[1];
  a.B = (int32_t)q->shape[0]; a.Hq = (int32_t)q->shape[1]; a.Sq = (int32_t)q->shape[2];
  a.Hkv = (int32_t)k->shape[1]; a.Skv = (int32_t)k->shape[2];
  a.group = a.Hq / a.Hkv;
  a.num_chunks = p->num_chunks; a.start_chunk = p->start_chunk;
  a.chunk_len = a.Skv / a.num_chunks;
  a.q_offset = p->q_offset; a.kv_offset = p->kv_offset;
  a.scale_log2 = effective_scale(p, q->shape[3]) * kLog2eHost;
  a.o_is_f32 = o->dtype == RA_F32;
  a.sched = sched_of(p);
  return launch_attn_fwd(a, q->dtype, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

namespace {
// Packed documents: q and k/v hold the same T tokens; one chunk, no offsets; bf16.
int varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                    const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                    const ra_tensor *o, const ra_tensor *lse) {
  RA_TRY(fwd_validate(q, k, v, p, o, lse));
  if (q->shape[2] != k->shape[2]) return RA_ERR_SHAPE;
  if (p->num_chunks != 1 || p->start_chunk != 0 || p->q_offset != 0 || p->kv_offset != 0)
    return RA_ERR_RANGE;
  if (n_docs < 1 || n_docs > RA_MAX_DOCS) return RA_ERR_RANGE;
  if (!cu_seqlens) return RA_ERR_NULL;
  if (((uintptr_t)cu_seqlens) % 4) return RA_ERR_ALIGN;
  if (q->dtype != RA_BF16) return RA_ERR_UNSUPPORTED;
  return RA_OK;
}
}  // namespace

int ra_attn_fwd_varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                const int32_t *cu_seqlens, int32_t n_docs,
                                const ra_attn_params *p, const ra_tensor *o,
                                const ra_tensor *lse) {
  return varlen_validate(q, k, v, cu_seqlens, n_docs, p, o, lse);
}

int ra_attn_fwd_varlen(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                       const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                       ra_tensor *o, ra_tensor *lse, ra_stream stream) {
  RA_TRY(varlen_validate(q, k, v, cu_seqlens, n_docs, p, o, lse));
  if (numel(q) == 0) return RA_OK;
  FwdArgs a{};
  a.q = q->data; a.k = k->data; a.v = v->data; a.o = o->data; a.lse = (float *)lse->data;
  a.q_sb = q->stride[0]; a.q_sh = q->stride[1]; a.q_ss = q->stride[2];
  a.k_sb = k->stride[0]; a.k_sh = k->stride[1]; a.k_ss = k->stride[2];
  a.v_sb = v->stride[0]; a.v_sh = v->stride[1]; a.v_ss = v->stride[2];
  a.o_sb = o->stride[0]; a.o_sh = o->stride[1]; a.o_ss = o->stride[2];
  a.l_sb = lse->stride[0]; a.l_sh = lse->stride[1];
  a.B = (int32_t)q->shape[0]; a.Hq = (int32_t)q->shape[1]; a.Sq = (int32_t)q->shape[2];
  a.Hkv = (int32_t)k->shape[1]; a.Skv = (int32_t)k->shape[2];
  a.group = a.Hq / a.Hkv;
  a.num_chunks = 1; a.start_chunk = 0; a.chunk_len = a.Skv;
  a.q_offset = 0; a.kv_offset = 0;
  a.scale_log2 = effective_scale(p, q->shape[3]) * kLog2eHost;
  a.o_is_f32 = o->dtype == RA_F32;
  a.cu = cu_seqlens;
  a.n_docs = n_docs;
  a.sched = sched_of(p);
  return launch_attn_fwd_varlen(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

int ra_lse_merge_validate(int32_t n, const ra_tensor *o_parts, const ra_tensor *lse_parts,
                          const ra_tensor *o, const ra_tensor *lse) {
  return merge_validate(n, o_parts, lse_parts, o, lse);
}

int ra_lse_merge(int32_t n, const ra_tensor *o_parts, const ra_tensor *lse_parts, ra_tensor *o,
                 ra_tensor *lse, ra_stream stream) {
  RA_TRY(merge_validate(n, o_parts, lse_parts, o, lse));
  if (numel(o) == 0) return RA_OK;
  MergeArgs a{};
  for (int i = 0; i < n; ++i) {
    a.o_parts[i] = o_parts[i].data;
    a.lse_parts[i] = (const float *)lse_parts[i].data;
  }
  a.o = o->data; a.lse = (float *)lse->data;
  a.p_sb = o_parts[0].stride[0]; a.p_sh = o_parts[0].stride[1]; a.p_ss = o_parts[0].stride[2];
  a.pl_sb = lse_parts[0].stride[0]; a.pl_sh = lse_parts[0].stride[1];
  a.o_sb = o->stride[0]; a.o_sh = o->stride[1]; a.o_ss = o->stride[2];
  a.l_sb = lse->stride[0]; a.l_sh = lse->stride[1];
  a.n = n; a.B = (int32_t)o->shape[0]; a.H = (int32_t)o->shape[1];
  a.S = (int32_t)o->shape[2]; a.D = (int32_t)o->shape[3];
  a.parts_f32 = o_parts[0].dtype == RA_F32;
  a.out_f32 = o->dtype == RA_F32;
  return launch_lse_merge(a, (hipStream_t)stream);
}

namespace {
PermuteArgs permute_args(const ra_tensor *src, const ra_tensor *dst, int32_t P, int32_t rank,
                         int32_t dir) {
  const ra_tensor *seq = dir == 0 ? src : dst;
  const ra_tensor *head = dir == 0 ? dst : src;
  PermuteArgs a{};
  a.src = src->data; a.dst = dst->data;
  a.seq_s0 = seq->stride[0]; a.seq_s1 = seq->stride[1]; a.seq_s2 = seq->stride[2];
  const int off = head->ndim - 3;
  a.head_s0 = off ? head->stride[0] : 0;
  a.head_s1 = head->stride[off + 0]; a.head_s2 = head->stride[off + 1];
  a.P = P; a.Sl = (int32_t)seq->shape[1]; a.H = (int32_t)seq->shape[2]; a.Hl = a.H / P;
  a.elem_bytes = (int32_t)esize(src->dtype);
  a.row_bytes = (int32_t)(seq->shape[3] * a.elem_bytes);
  a.rank0 = rank == -1 ? 0 : rank;
  a.nranks = rank == -1 ? P : 1;
  a.dir = dir;
  return a;
}

// byte range [lo, hi) a tensor's elements can touch (a conservative extent)
void byte_span(const ra_tensor *t, uintptr_t &lo, uintptr_t &hi) {
  int64_t last = 0;
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] > 0) last += (t->shape[i] - 1) * t->stride[i];
  lo = (uintptr_t)t->data;
  hi = lo + (uintptr_t)((last + 1) * esize(t->dtype));
}

bool overlaps(const ra_tensor *a, const ra_tensor *b) {
  if (numel(a) == 0 || numel(b) == 0) return false;
  uintptr_t a0, a1, b0, b1;
  byte_span(a, a0, a1);
  byte_span(b, b0, b1);
  return a0 < b1 && b0 < a1;
}

int permute_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts, int32_t P,
                       int32_t rank, int32_t dir) {
  if (!srcs || !dsts) return RA_ERR_NULL;
  if (n < 1 || n > RA_MAX_PERMUTE_TENSORS) return RA_ERR_RANGE;
  for (int i = 0; i < n; ++i) RA_TRY(permute_validate(&srcs[i], &dsts[i], P, rank, dir));
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (overlaps(&dsts[i], &srcs[j]) || (i != j && overlaps(&dsts[i], &dsts[j])))
        return RA_ERR_STRIDE;
  return RA_OK;
}
}  // namespace

int ra_ulysses_permute_validate(const ra_tensor *src, const ra_tensor *dst, int32_t P,
                                int32_t rank, int32_t dir) {
  return permute_validate(src, dst, P, rank, dir);
}

int ra_ulysses_permute(const ra_tensor *src, ra_tensor *dst, int32_t P, int32_t rank, int32_t dir,
                       ra_stream stream) {
  RA_TRY(permute_validate(src, dst, P, rank, dir));
  if (numel(src) == 0) return RA_OK;
  const PermuteArgs a = permute_args(src, dst, P, rank, dir);
  return launch_ulysses_permute(a, (hipStream_t)stream);
}


int ra_ulysses_permute_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts,
                                  int32_t P, int32_t rank, int32_t dir) {
  return permute_n_validate(n, srcs, dsts, P, rank, dir);
}

namespace {

int quant_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts,
                     const ra_tensor *descales, const int32_t *transpose) {
  if (!srcs || !dsts || !descales || !transpose) return RA_ERR_NULL;
  if (n < 1 || n > RA_MAX_QUANT_TENSORS) return RA_ERR_RANGE;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    RA_TRY(quant_validate(&srcs[i], &dsts[i], &descales[i], transpose[i]));
    int32_t nsplit, rps;
    quant_split(srcs[i].shape[2], srcs[i].shape[3], nsplit, rps);
    const int64_t tiles = (srcs[i].shape[2] + 15) / 16 * 16 / 64 + 1;
    blocks += srcs[i].shape[0] * srcs[i].shape[1] * (nsplit > tiles ? nsplit : tiles);
  }
  if (blocks > (int64_t)INT32_MAX) return RA_ERR_SHAPE;  // one grid covers all tensors
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      if (overlaps(&dsts[i], &srcs[j]) || overlaps(&descales[i], &srcs[j]) ||
          overlaps(&descales[i], &dsts[j]))
        return RA_ERR_STRIDE;
      if (i != j && (overlaps(&dsts[i], &dsts[j]) || overlaps(&descales[i], &descales[j])))
        return RA_ERR_STRIDE;
    }
  return RA_OK;
}

// each tensor's partial maxima at a 256-byte aligned offset of the workspace
size_t quant_n_offsets(int32_t n, const ra_tensor *srcs, size_t *off) {
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (off) off[i] = total;
    total += quant_workspace_bytes(&srcs[i]);
  }
  return total;
}

}  // namespace

int ra_fp8_quantize_n_validate(int32_t n, const ra_tensor *srcs, const ra_tensor *dsts,
                               const ra_tensor *descales, const int32_t *transpose) {
  return quant_n_validate(n, srcs, dsts, descales, transpose);
}

size_t ra_fp8_quantize_n_workspace_size(int32_t n, const ra_tensor *srcs) {
  if (!srcs || n < 1 || n > RA_MAX_QUANT_TENSORS) return 0;
  for (int i = 0; i < n; ++i)
    if (check_tensor(&srcs[i], 4, 16, false) != RA_OK) return 0;
  return quant_n_offsets(n, srcs, nullptr);
}

int ra_fp8_quantize_n(int32_t n, const ra_tensor *srcs, ra_tensor *dsts, ra_tensor *descales,
                      const int32_t *transpose, void *workspace, size_t workspace_bytes,
                      ra_stream stream) {
  RA_TRY(quant_n_validate(n, srcs, dsts, descales, transpose));
  size_t off[RA_MAX_QUANT_TENSORS];
  const size_t need = quant_n_offsets(n, srcs, off);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace) % 256)
    return RA_ERR_WORKSPACE;
  QuantArgs a[RA_MAX_QUANT_TENSORS];
  for (int i = 0; i < n; ++i)
    a[i] = quant_args(&srcs[i], &dsts[i], &descales[i], transpose[i],
                      (char *)workspace + off[i]);
  return launch_fp8_quantize_n(a, n, (hipStream_t)stream);
}

int ra_ulysses_permute_n(int32_t n, const ra_tensor *srcs, ra_tensor *dsts, int32_t P,
                         int32_t rank, int32_t dir, ra_stream stream) {
  RA_TRY(permute_n_validate(n, srcs, dsts, P, rank, dir));
  PermuteArgs a[RA_MAX_PERMUTE_TENSORS];
  int k = 0;
  for (int i = 0; i < n; ++i)
    if (numel(&srcs[i]) > 0) a[k++] = permute_args(&srcs[i], &dsts[i], P, rank, dir);
  if (k == 0) return RA_OK;
  return launch_ulysses_permute_n(a, k, (hipStream_t)stream);
}

int ra_attn_bwd_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                         const ra_attn_params *p, const ra_tensor *dq, const ra_tensor *dk,
                         const ra_tensor *dv) {
  return bwd_validate(q, k, v, o, dout, lse, p, dq, dk, dv);
}

size_t ra_attn_bwd_workspace_size(const ra_tensor *q, const ra_tensor *k, const ra_attn_params *p) {
  if (!q || !k || !p) return 0;
  if (check_qkv(q, k, k) != RA_OK || check_params(p, k->shape[2]) != RA_OK) return 0;
  return bwd_need_bytes(q, k);
}

int ra_attn_bwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, const ra_tensor *o,
                const ra_tensor *dout, const ra_tensor *lse, const ra_attn_params *p,
                ra_tensor *dq, ra_tensor *dk, ra_tensor *dv, void *workspace,
                size_t workspace_bytes, ra_stream stream) {
  RA_TRY(bwd_validate(q, k, v, o, dout, lse, p, dq, dk, dv));
  const size_t need = bwd_need_bytes(q, k);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace) % 256))
    return RA_ERR_WORKSPACE;
  if (numel(q) == 0 && numel(k) == 0) return RA_OK;
  BwdArgs a = bwd_args(q, k, v, o, dout, lse, p, dq, dk, dv, workspace);
  bwd_set_parts(a, q, k, workspace);
  if (q->dtype == RA_F32)
    return launch_attn_bwd_f32(a, (int)q->shape[3], p->causal, false, (hipStream_t)stream);
  return launch_attn_bwd(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

int ra_attn_bwd_varlen_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                                const int32_t *cu_seqlens, int32_t n_docs,
                                const ra_attn_params *p, const ra_tensor *dq, const ra_tensor *dk,
                                const ra_tensor *dv) {
  return bwd_varlen_validate(q, k, v, o, dout, lse, cu_seqlens, n_docs, p, dq, dk, dv);
}

int ra_attn_bwd_varlen(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                       const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                       const int32_t *cu_seqlens, int32_t n_docs, const ra_attn_params *p,
                       ra_tensor *dq, ra_tensor *dk, ra_tensor *dv, void *workspace,
                       size_t workspace_bytes, ra_stream stream) {
  RA_TRY(bwd_varlen_validate(q, k, v, o, dout, lse, cu_seqlens, n_docs, p, dq, dk, dv));
  const size_t need = bwd_need_bytes(q, k);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace) % 256))
    return RA_ERR_WORKSPACE;
  if (numel(q) == 0 && numel(k) == 0) return RA_OK;
  BwdArgs a = bwd_args(q, k, v, o, dout, lse, p, dq, dk, dv, workspace);
  bwd_set_parts(a, q, k, workspace);
  a.cu = cu_seqlens;
  a.n_docs = n_docs;
  return launch_attn_bwd_varlen(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

int ra_attn_fwd_fp8_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *vt,
                             const ra_tensor *q_descale, const ra_tensor *k_descale,
                             const ra_tensor *v_descale, const ra_attn_params *p,
                             const ra_tensor *o, const ra_tensor *lse) {
  return fp8_validate(q, k, vt, q_descale, k_descale, v_descale, p, o, lse);
}

int ra_attn_fwd_fp8(const ra_tensor *q, const ra_tensor *k, const ra_tensor *vt,
                    const ra_tensor *q_descale, const ra_tensor *k_descale,
                    const ra_tensor *v_descale, const ra_attn_params *p, ra_tensor *o,
                    ra_tensor *lse, ra_stream stream) {
  RA_TRY(fp8_validate(q, k, vt, q_descale, k_descale, v_descale, p, o, lse));
  if (numel(q) == 0) return RA_OK;
  Fp8Args a{};
  FwdArgs &f = a.f;
  f.q = q->data; f.k = k->data; f.v = vt->data; f.o = o->data; f.lse = (float *)lse->data;
  f.q_sb = q->stride[0]; f.q_sh = q->stride[1]; f.q_ss = q->stride[2];
  f.k_sb = k->stride[0]; f.k_sh = k->stride[1]; f.k_ss = k->stride[2];
  f.v_sb = vt->stride[0]; f.v_sh = vt->stride[1]; f.v_ss = vt->stride[2];
  f.o_sb = o->stride[0]; f.o_sh = o->stride[1]; f.o_ss = o->stride[2];
  f.l_sb = lse->stride[0]; f.l_sh = lse->stride[1];
  f.B = (int32_t)q->shape[0]; f.Hq = (int32_t)q->shape[1]; f.Sq = (int32_t)q->shape[2];
  f.Hkv = (int32_t)k->shape[1]; f.Skv = (int32_t)k->shape[2];
  f.group = f.Hq / f.Hkv;
  f.num_chunks = p->num_chunks; f.start_chunk = p->start_chunk;
  f.chunk_len = f.Skv / f.num_chunks;
  f.q_offset = p->q_offset; f.kv_offset = p->kv_offset;
  f.scale_log2 = effective_scale(p, q->shape[3]) * kLog2eHost;
  f.o_is_f32 = o->dtype == RA_F32;
  a.q_desc = (const float *)q_descale->data;
  a.k_desc = (const float *)k_descale->data;
  a.v_desc = (const float *)v_descale->data;
  a.qd_sb = q_descale->stride[0]; a.qd_sh = q_descale->stride[1];
  a.kd_sb = k_descale->stride[0]; a.kd_sh = k_descale->stride[1];
  a.vd_sb = v_descale->stride[0]; a.vd_sh = v_descale->stride[1];
  a.vt_cols = (int32_t)vt->shape[3];
  f.sched = sched_of(p);
  return launch_attn_fwd_fp8(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

int ra_fp8_quantize_validate(const ra_tensor *src, const ra_tensor *dst,
                             const ra_tensor *descale, int32_t transpose) {
  return quant_validate(src, dst, descale, transpose);
}

size_t ra_fp8_quantize_workspace_size(const ra_tensor *src) {
  if (!src || check_tensor(src, 4, 16, false) != RA_OK) return 0;
  return quant_workspace_bytes(src);
}

int ra_fp8_quantize(const ra_tensor *src, ra_tensor *dst, ra_tensor *descale, int32_t transpose,
                    void *workspace, size_t workspace_bytes, ra_stream stream) {
  RA_TRY(quant_validate(src, dst, descale, transpose));
  const size_t need = quant_workspace_bytes(src);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace) % 256)
    return RA_ERR_WORKSPACE;
  const QuantArgs a = quant_args(src, dst, descale, transpose, workspace);
  return launch_fp8_quantize(a, (hipStream_t)stream);
}

int ra_attn_bwd_accum_validate(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                               const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                               const ra_attn_params *p, const ra_tensor *dq_acc,
                               const ra_tensor *dk_acc, const ra_tensor *dv_acc) {
  return bwd_accum_validate(q, k, v, o, dout, lse, p, dq_acc, dk_acc, dv_acc);
}

int ra_attn_bwd_accum(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                      const ra_tensor *o, const ra_tensor *dout, const ra_tensor *lse,
                      const ra_attn_params *p, ra_tensor *dq_acc, ra_tensor *dk_acc,
                      ra_tensor *dv_acc, void *workspace, size_t workspace_bytes,
                      ra_stream stream) {
  RA_TRY(bwd_accum_validate(q, k, v, o, dout, lse, p, dq_acc, dk_acc, dv_acc));
  const size_t need = bwd_need_bytes(q, k);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace) % 256))
    return RA_ERR_WORKSPACE;
  if (numel(q) == 0 || numel(k) == 0) return RA_OK;  // nothing to add
  // causal chunk skip: a chunk after the block's last query adds nothing
  if (p->causal && p->kv_offset > p->q_offset + q->shape[2] - 1) return RA_OK;
  BwdArgs a = bwd_args(q, k, v, o, dout, lse, p, dq_acc, dk_acc, dv_acc, workspace);
  bwd_set_parts(a, q, k, workspace);
  if (q->dtype == RA_F32)
    return launch_attn_bwd_f32(a, (int)q->shape[3], p->causal, true, (hipStream_t)stream);
  return launch_attn_bwd_accum(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// ra_attn_bwd_noalloc: ra_attn_bwd with its workspace in a fixed device array of this
// library, for callers that cannot allocate.  The array is a file-scope __device__
// object, so every GPU the library runs on holds its own copy (RA_NOALLOC_SCRATCH_BYTES)
// from module load until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only names a stand-in): the device address of the current GPU's
// copy is looked up once per device with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------------
namespace {

__device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, or null

// The current device's copy of `scratch` (looked up on the first call on that device).
int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return RA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" int ra_attn_bwd_noalloc(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                   const ra_tensor *o, const ra_tensor *dout,
                                   const ra_tensor *lse, const ra_attn_params *p, ra_tensor *dq,
                                   ra_tensor *dk, ra_tensor *dv, ra_stream stream) {
  RA_TRY(bwd_validate(q, k, v, o, dout, lse, p, dq, dk, dv));
  const size_t need = bwd_workspace_bytes(q->shape[0], q->shape[1], q->shape[2]);
  if (need > (size_t)RA_NOALLOC_SCRATCH_BYTES) return RA_ERR_SCRATCH;
  if (numel(q) == 0 && numel(k) == 0) return RA_OK;
  void *ws = nullptr;
  RA_TRY(scratch_of_current_device(&ws));
  BwdArgs a = bwd_args(q, k, v, o, dout, lse, p, dq, dk, dv, ws);
  if (q->dtype == RA_F32)
    return launch_attn_bwd_f32(a, (int)q->shape[3], p->causal, false, (hipStream_t)stream);
  return launch_attn_bwd(a, (int)q->shape[3], p->causal, (hipStream_t)stream);
}

extern "C" size_t ra_noalloc_scratch_bytes(void) { return (size_t)RA_NOALLOC_SCRATCH_BYTES; }
