// attn_bwd_f32 -- the backward of exact softmax attention for fp32 inputs: the same
// gradients as attn_bwd.hip (P recomputed from the forward's saved log-sum-exp), with
// 32x32x2 fp32 MFMAs and fp32 throughout.
//
// Sources (page title, host):
//   [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn), section
//        "为什么传统注意力这么“吃”显存？": the backward pass needs the attention
//        intermediates, kept or recomputed; here they are recomputed tile by tile.
//   [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn), section
//        "Ring-Attention：面向大规模部署的工程利器": gradients travel back along the ring.
// Textbook formulas (not on the pages), L = sum(dO * O):
//   P = exp(scale q.k - lse), D_i = rowsum(dO * O), dV = P^T dO, dP = dO V^T,
//   dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels, no atomics (bitwise deterministic):
//   * bwd_delta_f32 -- D_i, one 64-lane group per 2 rows;
//   * bwd_dq_f32    -- 4 waves x 32 query rows; 32-key K/V tiles staged through registers
//                      into LDS in ring order; per tile S^T = K Q^T and dP^T = V dO^T (Q, dO
//                      in registers), then dQ^T += K^T dS^T;
//   * bwd_dkdv_f32  -- 4 waves x 32 keys of one key/value head; 32-row Q/dO tiles of every
//                      query head of its group through LDS: S = Q K^T, dP = dO V^T (K^T, V^T
//                      in registers), dV^T += dO^T P, dK^T += Q^T dS.  A workgroup keeps
//                      the dK, dV accumulators of 64 head dims; with D = 128 two workgroups
//                      share a key block (grid y), each recomputing S and dP, so that one
//                      wave's registers hold K^T, V^T and its accumulators without spills.
// The 32x32x2 fp32 MFMA: lane l holds A[l%32][k = l/32] and B[k = l/32][l%32]; the result
// element i of lane l is row (i/4)*8 + 4(l/32) + i%4, column l%32.  Head dims are walked
// as in the fp32 forward: MFMA step 2j+e of lane half h uses dim 4j + 2h + e (A and B
// agree); key (or query) contractions over a 32-row block use, at step t, the row that
// the lane's own result element t holds, so P and dS feed the next product from
// registers.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kTile = 32;  // keys (dQ kernel) or query rows (dK/dV kernel) per LDS tile
static_assert(kTile <= kMaxTileRows, "tile offsets");

__global__ void __launch_bounds__(256) bwd_delta_f32_kernel(BwdArgs a, int D) {
  // 32 lanes per row, each D/32 consecutive floats (D = 64 or 128)
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Sq;
  const int sub = threadIdx.x & 31;
  const int per = D / 32;
  for (int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 32; row < nrows;
       row += (int64_t)gridDim.x * 8) {
    const int s = (int)(row % a.Sq);
    const int64_t bh = row / a.Sq;
    const int hh = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const float *o = (const float *)a.o + b * a.o_sb + hh * a.o_sh + (int64_t)s * a.o_ss;
    const float *g = (const float *)a.dout + b * a.do_sb + hh * a.do_sh + (int64_t)s * a.do_ss;
    float acc = 0.f;
    for (int e = 0; e < per; ++e) acc = fmaf(o[sub * per + e], g[sub * per + e], acc);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 32);
    if (sub == 0) a.delta[row] = acc;
  }
}

// Next 32-key tile in ring order (as in the forward); t == P means done.
__device__ __forceinline__ void ring_next_f32(const BwdArgs &a, bool causal, int64_t vis_lim,
                                              int &t, int &kb, int &kend, int &cend) {
  kb += kTile;
  while (kb >= kend) {
    ++t;
    if (t >= a.num_chunks) return;
    int c = a.start_chunk + t;
    if (c >= a.num_chunks) c -= a.num_chunks;
    kb = c * a.chunk_len;
    cend = kb + a.chunk_len;
    kend = cend;
    if (causal && vis_lim < (int64_t)kend) kend = vis_lim > kb ? (int)vis_lim : kb;
  }
}

// A [32, D] fp32 tile in LDS, rows padded by 4 floats (conflict-free column reads),
// staged through registers: 256 threads, D/16 16-byte pieces each per tensor pair.
template <int D>
struct F32Tile {
  static constexpr int STR = D + 4;
  static constexpr int FLOATS = kTile * STR;
  static constexpr int PIECES = kTile * D / 4 / 256;  // float4 per thread per tensor
  struct Stage { f32x4 x[PIECES]; f32x4 y[PIECES]; };
  // rows row0 .. row0+31 of two [rows, D] matrices (row strides sx, sy); rows at or past
  // nrows read row nrows-1 (their products are masked)
  __device__ static void load(Stage &st, const float *x, int64_t sx, const float *y, int64_t sy,
                              int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int id = tid + 256 * i;
      const int r = id / (D / 4), c4 = id % (D / 4);
      const int64_t row = min(row0 + r, nrows - 1);
      st.x[i] = *(const f32x4 *)(x + row * sx + 4 * c4);
      st.y[i] = *(const f32x4 *)(y + row * sy + 4 * c4);
    }
  }
  __device__ static void store(const Stage &st, float *xs, float *ys, int tid) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int id = tid + 256 * i;
      const int r = id / (D / 4), c4 = id % (D / 4);
      *(f32x4 *)(xs + r * STR + 4 * c4) = st.x[i];
      *(f32x4 *)(ys + r * STR + 4 * c4) = st.y[i];
    }
  }
};

// row of result element i (within a 32-row block) for lane half h
__device__ __forceinline__ int crow(int i, int h) { return (i >> 2) * 8 + 4 * h + (i & 3); }

// ---------------------------------------------------------------------------------
// dQ: 4 waves x 32 query rows; the lane owns query row q0 + 32*wave + (lane & 31).
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool ACC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dq_f32_kernel(BwdArgs a, int num_q_tiles) {
  using Tile = F32Tile<D>;
  constexpr int BM = 128;
  __shared__ __attribute__((aligned(16))) float ks[Tile::FLOATS];
  __shared__ __attribute__((aligned(16))) float vs[Tile::FLOATS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int HB = a.Hq * a.B;
  const int trank = blockIdx.x / HB;
  const int j = blockIdx.x - trank * HB;
  const int hq = j % a.Hq, b = j / a.Hq, hk = hq / a.group;
  const int q0 = (num_q_tiles - 1 - trank) * BM;  // heaviest (most keys) first
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const int qrow = q0 + 32 * wave + r32;
  const int qr = min(qrow, a.Sq - 1);
  const int64_t qpos = a.q_offset + qrow;
  const float c = a.scale_log2;

  const float *qb = (const float *)a.q + b * a.q_sb + hq * a.q_sh + (int64_t)qr * a.q_ss;
  const float *db = (const float *)a.dout + b * a.do_sb + hq * a.do_sh + (int64_t)qr * a.do_ss;
  const float *kbase = (const float *)a.k + b * a.k_sb + hk * a.k_sh;
  const float *vbase = (const float *)a.v + b * a.v_sb + hk * a.v_sh;
  f32x2 qf[D / 4], df[D / 4];  // dims 4jj + 2h, +1
#pragma unroll
  for (int jj = 0; jj < D / 4; ++jj) {
    qf[jj] = *(const f32x2 *)(qb + 4 * jj + 2 * h);
    df[jj] = *(const f32x2 *)(db + 4 * jj + 2 * h);
  }
  const float lse = a.lse[b * a.l_sb + hq * a.l_sh + qr];
  const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;  // empty row: P = 0
  const float dlt = a.delta[((int64_t)b * a.Hq + hq) * a.Sq + qr];

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = f32x16{};

  const int64_t vis_lim = a.q_offset + qlast - a.kv_offset + 1;
  int t = -1, kb = 0, kend = 0, cend = 0;
  ring_next_f32(a, CAUSAL, vis_lim, t, kb, kend, cend);
  typename Tile::Stage st;
  if (t < a.num_chunks) Tile::load(st, kbase, a.k_ss, vbase, a.v_ss, kb, a.Skv, tid);
  while (t < a.num_chunks) {
    const int kb_cur = kb, cend_cur = cend;
    __syncthreads();  // the previous tile's readers are done
    Tile::store(st, ks, vs, tid);
    __syncthreads();
    ring_next_f32(a, CAUSAL, vis_lim, t, kb, kend, cend);
    if (t < a.num_chunks) Tile::load(st, kbase, a.k_ss, vbase, a.v_ss, kb, a.Skv, tid);
    if (qrow - r32 < a.Sq) {  // the wave has rows
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int jj = 0; jj < D / 4; ++jj)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = 4 * jj + 2 * h + e;
          s = mfma_f32(ks[r32 * Tile::STR + d], qf[jj][e], s);
          dp = mfma_f32(vs[r32 * Tile::STR + d], df[jj][e], dp);
        }
      // lane: query row qrow; element i: key kb_cur + crow(i, h)
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = crow(i, h);
        const int key = kb_cur + kk;
        bool vis = key < cend_cur && qrow < a.Sq;
        if (CAUSAL) vis = vis && a.kv_offset + key <= qpos;
        const float p = vis ? fast_exp2(fmaf(s[i], c, -lse2)) : 0.f;
        ds[i] = p * (dp[i] - dlt);
      }
      // dQ^T[D x 32 q] += K^T[D x 32 keys] dS^T: step t takes key crow(t, h)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dq[dt] = mfma_f32(ks[crow(i, h) * Tile::STR + 32 * dt + r32], ds[i], dq[dt]);
    }
  }

  if (qrow < a.Sq) {
    float *orow = (float *)a.dq + b * a.dq_sb + hq * a.dq_sh + (int64_t)qrow * a.dq_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 *p = (f32x4 *)(orow + 32 * dt + 8 * g + 4 * h);
        const f32x4 add = {dq[dt][4 * g] * a.scale, dq[dt][4 * g + 1] * a.scale,
                           dq[dt][4 * g + 2] * a.scale, dq[dt][4 * g + 3] * a.scale};
        if (ACC) {
          const f32x4 prev = *p;
          *p = f32x4{prev[0] + add[0], prev[1] + add[1], prev[2] + add[2], prev[3] + add[3]};
        } else {
          *p = add;
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV: 4 waves x 32 keys; the lane owns key k0 + 32*wave + (lane & 31).
// ---------------------------------------------------------------------------------
constexpr int kAccDims = 64;  // head dims of dK, dV accumulated per workgroup

template <int D, bool CAUSAL, bool ACC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_f32_kernel(BwdArgs a, int num_kv_tiles) {
  constexpr int NDT = kAccDims / 32;  // 32-dim blocks of the accumulators
  const int dt0 = blockIdx.y * NDT;   // first accumulated 32-dim block
  using Tile = F32Tile<D>;
  constexpr int BK = 128;
  __shared__ __attribute__((aligned(16))) float qs[Tile::FLOATS];
  __shared__ __attribute__((aligned(16))) float gs[Tile::FLOATS];
  __shared__ float st_lse2[kTile], st_dlt[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int HB = a.Hkv * a.B;
  const int kt_i = blockIdx.x / HB;
  const int j = blockIdx.x - kt_i * HB;
  const int hk = j % a.Hkv, b = j / a.Hkv;
  const int k0 = kt_i * BK;
  const int krow = k0 + 32 * wave + r32;
  const int kr = min(krow, a.Skv - 1);
  const int64_t kpos = a.kv_offset + krow;
  const float c = a.scale_log2;
  (void)num_kv_tiles;

  const float *kb_ = (const float *)a.k + b * a.k_sb + hk * a.k_sh + (int64_t)kr * a.k_ss;
  const float *vb_ = (const float *)a.v + b * a.v_sb + hk * a.v_sh + (int64_t)kr * a.v_ss;
  f32x2 kf[D / 4], vf[D / 4];
#pragma unroll
  for (int jj = 0; jj < D / 4; ++jj) {
    kf[jj] = *(const f32x2 *)(kb_ + 4 * jj + 2 * h);
    vf[jj] = *(const f32x2 *)(vb_ + 4 * jj + 2 * h);
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // first query row that can see the block's first key (causal), as a tile start
  int qstart = 0;
  if (CAUSAL) {
    const int64_t first = a.kv_offset + k0 - a.q_offset;
    qstart = first <= 0 ? 0 : (first >= (int64_t)a.Sq ? a.Sq : (int)first);
    qstart = (qstart / kTile) * kTile;
  }
  const int nqt = qstart >= a.Sq ? 0 : (a.Sq - qstart + kTile - 1) / kTile;
  const int total = nqt * a.group;
  const bool wave_active = k0 + 32 * wave < a.Skv;

  typename Tile::Stage st;
  float sv = 0.f;
  auto fetch = [&](int it) {
    const int hq = hk * a.group + it / nqt;
    const int q0 = qstart + (it % nqt) * kTile;
    const float *qb = (const float *)a.q + b * a.q_sb + hq * a.q_sh;
    const float *gb = (const float *)a.dout + b * a.do_sb + hq * a.do_sh;
    Tile::load(st, qb, a.q_ss, gb, a.do_ss, q0, a.Sq, tid);
    const int q = min(q0 + (tid & 31), a.Sq - 1);
    if (tid < 32) {
      const float l = a.lse[b * a.l_sb + hq * a.l_sh + q];
      sv = l == -INFINITY ? INFINITY : l * kLog2e;
    } else if (tid < 64) {
      sv = a.delta[((int64_t)b * a.Hq + hq) * a.Sq + q];
    }
  };
  if (total > 0) fetch(0);
  for (int it = 0; it < total; ++it) {
    const int q0 = qstart + (it % nqt) * kTile;
    __syncthreads();
    Tile::store(st, qs, gs, tid);
    if (tid < 32) st_lse2[tid] = sv;
    else if (tid < 64) st_dlt[tid - 32] = sv;
    __syncthreads();
    const int64_t qpos0 = a.q_offset + q0;
    if (wave_active && !(CAUSAL && a.kv_offset + k0 + 32 * wave > qpos0 + kTile - 1)) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int jj = 0; jj < D / 4; ++jj) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = 4 * jj + 2 * h + e;
          s = mfma_f32(qs[r32 * Tile::STR + d], kf[jj][e], s);
          dp = mfma_f32(gs[r32 * Tile::STR + d], vf[jj][e], dp);
        }
      }
      // lane: key krow; element i: query row q0 + crow(i, h).  P and dS replace S and dP
      // in place (register pressure: one wave holds K^T, V^T and the dK, dV accumulators)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = crow(i, h);
        bool vis = q0 + qi < a.Sq && krow < a.Skv;
        if (CAUSAL) vis = vis && kpos <= qpos0 + qi;
        const float pv = vis ? fast_exp2(fmaf(s[i], c, -st_lse2[qi])) : 0.f;
        s[i] = pv;
        dp[i] = pv * (dp[i] - st_dlt[qi]);
      }
      // dV^T[D x 32 keys] += dO^T[D x 32 q] P, dK^T += Q^T dS: step i takes row crow(i, h)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = crow(i, h) * Tile::STR + 32 * (dt0 + dt) + r32;
          dv[dt] = mfma_f32(gs[row], s[i], dv[dt]);
          dk[dt] = mfma_f32(qs[row], dp[i], dk[dt]);
        }
    }
    // the next tile's loads after this tile's products: their staging registers are not
    // live across the products (the wave already holds ~320 values)
    if (it + 1 < total) fetch(it + 1);
  }

  if (krow < a.Skv) {
    float *krow_dk = (float *)a.dk + b * a.dk_sb + hk * a.dk_sh + (int64_t)krow * a.dk_ss;
    float *krow_dv = (float *)a.dv + b * a.dv_sb + hk * a.dv_sh + (int64_t)krow * a.dv_ss;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * (dt0 + dt) + 8 * g + 4 * h;
        const f32x4 k4 = {dk[dt][4 * g] * a.scale, dk[dt][4 * g + 1] * a.scale,
                          dk[dt][4 * g + 2] * a.scale, dk[dt][4 * g + 3] * a.scale};
        const f32x4 v4 = {dv[dt][4 * g], dv[dt][4 * g + 1], dv[dt][4 * g + 2], dv[dt][4 * g + 3]};
        f32x4 *pk = (f32x4 *)(krow_dk + d);
        f32x4 *pv = (f32x4 *)(krow_dv + d);
        if (ACC) {
          const f32x4 ok = *pk, ov = *pv;
          *pk = f32x4{ok[0] + k4[0], ok[1] + k4[1], ok[2] + k4[2], ok[3] + k4[3]};
          *pv = f32x4{ov[0] + v4[0], ov[1] + v4[1], ov[2] + v4[2], ov[3] + v4[3]};
        } else {
          *pk = k4;
          *pv = v4;
        }
      }
  }
}

template <int D, bool CAUSAL, bool ACC>
int launch_f32(const BwdArgs &a, hipStream_t stream) {
  {
    const int64_t nrows = (int64_t)a.B * a.Hq * a.Sq;
    int64_t blocks = (nrows + 7) / 8;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (blocks > 0)
      hipLaunchKernelGGL(bwd_delta_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, D);
  }
  {
    const int nkt = (a.Skv + 127) / 128;
    const int64_t blocks = (int64_t)nkt * a.Hkv * a.B;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, ACC>),
                         dim3((unsigned)blocks, D / kAccDims), dim3(256), 0, stream, a, nkt);
  }
  {
    const int nqt = (a.Sq + 127) / 128;
    const int64_t blocks = (int64_t)nqt * a.Hq * a.B;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, ACC>), dim3((unsigned)blocks), dim3(256),
                         0, stream, a, nqt);
  }
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace

int launch_attn_bwd_f32(const BwdArgs &a, int D, int causal, bool acc, hipStream_t stream) {
  if (D == 128) {
    if (acc) return causal ? launch_f32<128, true, true>(a, stream) : launch_f32<128, false, true>(a, stream);
    return causal ? launch_f32<128, true, false>(a, stream) : launch_f32<128, false, false>(a, stream);
  }
  if (D == 64) {
    if (acc) return causal ? launch_f32<64, true, true>(a, stream) : launch_f32<64, false, true>(a, stream);
    return causal ? launch_f32<64, true, false>(a, stream) : launch_f32<64, false, false>(a, stream);
  }
  return RA_ERR_UNSUPPORTED;
}

}  // namespace ra
