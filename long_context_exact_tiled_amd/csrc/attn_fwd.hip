// attn_fwd -- exact softmax attention of a query block over P key/value chunks in ring
// order, with the running row max and exponential sum carried across chunks.
//
// Sources (page title, host):
//   [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn),
//        section "Ring-Attention：面向大规模部署的工程利器": the sequence split into P
//        chunks, local max and exponential sums combined into global statistics.
//   [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com): the ring_attention_forward
//        listing -- a device's local Q visits every K/V block in turn, folding each
//        step into a log-space accumulator.
//   [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn),
//        section "FlashAttention 如何破局？不只是融合内核": Q, K, V tiled along the sequence,
//        each block keeps a Q tile on chip while K/V tiles stream through, the online
//        softmax keeps a running max and normaliser, only the output is written back.
//
// Design on gfx950 (CDNA4):
//   * one workgroup = 4 wavefronts = 128 query rows (32 per wave) of one (batch, head);
//   * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global loads
//     are issued before the current tile's math and land in the other buffer after it;
//   * scores are computed transposed, S^T = K Q^T, so each lane owns ONE query row
//     (column l%32 of the MFMA output) and 16 of the 32 keys of each 32-key block:
//     the row max / row sum are 32 in-register ops plus one v_permlane32_swap;
//   * P^T stays in registers and feeds O^T += V^T P^T directly (the MFMA output
//     layout of S^T is the B-operand layout of the next MFMA once the k order of V^T
//     is chosen to match); V is transposed on its way into LDS for the bf16 path;
//   * exponentials are base 2 with scale*log2(e) folded into one FMA per score;
//   * the ring walk skips chunks (and tiles) that lie entirely after the block's last
//     query position under the causal mask; only tiles that straddle the diagonal or a
//     chunk end pay for the element mask.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // keys per tile

// ---------------------------------------------------------------------------------
// Ring walk: tiles of BN keys, chunk by chunk in the order (start + t) mod P.  Inside
// a chunk, tiles stop at the last key any query row of the block can see.
// ---------------------------------------------------------------------------------
struct RingWalk {
  int P, start, L;
  bool causal;
  int64_t vis_lim;  // keys with local index < vis_lim are visible to the block's last row

  int t, kb, kend, cend;  // ring step, tile start, visible end of chunk, chunk end

  __device__ void init(const FwdArgs &a, bool causal_, int64_t qpos_hi) {
    P = a.num_chunks;
    start = a.start_chunk;
    L = a.chunk_len;
    causal = causal_;
    vis_lim = qpos_hi - a.kv_offset + 1;
    t = -1;
    kb = 0;
    kend = 0;
    cend = 0;
    advance();
  }
  __device__ bool valid() const { return t < P; }
  __device__ void advance() {
    kb += BN;
    while (kb >= kend) {
      ++t;
      if (t >= P) return;
      int c = start + t;
      if (c >= P) c -= P;
      kb = c * L;
      cend = kb + L;
      kend = cend;
      if (causal && vis_lim < (int64_t)kend) kend = vis_lim > kb ? (int)vis_lim : kb;
    }
  }
};

// ---------------------------------------------------------------------------------
// bf16 traits: 32x32x16 bf16 MFMA; K row-major in LDS, V transposed in LDS.
// ---------------------------------------------------------------------------------
template <int D>
struct Bf16Path {
  using elem_t = uint16_t;
  static constexpr int KSTR = D + 8;    // K row stride (elements): 16-byte pad
  static constexpr int VSTR = BN + 4;   // V^T row stride: 34 dwords, conflict-free reads
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 2;
  static constexpr int KCH = BN * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int VBC = D / 8;                   // 8-wide column groups of V
  static constexpr int VBLK = (BN / 4) * VBC;         // 4x8 V blocks per tile

  struct QFrag { bf16x8 x[D / 16]; };
  struct Stage { u32x4 k[KCH]; u32x4 v[4]; };

  __device__ static void load_q(QFrag &qf, const FwdArgs &a, const elem_t *qbase, int qrow, int h) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (qrow < a.Sq) u = *(const u32x4 *)(qbase + (int64_t)qrow * a.q_ss + ks * 16 + 8 * h);
      qf.x[ks] = as_bf16x8(u);
    }
  }

  __device__ static void load_tile(Stage &st, const FwdArgs &a, const elem_t *kbase,
                                   const elem_t *vbase, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int id = tid + kThreads * i;
      int row = id / (D / 8), c8 = id % (D / 8);
      int kv = kb + row;
      u32x4 u = {0u, 0u, 0u, 0u};
      if (kv < a.Skv) u = *(const u32x4 *)(kbase + (int64_t)kv * a.k_ss + c8 * 8);
      st.k[i] = u;
    }
    if (tid < VBLK) {
      int r = tid / VBC, c = tid % VBC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int kv = kb + 4 * r + i;
        u32x4 u = {0u, 0u, 0u, 0u};
        if (kv < a.Skv) u = *(const u32x4 *)(vbase + (int64_t)kv * a.v_ss + c * 8);
        st.v[i] = u;
      }
    }
  }

  __device__ static void store_tile(const Stage &st, elem_t *buf, int tid) {
    elem_t *Ks = buf;
    elem_t *Vt = buf + K_ELEMS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int id = tid + kThreads * i;
      int row = id / (D / 8), c8 = id % (D / 8);
      *(u32x4 *)(Ks + row * KSTR + c8 * 8) = st.k[i];
    }
    if (tid < VBLK) {
      int r = tid / VBC, c = tid % VBC;
      // 4 keys x 8 dims -> 8 dims x 4 keys (transpose through byte permutes)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const int w = j >> 1;
        uint32_t lo = perm_b32(st.v[1][w], st.v[0][w], sel);
        uint32_t hi = perm_b32(st.v[3][w], st.v[2][w], sel);
        u32x2 pr = {lo, hi};
        *(u32x2 *)(Vt + (c * 8 + j) * VSTR + 4 * r) = pr;
      }
    }
  }

  // S^T[32 keys x 32 queries] for the two 32-key halves of the tile.
  __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const elem_t *buf, int lane) {
    const elem_t *Ks = buf;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) s[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        u32x4 kf = *(const u32x4 *)(Ks + (32 * mt + r) * KSTR + ks * 16 + 8 * h);
        s[mt] = mfma_bf16(as_bf16x8(kf), qf.x[ks], s[mt]);
      }
    }
  }

  // O^T[D x 32 queries] += V^T P^T, P^T taken from the S^T registers (already exp'd).
  __device__ static void pv(f32x16 (&o)[D / 32], const f32x16 (&p)[2], const elem_t *buf,
                            int lane) {
    const elem_t *Vt = buf + K_ELEMS;
    const int r = lane & 31, h = lane >> 5;
    u32x4 pf[4];
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int mt = kstep >> 1, s2 = kstep & 1;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        pf[kstep][w] = pack_bf16x2(p[mt][8 * s2 + 2 * w], p[mt][8 * s2 + 2 * w + 1]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int kstep = 0; kstep < 4; ++kstep) {
        const elem_t *row = Vt + (32 * dt + r) * VSTR + 16 * kstep + 4 * h;
        u32x2 a0 = *(const u32x2 *)row;
        u32x2 a1 = *(const u32x2 *)(row + 8);
        u32x4 af = {a0[0], a0[1], a1[0], a1[1]};
        o[dt] = mfma_bf16(as_bf16x8(af), as_bf16x8(pf[kstep]), o[dt]);
      }
    }
  }
};

// ---------------------------------------------------------------------------------
// fp32 traits: 32x32x2 fp32 MFMA; K and V row-major in LDS.
// ---------------------------------------------------------------------------------
template <int D>
struct F32Path {
  using elem_t = float;
  static constexpr int KSTR = D + 4;
  static constexpr int VSTR = D + 4;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = BN * VSTR;
  static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 4;
  static constexpr int CH = BN * D / 4 / kThreads;  // 16-byte chunks per thread, per tensor

  struct QFrag { f32x2 x[D / 4]; };
  struct Stage { u32x4 k[CH]; u32x4 v[CH]; };

  // MFMA step 2j+e of half h uses head dim 4j + 2h + e (A and B agree).
  __device__ static void load_q(QFrag &qf, const FwdArgs &a, const elem_t *qbase, int qrow, int h) {
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      f32x2 u = {0.f, 0.f};
      if (qrow < a.Sq) u = *(const f32x2 *)(qbase + (int64_t)qrow * a.q_ss + 4 * j + 2 * h);
      qf.x[j] = u;
    }
  }

  __device__ static void load_tile(Stage &st, const FwdArgs &a, const elem_t *kbase,
                                   const elem_t *vbase, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      int id = tid + kThreads * i;
      int row = id / (D / 4), c4 = id % (D / 4);
      int kv = kb + row;
      u32x4 uk = {0u, 0u, 0u, 0u}, uv = {0u, 0u, 0u, 0u};
      if (kv < a.Skv) {
        uk = *(const u32x4 *)(kbase + (int64_t)kv * a.k_ss + c4 * 4);
        uv = *(const u32x4 *)(vbase + (int64_t)kv * a.v_ss + c4 * 4);
      }
      st.k[i] = uk;
      st.v[i] = uv;
    }
  }

  __device__ static void store_tile(const Stage &st, elem_t *buf, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      int id = tid + kThreads * i;
      int row = id / (D / 4), c4 = id % (D / 4);
      *(u32x4 *)(buf + row * KSTR + c4 * 4) = st.k[i];
      *(u32x4 *)(buf + K_ELEMS + row * VSTR + c4 * 4) = st.v[i];
    }
  }

  __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const elem_t *buf, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) s[mt] = f32x16{};
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x2 kf = *(const f32x2 *)(buf + (32 * mt + r) * KSTR + 4 * j + 2 * h);
        s[mt] = mfma_f32(kf[0], qf.x[j][0], s[mt]);
        s[mt] = mfma_f32(kf[1], qf.x[j][1], s[mt]);
      }
    }
  }

  __device__ static void pv(f32x16 (&o)[D / 32], const f32x16 (&p)[2], const elem_t *buf,
                            int lane) {
    const elem_t *Vs = buf + K_ELEMS;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kv = 32 * mt + (i >> 2) * 8 + 4 * h + (i & 3);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = mfma_f32(Vs[kv * VSTR + 32 * dt + r], p[mt][i], o[dt]);
      }
    }
  }
};

// ---------------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------------
template <class Path, int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(FwdArgs a) {
  using elem_t = typename Path::elem_t;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * Path::BUF_BYTES];
  auto buf_at = [&](int i) { return (elem_t *)(smem + i * Path::BUF_BYTES); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int h = lane >> 5;

  // Heaviest query tiles first (causal work grows with the tile index), heads fastest.
  const int bid = blockIdx.x;
  const int per_tile = a.Hq * a.B;
  const int qt = a.num_q_tiles - 1 - bid / per_tile;
  const int rest = bid % per_tile;
  const int hq = rest % a.Hq;
  const int b = rest / a.Hq;
  const int hk = hq / a.group;

  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const elem_t *qbase = (const elem_t *)a.q + b * a.q_sb + hq * a.q_sh;
  const elem_t *kbase = (const elem_t *)a.k + b * a.k_sb + hk * a.k_sh;
  const elem_t *vbase = (const elem_t *)a.v + b * a.v_sb + hk * a.v_sh;

  // This lane's query row and the wave's row range (global positions).
  const int qrow = q0 + 32 * wave + r32;
  const int64_t qpos = a.q_offset + qrow;
  const int64_t wpos_first = a.q_offset + q0 + 32 * wave;
  const int64_t wpos_last = wpos_first + 31;
  const bool wave_active = (q0 + 32 * wave) < a.Sq;

  typename Path::QFrag qf;
  Path::load_q(qf, a, qbase, qrow, h);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max, scaled log2 domain (scale*log2e*s)
  float l_run = 0.f;        // running exp-sum of this lane's keys (halves summed at the end)

  RingWalk walk;
  walk.init(a, CAUSAL, a.q_offset + qlast);

  typename Path::Stage st;
  if (walk.valid()) {
    Path::load_tile(st, a, kbase, vbase, walk.kb, tid);
    Path::store_tile(st, buf_at(0), tid);
  }
  __syncthreads();

  int cur = 0;
  while (walk.valid()) {
    const int kb = walk.kb;
    const int cend = walk.cend;
    RingWalk nxt = walk;
    nxt.advance();
    if (nxt.valid()) Path::load_tile(st, a, kbase, vbase, nxt.kb, tid);

    const int64_t kpos0 = a.kv_offset + kb;
    const int kvalid = min(BN, cend - kb);  // keys of this tile inside the chunk
    const bool skip = !wave_active || (CAUSAL && kpos0 > wpos_last);
    if (!skip) {
      f32x16 s[2];
      Path::qk(s, qf, buf_at(cur), lane);

      const bool need_mask =
          (kvalid < BN) || (CAUSAL && kpos0 + kvalid - 1 > wpos_first);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * mt + (i >> 2) * 8 + 4 * h + (i & 3);
            bool vis = kk < kvalid;
            if (CAUSAL) vis = vis && (kpos0 + kk <= qpos);
            s[mt][i] = vis ? s[mt][i] : -INFINITY;
          }
      }
      // online softmax (base 2)
      float mx = s[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mt][i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(fmaf(s[mt][i], a.scale_log2, -m_use));
          s[mt][i] = pv;
          rs += pv;
        }
      l_run = fmaf(l_run, alpha, rs);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      Path::pv(o, s, buf_at(cur), lane);
    }

    if (nxt.valid()) Path::store_tile(st, buf_at(cur ^ 1), tid);
    __syncthreads();
    cur ^= 1;
    walk = nxt;
  }

  // Epilogue: o = O / l, lse = ln(sum) = (m + log2 l) * ln 2.
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < a.Sq) {
    if (h == 0) {
      float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      a.lse[b * a.l_sb + hq * a.l_sh + qrow] = lse;
    }
    const int64_t orow = b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        float x0 = o[dt][4 * g + 0] * inv, x1 = o[dt][4 * g + 1] * inv;
        float x2 = o[dt][4 * g + 2] * inv, x3 = o[dt][4 * g + 3] * inv;
        if (a.o_is_f32) {
          float4 w = {x0, x1, x2, x3};
          *(float4 *)((float *)a.o + orow + d) = w;
        } else {
          u32x2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          *(u32x2 *)((uint16_t *)a.o + orow + d) = w;
        }
      }
  }
}

template <class Path, int D, bool CAUSAL>
int launch_one(const FwdArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.num_q_tiles * a.Hq * a.B;
  if (blocks <= 0) return RA_OK;
  hipLaunchKernelGGL((attn_fwd_kernel<Path, D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace

int launch_attn_fwd(const FwdArgs &args, int dtype, int D, int causal, hipStream_t stream) {
  FwdArgs a = args;
  a.num_q_tiles = (a.Sq + BM - 1) / BM;
  if (dtype == RA_BF16) {
    if (D == 128) return causal ? launch_one<Bf16Path<128>, 128, true>(a, stream)
                                : launch_one<Bf16Path<128>, 128, false>(a, stream);
    if (D == 64) return causal ? launch_one<Bf16Path<64>, 64, true>(a, stream)
                               : launch_one<Bf16Path<64>, 64, false>(a, stream);
  } else if (dtype == RA_F32) {
    if (D == 128) return causal ? launch_one<F32Path<128>, 128, true>(a, stream)
                                : launch_one<F32Path<128>, 128, false>(a, stream);
    if (D == 64) return causal ? launch_one<F32Path<64>, 64, true>(a, stream)
                               : launch_one<F32Path<64>, 64, false>(a, stream);
  }
  return RA_ERR_UNSUPPORTED;
}

}  // namespace ra
