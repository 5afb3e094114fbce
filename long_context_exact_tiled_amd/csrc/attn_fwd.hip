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
// Design on gfx950 (CDNA4), from measured rates (MFMA 32x32x16 bf16 ~37 clk/SIMD;
// v_exp_f32 ~4-5x a plain VALU op; ds_read_b128 ~190 B/clk/CU vs ~120 for b64):
//   * bf16 (attn_fwd_direct_kernel): one workgroup = 8 wavefronts = 256 query rows (32
//     per wave) of one (batch, head), two waves per SIMD, so one wave's softmax (VALU)
//     runs under the other's MFMAs; all 8 waves share each K/V tile in LDS;
//   * K/V tiles of 128 keys go straight from global memory into LDS
//     (global_load_lds_dwordx4), double-buffered, XOR-swizzled so every operand read is
//     bank-conflict free; the next tile's loads are in flight under the current tile's
//     math and are issued by one wave per SIMD only, which staggers the two waves of a
//     SIMD;
//   * scores are computed transposed, S^T = K Q^T (Q stays in registers as the B
//     operand): each lane owns ONE query row and 16 of each 32 keys, so the row max is
//     in-register v_max3 plus one v_permlane32_swap and the row sum needs no shuffle;
//   * P^T feeds O^T += V^T P^T straight from registers; the V^T operand comes from the
//     row-major V tile through the transposing LDS read (ds_read_b64_tr_b16);
//   * exp2 with scale*log2(e) folded into one FMA per score; P rounded to bf16 with one
//     v_cvt_pk per pair for the PV MFMA, while the row sum adds the fp32 values;
//   * lazy rescale: the running max only moves (and O, l are only rescaled) when a
//     tile's max exceeds it by more than 2^8; otherwise P <= 256, which fp32 and bf16
//     hold exactly as well as P <= 1.  The final o = O / l and lse = m + log2 l use the
//     same max, so the result is unchanged;
//   * the ring walk skips chunks (and tiles) that lie entirely after the block's last
//     query position under the causal mask; only tiles that straddle the diagonal or a
//     chunk end pay for the element mask; waves whose rows all precede a tile skip it;
//   * heaviest query tiles first (causal work grows with the tile index); with 8 | B*Hq
//     the heads are grouped so that each XCD sees a fixed subset of them, otherwise the
//     workgroups take their tiles from a work counter in start order;
//   * fp32 (attn_fwd_kernel<F32Path>): the same walk and softmax with 32x32x2 fp32 MFMAs,
//     64-key tiles staged through registers into LDS.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int BN = 64;           // keys per tile of the fp32 path
constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kDirectWaves = 8;  // waves per workgroup on the bf16 path (32 query rows each)
constexpr int kDirectKN = 128;   // keys per tile on the bf16 path (measured 3.6 % faster than 64)
static_assert(kDirectKN <= kMaxTileRows && BN <= kMaxTileRows, "tile offsets are 32-bit");


// ---------------------------------------------------------------------------------
// bf16 direct path: K and V go straight from global memory into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l), dense and
// XOR-swizzled so that every MFMA operand read is bank-conflict free.  V stays
// row-major; its transposed MFMA operand comes from ds_read_b64_tr_b16, which within
// each 16-lane group hands lane 4a+b the b-th 16-bit element of the 8-byte pieces
// addressed by lanes a, a+4, a+8, a+12.  No staging registers, no transpose ALU work
// and no LDS store instructions.
// ---------------------------------------------------------------------------------
template <int D, int NW = 8, int KN = BN>
struct Bf16DirectPath {
  static constexpr int NMT = KN / 32;              // 32-key S^T tiles per key tile
  using elem_t = uint16_t;
  static constexpr int kWaves = NW;                // 32 query rows per wave
  static constexpr int kThreads = 64 * NW;
  static constexpr int RB = 2 * D;                 // row bytes
  static constexpr int TILE_BYTES = KN * RB;       // one of K or V
  static constexpr int BUF_BYTES = 2 * TILE_BYTES; // K then V
  static constexpr int NBLK = TILE_BYTES / 1024;   // 1-KiB load blocks per tensor
  static constexpr int BPW = NBLK / kWaves;        // blocks per wave per tensor
  static constexpr int RSTEP = kWaves * 1024 / RB;  // rows between a lane's pieces
  static_assert((kWaves * 1024) % RB == 0 && RSTEP % 16 == 0,
                "a lane's pieces share the in-row chunk (swizzles repeat every 16 rows)");
  static constexpr int kDepth = 4;                 // K operand reads in flight
  static constexpr int kVDepth = 2;                // V operand MFMAs in flight
  static_assert(NBLK % kWaves == 0, "tile must split evenly over the waves");

  // swizzles (16-byte chunk index within a row)
  __device__ static int ksw(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int vsw(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

  struct QFrag { bf16x8 x[D / 16]; };
  struct PFrag { u32x4 x[KN / 16]; };
  struct Lane {
    int k_goff[BPW], v_goff[BPW];  // byte offsets of this lane's 16 B in the tile (row 0 = kb)
    int row0;                      // tile row of piece 0; piece i is RSTEP*i rows further
    int k_chunk, v_chunk;          // the 16-byte chunk within the row (the same for every i)
    // operand read addresses per LDS slot: K for head-dim step ks, V^T for block dt
    // (the swizzle XORs applied); block offsets within a slot are immediates
    uint32_t kx[2][D / 16], vx[2][D / 32];
  };

  __device__ static void setup(Lane &L, const FwdArgs &a, int tid, uint32_t smem_base) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = wave + kWaves * i;
      const int byte = blk * 1024 + 16 * lane;
      const int r = byte / RB, p = (byte % RB) / 16;
      if (i == 0) {
        L.row0 = r;
        L.k_chunk = p ^ ksw(r);
        L.v_chunk = p ^ vsw(r);
      }
      L.k_goff[i] = (int)(r * a.k_ss * 2) + 16 * L.k_chunk;
      L.v_goff[i] = (int)(r * a.v_ss * 2) + 16 * L.v_chunk;
    }
    const int r = lane & 31, h = lane >> 5;
    const uint32_t ka = smem_base + (uint32_t)(r * RB + 16 * (ksw(r) ^ h));
    const int g = lane >> 4, ap = lane & 15, z = ap >> 2;
    const int w = 2 * (g & 1) + ((ap & 3) >> 1);
    const int zz = D == 128 ? z : (z >> 1);
    const uint32_t vb = smem_base + TILE_BYTES +
                        (uint32_t)((4 * h + z) * RB + 64 * zz + 16 * w + 8 * (ap & 1));
    // The slot-1 addresses pass through an empty asm so that the compiler keeps them in
    // registers instead of re-deriving them as slot-0 address + 64 KiB (too large for
    // the 16-bit immediate of an LDS read).
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        L.kx[sl][ks] = (ka ^ (uint32_t)(32 * ks)) + sl * BUF_BYTES;
        if (sl) asm volatile("" : "+v"(L.kx[sl][ks]));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        L.vx[sl][dt] = (vb ^ (uint32_t)(64 * dt)) + sl * BUF_BYTES;
        if (sl) asm volatile("" : "+v"(L.vx[sl][dt]));
      }
    }
  }

  __device__ static void load_q(QFrag &qf, const FwdArgs &a, const elem_t *qbase, int qrow, int h) {
    const int row = min(qrow, a.Sq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf.x[ks] = as_bf16x8(*(const u32x4 *)(qbase + (int64_t)row * a.q_ss + ks * 16 + 8 * h));
  }

  // Issue the direct loads of the tile starting at key kb into the LDS slot at byte
  // offset `slot` (from the start of LDS).
  __device__ static void load_tile(const Lane &L, const FwdArgs &a, const elem_t *kbase,
                                   const elem_t *vbase, int kb, uint32_t slot, int wave) {
    const bool tail = kb + KN > a.Skv;
    const elem_t *kt = kbase + (int64_t)kb * a.k_ss;
    const elem_t *vt = vbase + (int64_t)kb * a.v_ss;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane(wave + kWaves * i);
      int koff = L.k_goff[i], voff = L.v_goff[i];
      if (tail) {  // rows past the end read the last row (their scores are masked)
        const int r = min(kb + L.row0 + RSTEP * i, a.Skv - 1) - kb;
        koff = (int)(r * a.k_ss * 2) + 16 * L.k_chunk;
        voff = (int)(r * a.v_ss * 2) + 16 * L.v_chunk;
      }
      dma_b128(kt, koff, slot + blk * 1024);
      dma_b128(vt, voff, slot + TILE_BYTES + blk * 1024);
    }
  }

  __device__ static u32x4 k_frag(const Lane &L, int sl, int step) {
    const int ks = step / NMT, mt = step % NMT;
    return lds_read_b128(L.kx[sl][ks] + (uint32_t)(mt * 32 * RB));
  }

  // S^T[32 keys x 32 queries] for the 32-key blocks of the tile in LDS slot sl.
  __device__ static void qk(f32x16 (&s)[NMT], const QFrag &qf, const Lane &L, int sl) {
    constexpr int NSTEP = NMT * (D / 16);
    u32x4 kf[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) kf[i] = k_frag(L, sl, i);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) s[mt] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      const int ks = step / NMT, mt = step % NMT;
      s[mt] = mfma_bf16(as_bf16x8(kf[step % kDepth]), qf.x[ks], s[mt]);
      if (step + kDepth < NSTEP) kf[step % kDepth] = k_frag(L, sl, step + kDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  __device__ static float exp_pack(const f32x16 (&s)[NMT], float c, float mneg, PFrag &pf) {
    float acc0 = -0.f, acc1 = -0.f;  // x + -0 is x: the first additions fold away
#pragma unroll
    for (int kstep = 0; kstep < KN / 16; ++kstep) {
      const int mt = kstep >> 1, s2 = kstep & 1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(fmaf(s[mt][8 * s2 + 2 * w], c, mneg));
        const float p1 = fast_exp2(fmaf(s[mt][8 * s2 + 2 * w + 1], c, mneg));
        const bf16x2 pk = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
        pf.x[kstep][w] = __builtin_bit_cast(uint32_t, pk);
        acc0 += p0;
        acc1 += p1;
      }
    }
    return acc0 + acc1;
  }

  // V^T operand for PV step (kstep, dt): two transposing 8-byte reads (keys
  // 16*kstep + 4h + 0..3 and + 8), matching the k order of the P^T registers.
  __device__ static u32x4 v_frag(const Lane &L, int sl, int step) {
    const int kstep = step / (D / 32), dt = step % (D / 32);
    const uint32_t base = L.vx[sl][dt] + (uint32_t)(16 * kstep * RB);
    const s16x4 lo = lds_read_tr16_b64(base);
    const s16x4 hi = lds_read_tr16_b64(base + 8 * RB);
    u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }

  __device__ static void pv(f32x16 (&o)[D / 32], const PFrag &pf, const Lane &L, int sl) {
    constexpr int NSTEP = (KN / 16) * (D / 32);
    u32x4 vf[kVDepth];
#pragma unroll
    for (int i = 0; i < kVDepth; ++i) vf[i] = v_frag(L, sl, i);
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      const int kstep = step / (D / 32), dt = step % (D / 32);
      o[dt] = mfma_bf16(as_bf16x8(vf[step % kVDepth]), as_bf16x8(pf.x[kstep]), o[dt]);
      if (step + kVDepth < NSTEP) vf[step % kVDepth] = v_frag(L, sl, step + kVDepth);
    }
  }
};

// ---------------------------------------------------------------------------------
// fp32 path: 32x32x2 fp32 MFMA; K and V row-major in LDS; P stays fp32.
// ---------------------------------------------------------------------------------
template <int D>
struct F32Path {
  using elem_t = float;
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int KSTR = D + 4;
  static constexpr int VSTR = D + 4;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = BN * VSTR;
  static constexpr int BUF_BYTES = (K_ELEMS + V_ELEMS) * 4;
  static constexpr int CH = BN * D / 4 / kThreads;  // 16-byte chunks per thread, per tensor

  struct QFrag { f32x2 x[D / 4]; };
  struct Stage { u32x4 k[CH]; u32x4 v[CH]; };
  struct PFrag { f32x16 x[2]; };

  // MFMA step 2j+e of half h uses head dim 4j + 2h + e (A and B agree).
  __device__ static void load_q(QFrag &qf, const FwdArgs &a, const elem_t *qbase, int qrow, int h) {
    const int row = min(qrow, a.Sq - 1);
#pragma unroll
    for (int j = 0; j < D / 4; ++j)
      qf.x[j] = *(const f32x2 *)(qbase + (int64_t)row * a.q_ss + 4 * j + 2 * h);
  }

  __device__ static void load_tile(Stage &st, const FwdArgs &a, const elem_t *kbase,
                                   const elem_t *vbase, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + kThreads * i;
      const int row = id / (D / 4), c4 = id % (D / 4);
      const int kv = min(kb + row, a.Skv - 1);
      st.k[i] = *(const u32x4 *)(kbase + (int64_t)kv * a.k_ss + c4 * 4);
      st.v[i] = *(const u32x4 *)(vbase + (int64_t)kv * a.v_ss + c4 * 4);
    }
  }

  __device__ static void store_tile(const Stage &st, elem_t *buf, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int id = tid + kThreads * i;
      const int row = id / (D / 4), c4 = id % (D / 4);
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
        const f32x2 kf = *(const f32x2 *)(buf + (32 * mt + r) * KSTR + 4 * j + 2 * h);
        s[mt] = mfma_f32(kf[0], qf.x[j][0], s[mt]);
        s[mt] = mfma_f32(kf[1], qf.x[j][1], s[mt]);
      }
    }
  }

  __device__ static float exp_pack(const f32x16 (&s)[2], float c, float mneg, PFrag &pf) {
    float acc = -0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[mt][i], c, mneg));
        pf.x[mt][i] = p;
        acc += p;
      }
    return acc;
  }

  struct VPre {};
  __device__ static void pv_prefetch(VPre &, const elem_t *, int) {}
  __device__ static void pv(f32x16 (&o)[D / 32], const PFrag &pf, VPre &, const elem_t *buf,
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
          o[dt] = mfma_f32(Vs[kv * VSTR + 32 * dt + r], pf.x[mt][i], o[dt]);
      }
    }
  }
};

// Next tile of the ring walk: tiles of BN keys, chunk by chunk in the order
// (start + t) mod P; inside a chunk, tiles stop at the last key visible to the
// block's last query row (vis_lim).  t == P means done.
template <int KN = BN>
__device__ __forceinline__ void ring_next(const FwdArgs &a, bool causal, int64_t vis_lim,
                                          int &t, int &kb, int &kend, int &cend) {
  kb += KN;
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

// ---------------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------------
template <class Path, int D, bool CAUSAL>
__global__ void __launch_bounds__(Path::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(FwdArgs a) {
  using elem_t = typename Path::elem_t;
  constexpr int BM = 32 * Path::kWaves;  // query rows per workgroup
  constexpr int NBUF = 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * Path::BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int r32 = lane & 31;
  const int h = lane >> 5;

  // Workgroup -> (query tile, head, batch): heaviest tiles first; when the head count
  // is a multiple of 8, the heads a workgroup id maps to are grouped by id % 8 (the XCD).
  const int HB = a.Hq * a.B;
  const int bid = blockIdx.x;
  const int trank = bid / HB;
  int j = bid - trank * HB;
  if ((HB & 7) == 0) j = (j & 7) * (HB >> 3) + (j >> 3);
  const int hq = j % a.Hq;
  const int b = j / a.Hq;
  const int qt = a.num_q_tiles - 1 - trank;
  const int hk = hq / a.group;

  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const elem_t *qbase = (const elem_t *)a.q + b * a.q_sb + hq * a.q_sh;
  const elem_t *kbase = (const elem_t *)a.k + b * a.k_sb + hk * a.k_sh;
  const elem_t *vbase = (const elem_t *)a.v + b * a.v_sb + hk * a.v_sh;

  // This lane's query row and the wave's row range (global positions).
  const int qrow = q0 + 32 * wave + r32;
  const int64_t qpos = a.q_offset + qrow;
  const int64_t wpos_first = a.q_offset + q0 + 32 * wave_u;
  const int64_t wpos_last = wpos_first + 31;
  const bool wave_active = (q0 + 32 * wave_u) < a.Sq;
  const float c = a.scale_log2;

  typename Path::QFrag qf;
  Path::load_q(qf, a, qbase, qrow, h);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max in the scaled log2 domain (c * s)
  float l_run = 0.f;        // this lane's share of the exp-sum (halves summed at the end)

  auto tile_buf = [&](int i) { return (elem_t *)(smem + i * Path::BUF_BYTES); };
  // A wave skips a tile when every key of it is in the future of all its rows.
  auto skips = [&](int kbx) {
    return !wave_active || (CAUSAL && a.kv_offset + kbx > wpos_last);
  };
  // Mask a tile's scores (only tiles that straddle the diagonal or a chunk end), return
  // the row max in the scaled log2 domain and apply the lazy rescale to O and l.
  auto mask_max_rescale = [&](f32x16 (&s)[2], int kbx, int cendx) {
    const int64_t kpos0 = a.kv_offset + kbx;
    const int kvalid = min(BN, cendx - kbx);
    const bool need_mask = (kvalid < BN) || (CAUSAL && kpos0 + kvalid - 1 > wpos_first);
    if (need_mask) {
      int lim = kvalid;  // keys kk < lim are visible to this lane's row
      if (CAUSAL) {
        const int64_t vis = qpos - kpos0 + 1;  // may be <= 0 or > BN
        lim = vis < (int64_t)lim ? (vis > 0 ? (int)vis : 0) : lim;
      }
      lim -= 4 * h;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 32 * mt + (i >> 2) * 8 + (i & 3);  // minus the 4h offset
          s[mt][i] = kk < lim ? s[mt][i] : -INFINITY;
        }
    }
    float mx = fmaxf(max_finite(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[0][i]), s[0][i + 1]);
    mx = fmaxf(mx, s[0][15]);
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[1][i]), s[1][i + 1]);
    mx = halves_max(mx) * c;
    // lazy rescale: only when some row's max grew by more than kLazyRescale
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
  };

  const int64_t vis_lim = a.q_offset + qlast - a.kv_offset + 1;
  int t = -1, kb = 0, kend = 0, cend = 0;
  ring_next(a, CAUSAL, vis_lim, t, kb, kend, cend);
  typename Path::Stage st;

  // ---- double-buffered loop: load next tile | QK, softmax, PV of this tile | store.
  if (t < a.num_chunks) {
    Path::load_tile(st, a, kbase, vbase, kb, tid);
    Path::store_tile(st, tile_buf(0), tid);
  }
  // All prologue loads (Q included) have landed: without this the compiler keeps Q's
  // loads "pending" on the no-tile path and the loop's first MFMAs would wait on the
  // freshly issued prefetch as well (vmcnt counts in order).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  int cur = 0;
  while (t < a.num_chunks) {
    const int kb_cur = kb, cend_cur = cend;
    ring_next(a, CAUSAL, vis_lim, t, kb, kend, cend);
    const bool has_next = t < a.num_chunks;
    if (has_next) Path::load_tile(st, a, kbase, vbase, kb, tid);
    const elem_t *buf = tile_buf(cur);
    if (!skips(kb_cur)) {
      f32x16 s[2];
      Path::qk(s, qf, buf, lane);
      typename Path::VPre vp;
      Path::pv_prefetch(vp, buf, lane);
      mask_max_rescale(s, kb_cur, cend_cur);
      const float mneg = m_run == -INFINITY ? 0.f : -m_run;
      typename Path::PFrag pf;
      l_run += Path::exp_pack(s, c, mneg, pf);
      Path::pv(o, pf, vp, buf, lane);
    }
    if (has_next) Path::store_tile(st, tile_buf(cur ^ 1), tid);
    __syncthreads();
    cur ^= 1;
  }

  // Epilogue: o = O / l, lse = ln(sum) = (m + log2 l) * ln 2.
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < a.Sq) {
    if (h == 0) {
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      a.lse[b * a.l_sb + hq * a.l_sh + qrow] = lse;
    }
    const int64_t orow = b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        const float x0 = o[dt][4 * g + 0] * inv, x1 = o[dt][4 * g + 1] * inv;
        const float x2 = o[dt][4 * g + 2] * inv, x3 = o[dt][4 * g + 3] * inv;
        if (a.o_is_f32) {
          *(float4 *)((float *)a.o + orow + d) = float4{x0, x1, x2, x3};
        } else {
          const bf16x2 lo = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2){x2, x3}, bf16x2);
          *(u32x2 *)((uint16_t *)a.o + orow + d) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      }
  }
}

// ---------------------------------------------------------------------------------
// Kernel for the bf16 direct path: double-buffered LDS, the next tile's direct loads in
// flight under the current tile's math.
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL, int NW, int KN, bool VARLEN>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_direct_kernel(FwdArgs a) {
  using Path = Bf16DirectPath<D, NW, KN>;
  constexpr int NMT = KN / 32;
  using elem_t = uint16_t;
  constexpr int BM = 32 * Path::kWaves;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * Path::BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy
  const int r32 = lane & 31;
  const int h = lane >> 5;

  const int HB = a.Hq * a.B;
  // Query tile of this workgroup, heaviest (most keys) first.  Workgroups are placed on
  // the 8 XCDs round-robin by id, and XCDs run at different speeds (up to 17 % apart in
  // per-workgroup timestamps), so a fixed id -> tile map leaves the fast XCDs idle at the
  // end.  With a work counter each workgroup takes the next tile when it starts instead:
  // tickets are residues mod the grid (a permutation whatever the counter held), and the
  // holder of the last residue subtracts the grid again, so the counter ends as it began.
  __shared__ int s_job;
  int bid = blockIdx.x;
  if (a.sched != nullptr) {
    if (threadIdx.x == 0) {
      const unsigned long long g = gridDim.x;
      const unsigned long long tk = atomicAdd((unsigned long long *)a.sched, 1ull);
      const int job = (int)(tk % g);
      if (job == (int)g - 1) atomicAdd((unsigned long long *)a.sched, 0ull - g);
      s_job = job;
    }
    __syncthreads();
    bid = __builtin_amdgcn_readfirstlane(s_job);
  }
  const int trank = bid / HB;
  int j = bid - trank * HB;
  // Fixed order when B*Hq is a multiple of 8: XCD (id mod 8) sees a fixed subset of the
  // heads, whose K/V then stay in its L2.
  if ((HB & 7) == 0) j = (j & 7) * (HB >> 3) + (j >> 3);
  const int hq = j % a.Hq;
  const int b = j / a.Hq;
  const int qt = a.num_q_tiles - 1 - trank;
  const int hk = hq / a.group;

  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const elem_t *qbase = (const elem_t *)a.q + b * a.q_sb + hq * a.q_sh;
  const elem_t *kbase = (const elem_t *)a.k + b * a.k_sb + hk * a.k_sh;
  const elem_t *vbase = (const elem_t *)a.v + b * a.v_sb + hk * a.v_sh;

  const int qrow = q0 + 32 * wave + r32;
  const int64_t qpos = a.q_offset + qrow;
  const int64_t wpos_first = a.q_offset + q0 + 32 * wave_u;
  const int64_t wpos_last = wpos_first + 31;
  const bool wave_active = (q0 + 32 * wave_u) < a.Sq;
  const float c = a.scale_log2;

  typename Path::Lane L;
  Path::setup(L, a, tid, lds_offset(smem));
  // Tile loads: by waves NW/2 .. NW-1 only (one per SIMD: waves are placed on the SIMDs
  // round-robin).  Issuing a tile's direct loads holds a wave for about as long as one
  // MFMA phase, so the loading wave of each SIMD starts its QK^T MFMAs that much later
  // than the other: the two waves then alternate MFMA and softmax phases instead of
  // running them together (4.5 % on the 32K causal GQA workload).  Odd waves as loaders
  // (both on the same two SIMDs) measured no gain.
  using LoadPath = Bf16DirectPath<D, NW / 2, KN>;
  const int lw = wave_u - NW / 2;
  typename LoadPath::Lane LL;
  if (lw >= 0) LoadPath::setup(LL, a, 64 * lw + lane, lds_offset(smem));
  auto load_tile = [&](int kbx, uint32_t slot) {
    if (lw >= 0) LoadPath::load_tile(LL, a, kbase, vbase, kbx, slot, lw);
  };
  typename Path::QFrag qf;
  Path::load_q(qf, a, qbase, qrow, h);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  // exp2 offset -m_run (0 while m_run is -inf) and the rescale test's
  // -(m_run + kLazyRescale), both changed only when m_run is
  float mneg = 0.f, nthr = INFINITY;

  const int64_t vis_lim = a.q_offset + qlast - a.kv_offset + 1;
  int t = -1, kb = 0, kend = 0, cend = 0;
  ring_next<KN>(a, CAUSAL, vis_lim, t, kb, kend, cend);
  // Packed documents: this lane's row sees keys [ds, de) (causal: [ds, row]); the wave's
  // first and last rows bound the wave's keys; the block walks from the tile holding its
  // first row's document start.
  int ds = 0, de = 0, w_ds_first = 0, w_ds_last = 0, w_de_first = 0, w_de_last = 0;
  if (VARLEN) {
    doc_bounds(a.cu, a.n_docs, min(qrow, a.Sq - 1), a.Skv, ds, de);
    w_ds_first = __builtin_amdgcn_readlane(ds, 0);
    w_ds_last = __builtin_amdgcn_readlane(ds, 31);
    w_de_first = __builtin_amdgcn_readlane(de, 0);
    w_de_last = __builtin_amdgcn_readlane(de, 31);
    int b_ds, b_de, l_ds, l_de;
    doc_bounds(a.cu, a.n_docs, q0, a.Skv, b_ds, b_de);
    doc_bounds(a.cu, a.n_docs, qlast, a.Skv, l_ds, l_de);
    b_ds = __builtin_amdgcn_readfirstlane(min(b_ds, qlast));
    kb = (b_ds / KN) * KN;
    if (!CAUSAL) kend = __builtin_amdgcn_readfirstlane(max(l_de, l_ds));
    if (kb >= kend) t = a.num_chunks;
  }
  const uint32_t smem0 = lds_offset(smem);
  if (t < a.num_chunks) load_tile(kb, smem0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first tile have landed
  __syncthreads();

  // One tile from LDS slot `cur` (the next tile's loads go to the other slot); the loop
  // alternates the slots so that the operand addresses are per-slot registers with
  // immediate block offsets.  Returns false when the walk is done.
  auto tile = [&](auto cur_c) -> bool {
    constexpr int cur = decltype(cur_c)::value;
    const int kb_cur = kb, cend_cur = cend;
    ring_next<KN>(a, CAUSAL, vis_lim, t, kb, kend, cend);
    const bool has_next = t < a.num_chunks;
    if (has_next) load_tile(kb, smem0 + (cur ^ 1) * Path::BUF_BYTES);

    const int64_t kpos0 = a.kv_offset + kb_cur;
    const bool doc_skip =
        VARLEN && (kb_cur + KN <= w_ds_first || (!CAUSAL && kb_cur >= w_de_last));
    if (wave_active && !(CAUSAL && kpos0 > wpos_last) && !doc_skip) {
      f32x16 s[NMT];
      Path::qk(s, qf, L, cur);
      const int kvalid = min(KN, cend_cur - kb_cur);
      const bool need_mask =
          (kvalid < KN) || (CAUSAL && kpos0 + kvalid - 1 > wpos_first) ||
          (VARLEN && (kb_cur < w_ds_last || (!CAUSAL && kb_cur + kvalid > w_de_first)));
      if (need_mask) {
        int lim = kvalid;  // keys lo <= kk < lim are visible to this lane's row
        if (CAUSAL) {
          const int64_t vis = qpos - kpos0 + 1;
          lim = vis < (int64_t)lim ? (vis > 0 ? (int)vis : 0) : lim;
        }
        int lo = 0;
        if (VARLEN) {
          if (!CAUSAL) lim = min(lim, de - kb_cur);
          lo = ds - kb_cur;
        }
        lim -= 4 * h;
        lo -= 4 * h;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * mt + (i >> 2) * 8 + (i & 3);
            s[mt][i] = (kk < lim && (!VARLEN || kk >= lo)) ? s[mt][i] : -INFINITY;
          }
      }
      float mx = fmaxf(max_finite(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[0][i]), s[0][i + 1]);
      mx = fmaxf(mx, s[0][15]);
#pragma unroll
      for (int mt = 1; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[mt][i]), s[mt][i + 1]);
      mx = halves_max(mx);
      // c mx > m_run + kLazyRescale, as one FMA against the loop-carried
      // -(m_run + kLazyRescale)
      if (__builtin_amdgcn_ballot_w64(fmaf(mx, c, nthr) > 0.f) != 0) {
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
        mneg = m_new == -INFINITY ? 0.f : -m_new;
        nthr = -(m_new + kLazyRescale);
      }
      typename Path::PFrag pf;
      l_run += Path::exp_pack(s, c, mneg, pf);
      Path::pv(o, pf, L, cur);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile's direct loads landed
    __syncthreads();
    return has_next;
  };
  if (t < a.num_chunks) {
    while (tile(std::integral_constant<int, 0>{}) && tile(std::integral_constant<int, 1>{})) {
    }
  }

  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < a.Sq) {
    if (h == 0) {
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
      a.lse[b * a.l_sb + hq * a.l_sh + qrow] = lse;
    }
    const int64_t orow = b * a.o_sb + hq * a.o_sh + (int64_t)qrow * a.o_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        const float x0 = o[dt][4 * g + 0] * inv, x1 = o[dt][4 * g + 1] * inv;
        const float x2 = o[dt][4 * g + 2] * inv, x3 = o[dt][4 * g + 3] * inv;
        if (a.o_is_f32) {
          *(float4 *)((float *)a.o + orow + d) = float4{x0, x1, x2, x3};
        } else {
          const bf16x2 lo = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2){x2, x3}, bf16x2);
          *(u32x2 *)((uint16_t *)a.o + orow + d) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      }
  }
}

template <int D, bool CAUSAL, bool VARLEN = false>
int launch_direct(const FwdArgs &args, hipStream_t stream) {
  FwdArgs a = args;
  constexpr int NW = kDirectWaves;
  a.num_q_tiles = (a.Sq + 32 * NW - 1) / (32 * NW);
  const int64_t blocks = (int64_t)a.num_q_tiles * a.Hq * a.B;
  if (blocks <= 0) return RA_OK;
  // the work counter serves the shapes the fixed XCD head map cannot (B*Hq % 8 != 0):
  // with it the 32-head layers measured 1.8 % slower (their K/V leave the XCD's L2)
  if ((a.Hq * a.B) % 8 == 0) a.sched = nullptr;
  constexpr int KN = kDirectKN;
  hipLaunchKernelGGL((attn_fwd_direct_kernel<D, CAUSAL, NW, KN, VARLEN>), dim3((unsigned)blocks),
                     dim3(64 * NW), 0, stream, a);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

template <class Path, int D, bool CAUSAL>
int launch_one(const FwdArgs &args, hipStream_t stream) {
  FwdArgs a = args;
  a.num_q_tiles = (a.Sq + 32 * Path::kWaves - 1) / (32 * Path::kWaves);
  const int64_t blocks = (int64_t)a.num_q_tiles * a.Hq * a.B;
  if (blocks <= 0) return RA_OK;
  hipLaunchKernelGGL((attn_fwd_kernel<Path, D, CAUSAL>), dim3((unsigned)blocks),
                     dim3(Path::kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace

int launch_attn_fwd(const FwdArgs &a, int dtype, int D, int causal, hipStream_t stream) {
  if (dtype == RA_BF16) {
    if (D == 128) return causal ? launch_direct<128, true>(a, stream) : launch_direct<128, false>(a, stream);
    if (D == 64) return causal ? launch_direct<64, true>(a, stream) : launch_direct<64, false>(a, stream);
  } else if (dtype == RA_F32) {
    if (D == 128) return causal ? launch_one<F32Path<128>, 128, true>(a, stream)
                                : launch_one<F32Path<128>, 128, false>(a, stream);
    if (D == 64) return causal ? launch_one<F32Path<64>, 64, true>(a, stream)
                               : launch_one<F32Path<64>, 64, false>(a, stream);
  }
  return RA_ERR_UNSUPPORTED;
}

int launch_attn_fwd_varlen(const FwdArgs &a, int D, int causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_direct<128, true, true>(a, stream) : launch_direct<128, false, true>(a, stream);
  if (D == 64)
    return causal ? launch_direct<64, true, true>(a, stream) : launch_direct<64, false, true>(a, stream);
  return RA_ERR_UNSUPPORTED;
}

}  // namespace ra
