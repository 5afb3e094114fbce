// attn_bwd -- gradients of exact softmax attention, recomputing the attention weights
// from the forward's saved log-sum-exp instead of storing them.
//
// Sources (page title, host):
//   [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn), section
//        "为什么传统注意力这么“吃”显存？": the backward pass needs the attention
//        intermediates, kept or recomputed; here they are recomputed tile by tile.
//   [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn), section
//        "Ring-Attention：面向大规模部署的工程利器": gradients travel back along the ring.
// The gradient formulas are the textbook ones (not on the pages), for L = sum(dO * O):
//   P = exp(scale q.k - lse),  D_i = rowsum(dO * O),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, no atomics (bitwise deterministic):
//   * bwd_delta  -- D_i = sum_d dO_id O_id (fp32), a streaming pass;
//   * bwd_dq     -- one workgroup per 256 query rows (8 waves x 32); K/V tiles of 64 keys
//                   stream through LDS in ring order; per tile: S^T = K Q^T and
//                   dP^T = V dO^T (Q, dO in registers), P and dS in registers, then
//                   dQ^T += K^T dS^T with K^T read transposed from the same LDS tile;
//   * bwd_dkdv   -- one workgroup per 128 keys (4 waves x 32) of one key/value head
//                   (with grouped heads: of one query head, into fp32 partials that
//                   bwd_kv_reduce then sums over the group in a fixed order);
//                   loops over 64-row query tiles of every query head it covers,
//                   Q and dO tiles in LDS: S = Q K^T, dP = dO V^T (K^T, V^T in registers),
//                   dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read transposed.
// Tiles move global -> LDS with direct loads and a swizzle that keeps both row-wise
// (ds_read_b128) and transposed (ds_read_b64_tr_b16) operand reads conflict-free.
// The accumulating form (ACC) is one device's step of the ring backward: the key/value
// block is one chunk, and the epilogues add the step's dQ, dK, dV into fp32
// accumulators (dQ stays with the device, dK/dV travel with the chunk) instead of
// storing bf16 results.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int TN = 64;  // rows per LDS tile of queries in bwd_dkdv
static_assert(TN <= kMaxTileRows, "tile offsets are 32-bit");
#ifndef RA_BWD_DQ_UNROLL
#define RA_BWD_DQ_UNROLL 2  // 32-key halves of a dQ tile unrolled together
#endif
#ifndef RA_BWD_DQ_NW
#define RA_BWD_DQ_NW 8  // waves (32 query rows each) per dQ workgroup
#endif
#ifndef RA_BWD_DQ_LOADERS
#define RA_BWD_DQ_LOADERS (RA_BWD_DQ_NW / 2)  // dQ: waves (the last ones) that load K/V tiles
#endif
#ifndef RA_BWD_DKDV_NW
#define RA_BWD_DKDV_NW 4  // dK/dV: waves (32 keys each) per workgroup, one per SIMD
#endif
#ifndef RA_BWD_DKDV_LOADERS
#define RA_BWD_DKDV_LOADERS 2  // dK/dV: waves that issue the Q/dO tile loads (the last ones)
#endif
#ifndef RA_BWD_DQ_KT
#define RA_BWD_DQ_KT 64  // keys per LDS tile in bwd_dq (128 measured equal)
#endif

// Register placement in the dK/dV kernel (one wave per SIMD, ~370 live registers).  The
// compiler's choice -- every MFMA accumulator in VGPRs, other values spilled to AGPRs --
// cost ≈220 AGPR->VGPR copies per 64 MFMAs.  Here the MFMAs are written out so that
// the dK, dV accumulators and the resident K^T, V^T operands live in AGPRs (MFMAs read
// and write them there; no VALU touches them inside the loop) and the score products
// S, dP (read by the softmax VALU work) in VGPRs: no copies at all.  The compiler does
// not see these MFMAs, so every consumer is placed where no wait states are needed: a
// score chain's results are first read two MFMAs (≥64 clk) after its last step, the
// P/dS operands are written at least eight MFMAs before their use, chained
// accumulators overlap exactly, and the epilogue waits explicitly.  With D = 64 (about
// 330 registers, well inside one wave's 512) the written-out forms only made the
// register allocator copy the accumulators out of AGPRs inside the loop, so there W is
// false and the compiler's own MFMAs (and hazard handling) are used.
// dK or dV += A B (accumulator in AGPRs, A and B in VGPRs)
template <bool W>
__device__ __forceinline__ void mfma_grad(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
  if constexpr (W)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    acc = mfma_bf16(a, b, acc);
}
// S or dP: first step of a chain (C = 0) and further steps; the B operand (the key/value
// rows kept for the whole workgroup) is read straight from AGPRs, the result is a VGPR.
template <bool W>
__device__ __forceinline__ f32x16 mfma_score0_ab(const bf16x8 &a, const bf16x8 &b) {
  if constexpr (!W) return mfma_bf16(a, b, f32x16{});
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
template <bool W>
__device__ __forceinline__ f32x16 mfma_score_c_ab(const bf16x8 &a, const bf16x8 &b,
                                                   const f32x16 &c) {
  if constexpr (!W) return mfma_bf16(a, b, c);
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
  return d;
}
template <bool W>
__device__ __forceinline__ void mfma_score_ab(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
  if constexpr (W)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
  else
    acc = mfma_bf16(a, b, acc);
}

// 16-byte-chunk swizzle of a tile row: for 16 consecutive rows at one chunk the physical
// chunks differ (row-wise reads), and for 4 consecutive rows at 4 consecutive chunks
// they fall in different 64-byte segments (transposed reads).
template <int D>
__device__ __forceinline__ int usw(int r) {
  if (D == 128) return (r & 15) ^ ((r & 3) << 2);
  return ((r >> 1) & 7) ^ (((r >> 1) & 1) << 2);
}

// A TN x D bf16 tile in LDS (dense, swizzled), loaded with direct loads.
template <int D, int NW, int ROWS = TN>
struct STile {
  static constexpr int RB = 2 * D;
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NBLK = BYTES / 1024;
  static constexpr int BPW = NBLK / NW;  // 1-KiB blocks per wave
  static_assert(NBLK % NW == 0, "tile must split evenly over the waves");
  // A lane's rows in successive blocks are STEP apart; the swizzle repeats every 16
  // rows, so its chunk repeats every CP blocks (only CP chunks are kept per lane).
  static constexpr int STEP = NW * 1024 / RB;
  static constexpr int CP = STEP % 16 == 0 ? 1 : 16 / (STEP % 16);
  static_assert(STEP % 16 == 0 || 16 % (STEP % 16) == 0, "swizzle period");

  struct Lane {
    int row, chunk[CP < BPW ? CP : BPW];
  };
  __device__ static void setup(Lane &L, int lane, int wave) {
    L.row = (wave * 1024 + 16 * lane) / RB;
#pragma unroll
    for (int i = 0; i < (CP < BPW ? CP : BPW); ++i) {
      const int byte = (wave + NW * i) * 1024 + 16 * lane;
      L.chunk[i] = ((byte % RB) / 16) ^ usw<D>(byte / RB);
    }
  }
  // rows row0 .. row0+TN-1 of a [rows, D] matrix with row stride `ss` elements; rows
  // at or past `nrows` read row nrows-1 instead (callers mask them).
  __device__ static void load(const Lane &L, const uint16_t *base, int64_t ss, int row0,
                              int nrows, uint32_t lds, int wave) {
    const uint16_t *tb = base + (int64_t)row0 * ss;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int r = min(row0 + L.row + STEP * i, nrows - 1) - row0;
      const int off = (int)(r * ss * 2) + 16 * L.chunk[i % CP];
      const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane(wave + NW * i);
      dma_b128(tb, off, lds + blk * 1024);
    }
  }
  // Row-wise MFMA operand: 8 consecutive bf16 (chunk 2*ks + h) of row r.  Returns the
  // lane part; the read address is (part ^ 32*ks) + tile base (+ 32*RB per 32-row step).
  __device__ static uint32_t row_part(int r, int h) {
    return (uint32_t)(r * RB + 16 * (usw<D>(r) ^ h));
  }
  __device__ static u32x4 row_read(uint32_t base, uint32_t part, int ks) {
    return lds_read_b128(base + (part ^ (uint32_t)(32 * ks)));
  }
  // Transposed MFMA operand (M = head dim, K = tile rows): for rows r0 + 4h + (0..3)
  // and r0 + 8 + 4h + (0..3) and head dims 32*dt + (lane & 31).  lane_part(s) is the
  // per-lane address of sub-read s; the dt selection is an XOR by 64*dt.
  __device__ static uint32_t tr_part(int lane, int s) {
    const int h = lane >> 5, g = lane >> 4, ap = lane & 15, z = ap >> 2;
    const int w = 2 * (g & 1) + ((ap & 3) >> 1);
    const int r = 8 * s + 4 * h + z;  // row within a 16-row step
    const int f = usw<D>(r);
    // physical chunk = (4*dt + w) ^ f ; keep the dt part out (XORed per read)
    const int chunk_nodt = w ^ f;
    return (uint32_t)(r * RB + 16 * chunk_nodt + 8 * (ap & 1));
  }
  __device__ static u32x4 tr_read(uint32_t base, uint32_t part0, uint32_t part1, int r0, int dt) {
    const uint32_t x = (uint32_t)(64 * dt);
    const s16x4 lo = lds_read_tr16_b64(base + (uint32_t)(r0 * RB) + (part0 ^ x));
    const s16x4 hi = lds_read_tr16_b64(base + (uint32_t)(r0 * RB) + (part1 ^ x));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
};

// ---------------------------------------------------------------------------------
// D_i = sum_d dO_id * O_id  (one 64-lane wave per row group; D <= 128)
// ---------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row (8 bf16 each)
  const int64_t nrows = (int64_t)a.B * a.Hq * a.Sq;
  const int sub = threadIdx.x % LPR;
  for (int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR; row < nrows;
       row += (int64_t)gridDim.x * (256 / LPR)) {
    const int s = (int)(row % a.Sq);
    const int64_t bh = row / a.Sq;
    const int hh = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const u32x4 x = *(const u32x4 *)((const uint16_t *)a.o + b * a.o_sb + hh * a.o_sh +
                                       (int64_t)s * a.o_ss + 8 * sub);
    const u32x4 y = *(const u32x4 *)((const uint16_t *)a.dout + b * a.do_sb + hh * a.do_sh +
                                       (int64_t)s * a.do_ss + 8 * sub);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_bits_to_float(x[w] & 0xffffu), bf16_bits_to_float(y[w] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_float(x[w] >> 16), bf16_bits_to_float(y[w] >> 16), acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (sub == 0) a.delta[row] = acc;
  }
}

// Next key tile in ring order (as in the forward).  t == P means done.
template <int STEP>
__device__ __forceinline__ void ring_next_bwd(const BwdArgs &a, bool causal, int64_t vis_lim,
                                              int &t, int &kb, int &kend, int &cend) {
  kb += STEP;
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
// dQ: 8 waves x 32 query rows.  Per key tile (KT keys, 32-key blocks mt):
//   S^T_mt = K_mt Q^T, dP^T_mt = V_mt dO^T         (16 + 16 MFMAs over the tile)
//   P^T = exp2(c S^T - log2e lse), dS^T = P^T (dP^T - D)  -> bf16
//   dQ^T += K^T_mt dS^T_mt                          (16 MFMAs over the tile)
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN, bool ACC>
__global__ void __launch_bounds__(64 * RA_BWD_DQ_NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdArgs a, int num_q_tiles) {
  constexpr int NW = RA_BWD_DQ_NW, BM = 32 * NW;
  constexpr int KT = RA_BWD_DQ_KT;  // keys per LDS tile
  static_assert(KT <= kMaxTileRows, "tile offsets are 32-bit");
  using Tile = STile<D, NW, KT>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * Tile::BYTES];
  const uint32_t smem0 = lds_offset(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  const int HB = a.Hq * a.B;
  const int bid = blockIdx.x;
  const int trank = bid / HB;
  int j = bid - trank * HB;
  if ((HB & 7) == 0) j = (j & 7) * (HB >> 3) + (j >> 3);
  const int hq = j % a.Hq, b = j / a.Hq, hk = hq / a.group;
  const int qt = num_q_tiles - 1 - trank;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const int qrow = q0 + 32 * wave + r32;
  const int qr = min(qrow, a.Sq - 1);
  const int64_t qpos = a.q_offset + qrow;
  const int64_t wpos_first = a.q_offset + q0 + 32 * wave;
  const int64_t wpos_last = wpos_first + 31;
  const bool wave_active = (q0 + 32 * wave) < a.Sq;
  const float c = a.scale_log2;

  const uint16_t *qb = (const uint16_t *)a.q + b * a.q_sb + hq * a.q_sh;
  const uint16_t *dob = (const uint16_t *)a.dout + b * a.do_sb + hq * a.do_sh;
  const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_sb + hk * a.k_sh;
  const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_sb + hk * a.v_sh;

  // Q and dO as B operands (k = head dim 16*ks + 8h .. +8), one row per lane.
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = as_bf16x8(*(const u32x4 *)(qb + (int64_t)qr * a.q_ss + 16 * ks + 8 * h));
    df[ks] = as_bf16x8(*(const u32x4 *)(dob + (int64_t)qr * a.do_ss + 16 * ks + 8 * h));
  }
  const float lse = a.lse[b * a.l_sb + hq * a.l_sh + qr];
  // exp2 argument offset; an empty row (lse = -inf) gets +inf so every P is 0
  const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
  const float dlt = a.delta[((int64_t)b * a.Hq + hq) * a.Sq + qr];

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = f32x16{};

  // K/V tile loads by half of the waves (one per SIMD), which thereby start each tile's
  // MFMAs later than the other half: the two waves of a SIMD alternate MFMA and
  // softmax phases instead of running them together
  constexpr int NL = RA_BWD_DQ_LOADERS;
  using LTile = STile<D, NL, KT>;
  const int lw = __builtin_amdgcn_readfirstlane(wave) - (NW - NL);
  typename LTile::Lane TL;
  if (lw >= 0) LTile::setup(TL, lane, lw);
  auto load_kv = [&](int kbx, uint32_t lds) {
    if (lw >= 0) {
      LTile::load(TL, kbase, a.k_ss, kbx, a.Skv, lds, lw);
      LTile::load(TL, vbase, a.v_ss, kbx, a.Skv, lds + Tile::BYTES, lw);
    }
  };
  const uint32_t kpart = Tile::row_part(r32, h);  // rows r32 (+32 per mt)
  const uint32_t tp0 = Tile::tr_part(lane, 0), tp1 = Tile::tr_part(lane, 1);

  const int64_t vis_lim = a.q_offset + qlast - a.kv_offset + 1;
  int t = -1, kb = 0, kend = 0, cend = 0;
  ring_next_bwd<KT>(a, CAUSAL, vis_lim, t, kb, kend, cend);
  // Packed documents: this lane's row sees keys [ds, de) (causal: [ds, row]); the block
  // walks from the tile holding its first row's document start.
  int ds = 0, de = 0, w_ds_first = 0, w_ds_last = 0, w_de_first = 0, w_de_last = 0;
  if (VARLEN) {
    doc_bounds(a.cu, a.n_docs, qr, a.Skv, ds, de);
    w_ds_first = __builtin_amdgcn_readlane(ds, 0);
    w_ds_last = __builtin_amdgcn_readlane(ds, 31);
    w_de_first = __builtin_amdgcn_readlane(de, 0);
    w_de_last = __builtin_amdgcn_readlane(de, 31);
    int b_ds, b_de, l_ds, l_de;
    doc_bounds(a.cu, a.n_docs, q0, a.Skv, b_ds, b_de);
    doc_bounds(a.cu, a.n_docs, qlast, a.Skv, l_ds, l_de);
    b_ds = __builtin_amdgcn_readfirstlane(min(b_ds, qlast));
    kb = (b_ds / KT) * KT;
    if (!CAUSAL) kend = __builtin_amdgcn_readfirstlane(max(l_de, l_ds));
    if (kb >= kend) t = a.num_chunks;
  }
  if (t < a.num_chunks) load_kv(kb, smem0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // One key tile from LDS slot CUR (the next tile's loads go to the other slot); the
  // loop alternates the slots, so that slot, block and K-versus-V offsets are immediates
  // of the LDS reads and each lane forms its XOR-swizzled read addresses once per tile.
  auto tile = [&](auto cur_c) -> bool {
    constexpr uint32_t CUR = decltype(cur_c)::value;
    constexpr uint32_t SLOT = CUR * 2 * Tile::BYTES;
    const int kb_cur = kb, cend_cur = cend;
    ring_next_bwd<KT>(a, CAUSAL, vis_lim, t, kb, kend, cend);
    const bool has_next = t < a.num_chunks;
    if (has_next) load_kv(kb, smem0 + (CUR ^ 1) * 2 * Tile::BYTES);
    const int64_t kpos0 = a.kv_offset + kb_cur;
    const bool doc_skip =
        VARLEN && (kb_cur + KT <= w_ds_first || (!CAUSAL && kb_cur >= w_de_last));
    if (wave_active && !(CAUSAL && kpos0 > wpos_last) && !doc_skip) {
      // row reads: smem0 + (kpart ^ 32 ks); transposed reads: smem0 + (tp ^ 64 dt).  The
      // empty asm keeps them per tile (hoisted out of the loop they would hold 16
      // registers for its whole length).
      uint32_t kp = kpart, t0 = tp0, t1 = tp1;
      asm volatile("" : "+v"(kp), "+v"(t0), "+v"(t1));
      uint32_t ra[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) ra[ks] = smem0 + (kp ^ (uint32_t)(32 * ks));
      const int kvalid = min(KT, cend_cur - kb_cur);
      const bool need_mask =
          (kvalid < KT) || (CAUSAL && kpos0 + kvalid - 1 > wpos_first) ||
          (VARLEN && (kb_cur < w_ds_last || (!CAUSAL && kb_cur + kvalid > w_de_first)));
      int lim = kvalid;
      const int lo = VARLEN ? ds - kb_cur : 0;  // keys lo <= kk < lim are visible
      if (VARLEN && !CAUSAL) lim = min(lim, de - kb_cur);
      if (CAUSAL) {
        const int64_t vis = qpos - kpos0 + 1;
        lim = vis < (int64_t)lim ? (vis > 0 ? (int)vis : 0) : lim;
      }
#pragma unroll RA_BWD_DQ_UNROLL
      for (int mt = 0; mt < KT / 32; ++mt) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const uint32_t ko = SLOT + (uint32_t)(mt * 32 * Tile::RB);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          s = mfma_bf16(as_bf16x8(lds_read_b128(ra[ks] + ko)), qf[ks], s);
          dp = mfma_bf16(as_bf16x8(lds_read_b128(ra[ks] + ko + Tile::BYTES)), df[ks], dp);
        }
        // P^T and dS^T (lane: one query row, 16 of the 32 keys of this half); the element
        // mask only where this 32-key half needs it (a wave-uniform branch)
        float pv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[i] = fast_exp2(fmaf(s[i], c, -lse2));
        const bool nm = (kvalid < 32 * (mt + 1)) ||
                        (CAUSAL && kpos0 + 32 * mt + 31 > wpos_first) ||
                        (VARLEN && need_mask);
        if (__builtin_amdgcn_readfirstlane((int)nm)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * mt + (i >> 2) * 8 + 4 * h + (i & 3);
            if (kk >= lim || (VARLEN && kk < lo)) pv[i] = 0.f;
          }
        }
        u32x4 dsf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int i = 8 * s2 + 2 * w;
            const bf16x2 pk = __builtin_convertvector(
                (f32x2){pv[i] * (dp[i] - dlt), pv[i + 1] * (dp[i + 1] - dlt)}, bf16x2);
            dsf[s2][w] = __builtin_bit_cast(uint32_t, pk);
          }
        // dQ^T[D x 32 q] += K^T[D x 32 keys] dS^T[32 keys x 32 q]
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const uint32_t off = SLOT + (uint32_t)((32 * mt + 16 * s2) * Tile::RB);
            const uint32_t x = (uint32_t)(64 * dt);
            const s16x4 lo = lds_read_tr16_b64(smem0 + (t0 ^ x) + off);
            const s16x4 hi = lds_read_tr16_b64(smem0 + (t1 ^ x) + off);
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 kf = u32x4{l2[0], l2[1], h2[0], h2[1]};
            dq[dt] = mfma_bf16(as_bf16x8(kf), as_bf16x8(dsf[s2]), dq[dt]);
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed
    __syncthreads();
    return has_next;
  };
  if (t < a.num_chunks) {
    while (tile(std::integral_constant<uint32_t, 0>{}) &&
           tile(std::integral_constant<uint32_t, 1>{})) {
    }
  }

  if (qrow < a.Sq) {
    const int64_t orow = b * a.dq_sb + hq * a.dq_sh + (int64_t)qrow * a.dq_ss;
    // the lane half again, from the lane counter: keeping h alive across the key loop
    // cost a register spill
    const int he = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * he;
        if (ACC) {
          f32x4 *acc = (f32x4 *)((float *)a.dq + orow + d);
          const f32x4 prev = *acc;
          *acc = f32x4{prev[0] + dq[dt][4 * g] * a.scale, prev[1] + dq[dt][4 * g + 1] * a.scale,
                       prev[2] + dq[dt][4 * g + 2] * a.scale, prev[3] + dq[dt][4 * g + 3] * a.scale};
          continue;
        }
        const bf16x2 lo = __builtin_convertvector(
            (f32x2){dq[dt][4 * g] * a.scale, dq[dt][4 * g + 1] * a.scale}, bf16x2);
        const bf16x2 hi = __builtin_convertvector(
            (f32x2){dq[dt][4 * g + 2] * a.scale, dq[dt][4 * g + 3] * a.scale}, bf16x2);
        *(u32x2 *)((uint16_t *)a.dq + orow + d) =
            u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV: 4 waves x 32 keys.  Per query tile (64 rows, two 32-row steps qs), for each
// query head of the group:
//   S = Q K^T, dP = dO V^T                 (A: Q / dO rows from LDS, B: K^T / V^T regs)
//   P = exp2(c S - log2e lse), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS          (A: transposed reads of dO / Q)
// 128-dim heads run one wave per SIMD (their dK^T, dV^T accumulators fill the AGPRs);
// 64-dim heads fit two per SIMD, whose MFMA and softmax phases then overlap (16K
// causal, 32 heads: 4.66 -> 3.90 ms; 8K non-causal 2.33 -> 1.93 ms).
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN, bool ACC>
__global__ void __launch_bounds__(64 * RA_BWD_DKDV_NW)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
bwd_dkdv_kernel(BwdArgs a, int num_kv_tiles) {
  constexpr int NW = RA_BWD_DKDV_NW, BK = 32 * NW;
  using Tile = STile<D, NW>;
  // per slot: Q tile, dO tile, lse2[TN], delta[TN]
  constexpr int SLOT = 2 * Tile::BYTES + 2 * TN * 4;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * SLOT];
  const uint32_t smem0 = lds_offset(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, h = lane >> 5;
  // Grouped heads with a partials buffer: one workgroup per (key tile, query head), so
  // that each sweeps the queries of one head (the workgroups running together on an XCD
  // then share Q/dO tiles in L2, and the work splits into group-times more pieces);
  // otherwise one per (key tile, key/value head), looping over the group's heads.
  const bool split = a.kv_part != nullptr;
  const int HB = (split ? a.Hq : a.Hkv) * a.B;
  const int bid = blockIdx.x;
  const int kt_i = bid / HB;  // ascending key tiles: lowest keys see the most queries
  int j = bid - kt_i * HB;
  if ((HB & 7) == 0) j = (j & 7) * (HB >> 3) + (j >> 3);
  const int hx = split ? a.Hq : a.Hkv;
  const int b = j / hx;
  const int hk = split ? (j % hx) / a.group : j % hx;
  const int hg0 = split ? (j % hx) % a.group : 0;  // first query head within the group
  const int ngroup = split ? 1 : a.group;         // query heads this workgroup covers
  const int k0 = kt_i * BK;
  const int krow = k0 + 32 * wave + r32;  // this lane's key (column of S)
  const int kr = min(krow, a.Skv - 1);
  const int64_t kpos = a.kv_offset + krow;
  const int64_t wk_first = a.kv_offset + k0 + 32 * wave;
  const int64_t wk_last = wk_first + 31;
  const bool wave_active = (k0 + 32 * wave) < a.Skv;
  const float c = a.scale_log2;

  const uint16_t *kb_ = (const uint16_t *)a.k + b * a.k_sb + hk * a.k_sh;
  const uint16_t *vb_ = (const uint16_t *)a.v + b * a.v_sb + hk * a.v_sh;
  // K^T and V^T as B operands: column = key, k = head dim 16*ks + 8h .. +8
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    kf[ks] = as_bf16x8(*(const u32x4 *)(kb_ + (int64_t)kr * a.k_ss + 16 * ks + 8 * h));
    vf[ks] = as_bf16x8(*(const u32x4 *)(vb_ + (int64_t)kr * a.v_ss + 16 * ks + 8 * h));
  }
  constexpr bool kW = D == 128;  // written-out MFMAs (see mfma_grad)
  // K^T and V^T are only ever MFMA B operands from here on: keep them in AGPRs
  if (kW) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      asm volatile("" : "+a"(kf[ks]));
      asm volatile("" : "+a"(vf[ks]));
    }
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
    if (kW) {
      asm volatile("" : "+a"(dk[dt]));  // the accumulators live in AGPRs from the start
      asm volatile("" : "+a"(dv[dt]));
    }
  }

  // Q/dO tile loads by the last two waves only: issuing them holds those waves back, so
  // the workgroup's waves reach their LDS-heavy MFMA phases at different times instead
  // of all together (6 % faster than loads by every wave; one loader, no gain)
  using LTile = STile<D, RA_BWD_DKDV_LOADERS>;
  const int lw = __builtin_amdgcn_readfirstlane(wave) - (NW - RA_BWD_DKDV_LOADERS);
  typename LTile::Lane TL;
  LTile::setup(TL, lane, max(lw, 0));  // on every wave: defined on one branch, it was spilled
  const uint32_t qpart = Tile::row_part(r32, h);
  const uint32_t tp0 = Tile::tr_part(lane, 0), tp1 = Tile::tr_part(lane, 1);
  // swizzled operand offsets of this lane within a tile: row reads per head-dim step ks,
  // transposed reads per sub-read s and head-dim block dt (a slot base is added once per
  // tile, the block offsets are immediates)
  uint32_t rx[D / 16], tx[2][D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) rx[ks] = qpart ^ (uint32_t)(32 * ks);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    tx[0][dt] = tp0 ^ (uint32_t)(64 * dt);
    tx[1][dt] = tp1 ^ (uint32_t)(64 * dt);
  }

  // First query row that can see this workgroup's first key (causal), as a tile start.
  int qstart = 0;
  if (CAUSAL) {
    const int64_t first = a.kv_offset + k0 - a.q_offset;
    qstart = first <= 0 ? 0 : (first >= (int64_t)a.Sq ? a.Sq : (int)first);
    qstart = (qstart / TN) * TN;
  }
  int qend = a.Sq;
  // Packed documents: this lane's key is seen by the queries of its document [ds, de)
  // (causal: [key, de)); the block's queries run from its first key's document start
  // to its last key's document end.
  int ds = 0, de = 0, w_ds_first = 0, w_ds_last = 0, w_de_first = 0, w_de_last = 0;
  if (VARLEN) {
    doc_bounds(a.cu, a.n_docs, kr, a.Sq, ds, de);
    w_ds_first = __builtin_amdgcn_readlane(ds, 0);
    w_ds_last = __builtin_amdgcn_readlane(ds, 31);
    w_de_first = __builtin_amdgcn_readlane(de, 0);
    w_de_last = __builtin_amdgcn_readlane(de, 31);
    const int klast = min(k0 + BK, a.Skv) - 1;
    int f_ds, f_de, l_ds, l_de;
    doc_bounds(a.cu, a.n_docs, min(k0, a.Skv - 1), a.Sq, f_ds, f_de);
    doc_bounds(a.cu, a.n_docs, klast, a.Sq, l_ds, l_de);
    if (!CAUSAL) qstart = (__builtin_amdgcn_readfirstlane(min(f_ds, k0)) / TN) * TN;
    qend = __builtin_amdgcn_readfirstlane(min(max(l_de, l_ds), a.Sq));
  }
  const int nqt = qstart >= qend ? 0 : (qend - qstart + TN - 1) / TN;
  const int total = nqt * ngroup;  // (query head, query tile) pairs

  // tile `it` is query tile qt of query head hk * group + hg (qt fastest); the pair is
  // advanced by one per tile instead of divided out of it
  auto issue = [&](int hg, int qt, uint32_t slot) {
    const int hq = hk * a.group + hg0 + hg;
    const int q0 = qstart + qt * TN;
    const uint16_t *qb = (const uint16_t *)a.q + b * a.q_sb + hq * a.q_sh;
    const uint16_t *dob = (const uint16_t *)a.dout + b * a.do_sb + hq * a.do_sh;
    if (lw >= 0) {
      LTile::load(TL, qb, a.q_ss, q0, a.Sq, slot, lw);
      LTile::load(TL, dob, a.do_ss, q0, a.Sq, slot + Tile::BYTES, lw);
    }
  };
  // lse (as exp2 offsets) and -delta of the tile's 64 rows: threads 0-127
  auto stats = [&](int hg, int qt, float &val) {
    const int hq = hk * a.group + hg0 + hg;
    const int q0 = qstart + qt * TN;
    const int i = tid & 63;
    const int q = min(q0 + i, a.Sq - 1);
    if (tid < 64) {
      const float l = a.lse[b * a.l_sb + hq * a.l_sh + q];
      val = l == -INFINITY ? INFINITY : l * kLog2e;
    } else if (tid < 128) {
      val = -a.delta[((int64_t)b * a.Hq + hq) * a.Sq + q];  // stored negated
    }
  };
  auto stats_store = [&](float val, uint32_t slot) {
    if (tid < 128) {
      const uint32_t at = slot + 2 * Tile::BYTES + (uint32_t)(4 * tid);
      *(__attribute__((address_space(3))) float *)(size_t)at = val;
    }
  };

  float sv = 0.f;
  if (total > 0) {
    issue(0, 0, smem0);
    stats(0, 0, sv);
    stats_store(sv, smem0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  int cur = 0;
  int qt_c = 0, hg_c = 0;  // this tile's query tile and head within the group
  for (int it = 0; it < total; ++it) {
    const uint32_t slot = smem0 + cur * SLOT;
    const bool has_next = it + 1 < total;
    int qt_n = qt_c + 1, hg_n = hg_c;
    if (qt_n == nqt) {
      qt_n = 0;
      ++hg_n;
    }
    if (has_next) {
      issue(hg_n, qt_n, smem0 + (cur ^ 1) * SLOT);
      stats(hg_n, qt_n, sv);
    }
    const int q0 = qstart + qt_c * TN;
    qt_c = qt_n;
    hg_c = hg_n;
    const int64_t qpos0 = a.q_offset + q0;
    // The two 32-query steps of the tile as one stream of 4*NST MFMAs, operands read
    // kDep MFMAs ahead:  [S,dP of step 0] [S,dP of step 1 | P,dS of step 0]
    // [dV,dK of step 0 | P,dS of step 1] [dV,dK of step 1].  A step with no visible
    // (query, key) pair for this wave is computed and masked to zero (diagonal only).
    const int qv0 = min(32, a.Sq - q0), qv1 = min(32, a.Sq - (q0 + 32));
    // packed documents: a step wholly outside every document of this wave's keys
    auto doc_out = [&](int sq) {
      return VARLEN && (sq >= w_de_last || (!CAUSAL && sq + 32 <= w_ds_first));
    };
    const bool vis0 = !(CAUSAL && wk_first > qpos0 + 31) && !doc_out(q0);
    const bool vis1 = qv1 > 0 && !(CAUSAL && wk_first > qpos0 + 63) && !doc_out(q0 + 32);
    if (wave_active && (vis0 || vis1)) {
      constexpr int NST = D / 8;  // MFMAs per stage
      // LDS operand reads kept in flight ahead of their MFMA; with two waves per SIMD
      // (64-dim heads) the other wave hides the read latency and the shorter lead
      // saves registers in the halved budget.
      constexpr int kDep = D == 64 ? 2 : 4;
      auto doc_cross = [&](int sq) {
        return VARLEN && (sq + 32 > w_de_first || (!CAUSAL && sq < w_ds_last));
      };
      const bool nm0 = qv0 < 32 || (CAUSAL && wk_last > qpos0) || doc_cross(q0);
      const bool nm1 = qv1 < 32 || (CAUSAL && wk_last > qpos0 + 32) || doc_cross(q0 + 32);
      f32x16 s0, dp0, s1, dp1;
      u32x4 pf0[2], dsf0[2], pf1[2], dsf1[2];
      uint32_t rb[D / 16], tb[2][D / 32];  // this tile's operand addresses
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) rb[ks] = slot + rx[ks];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        tb[0][dt] = slot + tx[0][dt];
        tb[1][dt] = slot + tx[1][dt];
      }
      auto operand = [&](int i) -> u32x4 {
        const int stage = i / NST, j = i % NST;
        const int qs = stage & 1;
        const uint32_t qo = (uint32_t)(32 * qs * Tile::RB);
        if (stage < 2) return lds_read_b128(rb[j >> 1] + qo + ((j & 1) ? Tile::BYTES : 0u));
        const int pj = j >> 1, s2 = pj / (D / 32), dt = pj % (D / 32);
        const uint32_t off = qo + ((j & 1) ? 0u : (uint32_t)Tile::BYTES) +
                             (uint32_t)(16 * s2 * Tile::RB);
        const u32x2 l2 = __builtin_bit_cast(u32x2, lds_read_tr16_b64(tb[0][dt] + off));
        const u32x2 h2 = __builtin_bit_cast(u32x2, lds_read_tr16_b64(tb[1][dt] + off));
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      };
      // lse of the 4 rows of element group g of step qs, read one group ahead of its use
      const uint32_t sbase = slot + 2 * Tile::BYTES + (uint32_t)(16 * h);
      auto stats_rd = [&](int qs, int g, f32x4 &lg) {
        lg = *(const __attribute__((address_space(3))) f32x4 *)(size_t)(
            sbase + (uint32_t)(4 * 32 * qs + 32 * g));
      };
      // -D of the 16 rows of this lane's elements in step qs: the initial accumulator of
      // the step's dP chain, so that dP - D comes out of the MFMAs
      auto negd_rd = [&](int qs) -> f32x16 {
        f32x16 r;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v4 = *(const __attribute__((address_space(3))) f32x4 *)(size_t)(
              sbase + (uint32_t)(4 * TN + 4 * 32 * qs + 32 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) r[4 * g + e] = v4[e];
        }
        return r;
      };
      f32x4 lgn;  // the next group's
      // P and dS of 4 elements (element group g) of step qs
      auto pds = [&](const f32x16 &sv_, const f32x16 &dpv, bool nm, int qv, int64_t sfirst,
                     int qs, int g, u32x4 (&pf)[2], u32x4 (&dsf)[2]) {
        const f32x4 lg = lgn;
        if (qs == 0 || g < 3) stats_rd(qs + (g == 3), (g + 1) & 3, lgn);
        float pv[4], dv4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = fast_exp2(fmaf(sv_[4 * g + e], c, -lg[e]));
        // the element mask only in steps that need it (a wave-uniform branch)
        if (__builtin_amdgcn_readfirstlane((int)nm)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            const int qi = (i >> 2) * 8 + 4 * h + (i & 3);
            if (qi >= qv || (CAUSAL && kpos > sfirst + qi)) pv[e] = 0.f;
            if (VARLEN) {  // packed documents (offsets are 0): the key's document only
              const int64_t qabs = sfirst + qi;
              if (qabs >= de || (!CAUSAL && qabs < ds)) pv[e] = 0.f;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dv4[e] = pv[e] * dpv[4 * g + e];  // dpv holds dP - D
        const int s2 = g >> 1;
        const bf16x2 p01 = __builtin_convertvector((f32x2){pv[0], pv[1]}, bf16x2);
        const bf16x2 p23 = __builtin_convertvector((f32x2){pv[2], pv[3]}, bf16x2);
        const bf16x2 d01 = __builtin_convertvector((f32x2){dv4[0], dv4[1]}, bf16x2);
        const bf16x2 d23 = __builtin_convertvector((f32x2){dv4[2], dv4[3]}, bf16x2);
        pf[s2][2 * (g & 1)] = __builtin_bit_cast(uint32_t, p01);
        pf[s2][2 * (g & 1) + 1] = __builtin_bit_cast(uint32_t, p23);
        dsf[s2][2 * (g & 1)] = __builtin_bit_cast(uint32_t, d01);
        dsf[s2][2 * (g & 1) + 1] = __builtin_bit_cast(uint32_t, d23);
      };
      // step 0's -D read first: it lands before the first operand the MFMAs wait for
      const f32x16 nd0 = negd_rd(0);
      f32x16 nd1;
      u32x4 op[kDep];
#pragma unroll
      for (int i = 0; i < kDep; ++i) op[i] = operand(i);
      __builtin_amdgcn_sched_barrier(0);
      // stage 0: S, dP of step 0
#pragma unroll
      for (int i = 0; i < NST; ++i) {
        const bf16x8 A = as_bf16x8(op[i % kDep]);
        if (i < 2) {
          if (i & 1) dp0 = mfma_score_c_ab<kW>(A, vf[0], nd0); else s0 = mfma_score0_ab<kW>(A, kf[0]);
        } else {
          if (i & 1) mfma_score_ab<kW>(dp0, A, vf[i >> 1]); else mfma_score_ab<kW>(s0, A, kf[i >> 1]);
        }
        op[i % kDep] = operand(i + kDep);
        // the MFMA reads its C operand over several cycles: the -D registers are not
        // reallocated until two MFMAs later
        if (i == 3) asm volatile("" ::"v"(nd0));
        if (i == NST / 2) nd1 = negd_rd(1);
        if (i == NST - 4) stats_rd(0, 0, lgn);
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage 1: S, dP of step 1 | P, dS of step 0
#pragma unroll
      for (int j = 0; j < NST; ++j) {
        const int i = NST + j;
        const bf16x8 A = as_bf16x8(op[i % kDep]);
        if (j < 2) {
          if (j & 1) dp1 = mfma_score_c_ab<kW>(A, vf[0], nd1); else s1 = mfma_score0_ab<kW>(A, kf[0]);
        } else {
          if (j & 1) mfma_score_ab<kW>(dp1, A, vf[j >> 1]); else mfma_score_ab<kW>(s1, A, kf[j >> 1]);
        }
        op[i % kDep] = operand(i + kDep);
        if (j == 3) asm volatile("" ::"v"(nd1));
        if (j % (NST / 4) == 1) pds(s0, dp0, nm0, qv0, qpos0, 0, j / (NST / 4), pf0, dsf0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage 2: dV, dK of step 0 | P, dS of step 1
#pragma unroll
      for (int j = 0; j < NST; ++j) {
        const int i = 2 * NST + j;
        const bf16x8 A = as_bf16x8(op[i % kDep]);
        const int pj = j >> 1, s2 = pj / (D / 32), dt = pj % (D / 32);
        if (j & 1) mfma_grad<kW>(dk[dt], A, as_bf16x8(dsf0[s2]));
        else mfma_grad<kW>(dv[dt], A, as_bf16x8(pf0[s2]));
        op[i % kDep] = operand(i + kDep);
        if (j % (NST / 4) == 1) pds(s1, dp1, nm1, qv1, qpos0 + 32, 1, j / (NST / 4), pf1, dsf1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // stage 3: dV, dK of step 1
#pragma unroll
      for (int j = 0; j < NST; ++j) {
        const int i = 3 * NST + j;
        const bf16x8 A = as_bf16x8(op[i % kDep]);
        const int pj = j >> 1, s2 = pj / (D / 32), dt = pj % (D / 32);
        if (j & 1) mfma_grad<kW>(dk[dt], A, as_bf16x8(dsf1[s2]));
        else mfma_grad<kW>(dv[dt], A, as_bf16x8(pf1[s2]));
        if (i + kDep < 4 * NST) op[i % kDep] = operand(i + kDep);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (has_next) stats_store(sv, smem0 + (cur ^ 1) * SLOT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed
    __syncthreads();
    cur ^= 1;
  }

  // the compiler does not see the asm MFMAs: give their results time to land before
  // the epilogue reads the accumulators
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // the lane half taken afresh: otherwise its 64-bit byte offset from the K/V loads is
  // held across the loop (64-dim heads at two waves per SIMD spill it)
  int he = h;
  asm volatile("" : "+v"(he));
  if (split && krow < a.Skv) {
    // this query head's unscaled fp32 partials, [2][B, Hq, Skv, D] contiguous
    const int64_t n_part = (int64_t)a.B * a.Hq * a.Skv * D;
    const int hq = hk * a.group + hg0;
    float *pk = a.kv_part + (((int64_t)b * a.Hq + hq) * a.Skv + krow) * D;
    float *pv = pk + n_part;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * he;
        *(f32x4 *)(pk + d) = f32x4{dk[dt][4 * g], dk[dt][4 * g + 1], dk[dt][4 * g + 2],
                                   dk[dt][4 * g + 3]};
        *(f32x4 *)(pv + d) = f32x4{dv[dt][4 * g], dv[dt][4 * g + 1], dv[dt][4 * g + 2],
                                   dv[dt][4 * g + 3]};
      }
  } else if (krow < a.Skv) {
    const int64_t krow_dk = b * a.dk_sb + hk * a.dk_sh + (int64_t)krow * a.dk_ss;
    const int64_t krow_dv = b * a.dv_sb + hk * a.dv_sh + (int64_t)krow * a.dv_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * he;
        if (ACC) {
          f32x4 *ak = (f32x4 *)((float *)a.dk + krow_dk + d);
          f32x4 *av = (f32x4 *)((float *)a.dv + krow_dv + d);
          const f32x4 pk = *ak, pv = *av;
          *ak = f32x4{pk[0] + dk[dt][4 * g] * a.scale, pk[1] + dk[dt][4 * g + 1] * a.scale,
                      pk[2] + dk[dt][4 * g + 2] * a.scale, pk[3] + dk[dt][4 * g + 3] * a.scale};
          *av = f32x4{pv[0] + dv[dt][4 * g], pv[1] + dv[dt][4 * g + 1], pv[2] + dv[dt][4 * g + 2],
                      pv[3] + dv[dt][4 * g + 3]};
          continue;
        }
        const bf16x2 k01 = __builtin_convertvector(
            (f32x2){dk[dt][4 * g] * a.scale, dk[dt][4 * g + 1] * a.scale}, bf16x2);
        const bf16x2 k23 = __builtin_convertvector(
            (f32x2){dk[dt][4 * g + 2] * a.scale, dk[dt][4 * g + 3] * a.scale}, bf16x2);
        *(u32x2 *)((uint16_t *)a.dk + krow_dk + d) =
            u32x2{__builtin_bit_cast(uint32_t, k01), __builtin_bit_cast(uint32_t, k23)};
        const bf16x2 v01 = __builtin_convertvector((f32x2){dv[dt][4 * g], dv[dt][4 * g + 1]}, bf16x2);
        const bf16x2 v23 =
            __builtin_convertvector((f32x2){dv[dt][4 * g + 2], dv[dt][4 * g + 3]}, bf16x2);
        *(u32x2 *)((uint16_t *)a.dv + krow_dv + d) =
            u32x2{__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
      }
  }
}

// dK, dV of grouped heads: the sum over the group's query heads of the partials, in head
// order (deterministic), scaled (dK) and rounded to bf16, or added to the fp32
// accumulators (ACC).  One thread per 8 head dims of one key; HBM-bound.
template <int D, bool ACC>
__global__ void __launch_bounds__(256) bwd_kv_reduce_kernel(BwdArgs a) {
  constexpr int CPK = D / 8;  // chunks of 8 dims per key
  const int64_t n_part = (int64_t)a.B * a.Hq * a.Skv * D;
  const int64_t nchunks = (int64_t)a.B * a.Hkv * a.Skv * CPK;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * 256) {
    const int d = (int)(c % CPK) * 8;
    const int64_t key_all = c / CPK;  // (b, hk, key)
    const int key = (int)(key_all % a.Skv);
    const int64_t bh = key_all / a.Skv;
    const int hk = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
    float sk[8], sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.f;
    for (int hg = 0; hg < a.group; ++hg) {
      const float *pk =
          a.kv_part + (((int64_t)b * a.Hq + hk * a.group + hg) * a.Skv + key) * D + d;
      const f32x4 k0 = *(const f32x4 *)pk, k1 = *(const f32x4 *)(pk + 4);
      const f32x4 v0 = *(const f32x4 *)(pk + n_part), v1 = *(const f32x4 *)(pk + n_part + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[e] += k0[e]; sk[4 + e] += k1[e];
        sv[e] += v0[e]; sv[4 + e] += v1[e];
      }
    }
    const int64_t ok = b * a.dk_sb + hk * a.dk_sh + (int64_t)key * a.dk_ss + d;
    const int64_t ov = b * a.dv_sb + hk * a.dv_sh + (int64_t)key * a.dv_ss + d;
    if (ACC) {
      f32x4 *ak = (f32x4 *)((float *)a.dk + ok), *av = (f32x4 *)((float *)a.dv + ov);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x4 pk = ak[q], pv = av[q];
        ak[q] = f32x4{pk[0] + sk[4 * q] * a.scale, pk[1] + sk[4 * q + 1] * a.scale,
                      pk[2] + sk[4 * q + 2] * a.scale, pk[3] + sk[4 * q + 3] * a.scale};
        av[q] = f32x4{pv[0] + sv[4 * q], pv[1] + sv[4 * q + 1], pv[2] + sv[4 * q + 2],
                      pv[3] + sv[4 * q + 3]};
      }
    } else {
      u32x4 wk, wv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2 k2 = __builtin_convertvector(
            (f32x2){sk[2 * q] * a.scale, sk[2 * q + 1] * a.scale}, bf16x2);
        const bf16x2 v2 = __builtin_convertvector((f32x2){sv[2 * q], sv[2 * q + 1]}, bf16x2);
        wk[q] = __builtin_bit_cast(uint32_t, k2);
        wv[q] = __builtin_bit_cast(uint32_t, v2);
      }
      *(u32x4 *)((uint16_t *)a.dk + ok) = wk;
      *(u32x4 *)((uint16_t *)a.dv + ov) = wv;
    }
  }
}

template <int D, bool CAUSAL, bool VARLEN = false, bool ACC = false>
int launch_bwd(const BwdArgs &a, hipStream_t stream) {
  // 1. D_i
  {
    const int64_t nrows = (int64_t)a.B * a.Hq * a.Sq;
    int64_t blocks = (nrows * (D / 8) + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  }
  // 2. dK, dV (with grouped heads and a partials buffer: per query head, then summed)
  {
    constexpr int BK = 32 * RA_BWD_DKDV_NW;
    const int nkt = (a.Skv + BK - 1) / BK;
    const bool split = a.kv_part != nullptr;
    const int64_t blocks = (int64_t)nkt * (split ? a.Hq : a.Hkv) * a.B;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN, ACC>), dim3((unsigned)blocks),
                         dim3(64 * RA_BWD_DKDV_NW), 0,
                         stream, a, nkt);
    const int64_t nchunks = (int64_t)a.B * a.Hkv * a.Skv * (D / 8);
    if (split && nchunks > 0) {
      int64_t rblocks = (nchunks + 255) / 256;
      if (rblocks > (1 << 20)) rblocks = 1 << 20;
      hipLaunchKernelGGL((bwd_kv_reduce_kernel<D, ACC>), dim3((unsigned)rblocks), dim3(256), 0,
                         stream, a);
    }
  }
  // 3. dQ
  {
    constexpr int BM = 32 * RA_BWD_DQ_NW;
    const int nqt = (a.Sq + BM - 1) / BM;
    const int64_t blocks = (int64_t)nqt * a.Hq * a.B;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN, ACC>), dim3((unsigned)blocks),
                         dim3(64 * RA_BWD_DQ_NW), 0, stream, a, nqt);
  }
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq) {
  const size_t n = (size_t)(B * Hq * Sq) * sizeof(float);
  return (n + 255) / 256 * 256;
}

size_t bwd_kv_part_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D) {
  if (Hkv <= 0 || Hq <= Hkv) return 0;
  const size_t n = 2 * (size_t)(B * Hq * Skv * D) * sizeof(float);
  return (n + 255) / 256 * 256;
}

int launch_attn_bwd_varlen(const BwdArgs &a, int D, int causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_bwd<128, true, true>(a, stream) : launch_bwd<128, false, true>(a, stream);
  if (D == 64)
    return causal ? launch_bwd<64, true, true>(a, stream) : launch_bwd<64, false, true>(a, stream);
  return RA_ERR_UNSUPPORTED;
}

int launch_attn_bwd_accum(const BwdArgs &a, int D, int causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_bwd<128, true, false, true>(a, stream)
                  : launch_bwd<128, false, false, true>(a, stream);
  if (D == 64)
    return causal ? launch_bwd<64, true, false, true>(a, stream)
                  : launch_bwd<64, false, false, true>(a, stream);
  return RA_ERR_UNSUPPORTED;
}

int launch_attn_bwd(const BwdArgs &a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_bwd<128, true>(a, stream) : launch_bwd<128, false>(a, stream);
  if (D == 64) return causal ? launch_bwd<64, true>(a, stream) : launch_bwd<64, false>(a, stream);
  return RA_ERR_UNSUPPORTED;
}

}  // namespace ra
