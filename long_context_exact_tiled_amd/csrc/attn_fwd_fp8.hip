// attn_fwd_fp8 -- exact softmax attention over e4m3 (FP8) inputs with per-head scales,
// the ring walk and the online softmax of attn_fwd, on gfx950's 32x32x64 f8 MFMA.
//
// Sources (page title, host):
//   [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn), section
//        "那么，FlashAttention-2 和 -3 又改进了什么？": FlashAttention-3 supports the FP8
//        data type, halving key/value traffic; section "FlashAttention 如何破局？不只是
//        融合内核": tiling and the online softmax, as in attn_fwd.
//   [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com): the ring_attention_forward
//        listing (chunks visited in turn, log-space accumulation).
//
// Inputs: q, k codes [B, H, S, D] and v codes TRANSPOSED, [B, Hkv, D, S_pad] (keys
// contiguous), each with one fp32 descale per (batch, head): value = decode(code) *
// descale.  The descales of q and k fold into the softmax scale, v's into the epilogue.
//
// Design (the bf16 direct kernel's skeleton, shaped for a softmax that now costs more
// issue time than the MFMAs):
//   * 4 waves x 32 query rows per workgroup, three workgroups per CU (3 waves per SIMD):
//     their barriers are independent, so one workgroup's softmax runs under another's
//     MFMAs; K and V^T tiles of KN keys go from global memory straight into LDS
//     (global_load_lds_dwordx4), double-buffered, 16-byte chunks XOR-swizzled per row so
//     every operand read is a conflict-free ds_read_b128;
//   * S^T = K Q^T with 32x32x64 f8 MFMAs (Q in registers as the B operand): lane = one
//     query row, 16 of each 32 keys -- row max in registers plus one v_permlane32_swap;
//   * P' = 2^6 * exp2(c s - m) is rounded to e4m3 for O^T += V^T P'^T.  The 2^6 offset
//     and a lazy-rescale threshold of 2 (log2 units) keep P' <= 256 < 448 while all but
//     negligible weights (exp(s - max) >= 2^-12) stay in e4m3's normal range; the row
//     sum adds the unrounded fp32 values, so lse carries no fp8 rounding;
//   * after the f32 -> e4m3 conversion, one v_permlane32_swap per dword gathers each
//     64-key group's P'^T so that half h of the wave holds keys 32h .. 32h+31 in order:
//     the V^T operand is then a plain row read of 32 consecutive key bytes.
// The A and B operands of the f8 MFMA pair their bytes by (lane half, byte index), and
// the result has the usual 32x32 layout (both checked on the device).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Both operands e4m3 (format codes 0); zero scale operands select the unscaled form.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat8(const u32x4 &lo, const u32x4 &hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

constexpr float kP8Shift = 6.f;     // P' = 2^6 P
constexpr float kLazyFp8 = 2.f;     // running max lags the true one by < 2 (log2 units)
// Launch shape (measured on the 32K GQA workload, same call): 4 waves x 64-key tiles
// at 3 waves per SIMD (168 VGPRs, 32 KiB LDS, three workgroups per CU whose barriers are
// independent) 1.087 ms; 8 waves x 128-key tiles at 2 per SIMD 1.178 ms; 4 x 64 at 2
// per SIMD 1.155 ms.
#ifndef RA_FP8_KN
#define RA_FP8_KN 64                // keys per LDS tile
#endif
#ifndef RA_FP8_NW
#define RA_FP8_NW 4                 // waves (of 32 query rows) per workgroup
#endif
#ifndef RA_FP8_WPE
#define RA_FP8_WPE 3                // waves per SIMD the register budget is sized for
#endif

// 16-byte chunk swizzle of a row of RB bytes: rows sharing a 256-byte bank window
// keep their slots apart, and 16 consecutive rows at one chunk hit 16 distinct slots.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  return (r / (256 / RB)) % (RB / 16);
}

// Lane index, formed afresh where it is used: values derived from it that are only
// needed before or after the tile loop then hold no register across the loop.
__device__ __forceinline__ int lane_index() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

template <int D, int KN, int NW_>
struct Fp8Tile {
  static constexpr int NW = NW_;
  static constexpr int K_BYTES = KN * D;        // K tile: KN rows of D bytes
  static constexpr int V_BYTES = D * KN;        // V^T tile: D rows of KN bytes
  static constexpr int BUF = K_BYTES + V_BYTES;
  static constexpr int KBPW = K_BYTES / 1024 / NW;
  static constexpr int VBPW = V_BYTES / 1024 / NW;
  static_assert(K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0,
                "tiles split evenly into 1-KiB direct loads per wave");
  // rows between one lane's successive K (V^T) direct loads: a multiple of the swizzle's
  // 16-row period, so every load of a lane has the same swizzled column
  static constexpr int KRS = NW * 1024 / D;
  static constexpr int VRS = NW * 1024 / KN;
  static_assert(KRS % 16 == 0 && VRS % 16 == 0, "direct loads keep their swizzled column");
  static constexpr int KM = D / 64;   // 64-dim slices of a K row
  static constexpr int NG = KN / 64;   // 64-key groups of a V^T row
  struct Lane {
    int k_off, v_off;  // byte offsets of this lane's 16 bytes in its first K and V^T
                       // direct loads from the tile's first key (K row-major, V^T rows
                       // of keys); its i-th load is KRS i (VRS i) rows further on
    // operand read addresses in slot 0: K chunk 4m + 2h + e of row r, V^T chunk
    // 4g + 2h + e of row r (swizzled); block and slot offsets are immediates
    uint32_t ka[KM][2], va[NG][2];
  };

  // tile row and (swizzled) byte column of the 16 bytes lane `lane` of wave `wave` moves
  // in its i-th K or V^T direct load
  __device__ static void k_piece(int lane, int wave, int i, int &r, int &col) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    r = byte / D;
    col = 16 * (((byte % D) / 16) ^ swz<D>(r));
  }
  __device__ static void v_piece(int lane, int wave, int i, int &r, int &col) {
    const int byte = (wave + NW * i) * 1024 + 16 * lane;
    r = byte / KN;
    col = 16 * (((byte % KN) / 16) ^ swz<KN>(r));
  }

  __device__ static void setup(Lane &L, const FwdArgs &f, int lane, int wave, uint32_t smem0) {
    {
      int r, col;
      k_piece(lane, wave, 0, r, col);
      L.k_off = (int)(r * f.k_ss) + col;
      v_piece(lane, wave, 0, r, col);
      L.v_off = (int)(r * f.v_ss) + col;
    }
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
#pragma unroll
      for (int m = 0; m < KM; ++m)
        L.ka[m][e] = smem0 + (uint32_t)(r * D + 16 * ((4 * m + 2 * h + e) ^ swz<D>(r)));
#pragma unroll
      for (int g = 0; g < NG; ++g)
        L.va[g][e] = smem0 + K_BYTES + (uint32_t)(r * KN + 16 * ((4 * g + 2 * h + e) ^ swz<KN>(r)));
    }
  }

  // Direct loads of the tile at key kb into the LDS slot at byte offset `slot`.  Rows
  // past the last key read the last key; V^T 16-byte columns past the stored row read
  // its last 16 bytes.  Both are masked (their weights are exactly 0): kb is a multiple
  // of 16 (chunks of 16 keys, checked on the host), so a column that starts before the
  // last key lies wholly inside the padded row and is never clamped.  Away from the end
  // of the keys the lane offsets are the precomputed ones and only the scalar base moves.
  __device__ static void load(const Lane &L, const Fp8Args &a, const uint8_t *kbase,
                              const uint8_t *vbase, int kb, uint32_t slot, int wave) {
    const FwdArgs &f = a.f;
    if (kb + KN <= f.Skv && kb + KN <= a.vt_cols) {
      const uint8_t *kt = kbase + (int64_t)kb * f.k_ss;
      const uint8_t *vt = vbase + kb;
#pragma unroll
      for (int i = 0; i < KBPW; ++i)
        dma_b128(kt + (int64_t)(KRS * i) * f.k_ss, L.k_off,
                 slot + (uint32_t)__builtin_amdgcn_readfirstlane(wave + NW * i) * 1024);
#pragma unroll
      for (int i = 0; i < VBPW; ++i)
        dma_b128(vt + (int64_t)(VRS * i) * f.v_ss, L.v_off,
                 slot + K_BYTES + (uint32_t)__builtin_amdgcn_readfirstlane(wave + NW * i) * 1024);
      return;
    }
    // the last tile: clamp rows and columns.  These offsets are taken from the head's
    // first key: the load zero-extends its 32-bit lane offset, and a clamped column
    // can lie before the tile's own first key (a tile that starts in the last 16
    // columns of a padded V^T row).
    const int lane = lane_index();
#pragma unroll
    for (int i = 0; i < KBPW; ++i) {
      int r, col;
      k_piece(lane, wave, i, r, col);
      const int off = (int)(min(kb + r, f.Skv - 1) * f.k_ss) + col;
      dma_b128(kbase, off, slot + (uint32_t)__builtin_amdgcn_readfirstlane(wave + NW * i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < VBPW; ++i) {
      int r, col;
      v_piece(lane, wave, i, r, col);
      const int off = (int)(r * f.v_ss) + min(kb + col, a.vt_cols - 16);
      dma_b128(vbase, off, slot + K_BYTES + (uint32_t)__builtin_amdgcn_readfirstlane(wave + NW * i) * 1024);
    }
  }

  // K operand of S^T block mt, head-dim slice m (64 dims): row 32 mt + r, chunks
  // 4m + 2h + {0, 1}.  SLOT: byte offset of the LDS buffer (a compile-time constant).
  template <uint32_t SLOT>
  __device__ static i32x8 k_frag(const Lane &L, int mt, int m) {
    const uint32_t off = SLOT + (uint32_t)(32 * mt * D);
    return cat8(lds_read_b128(L.ka[m][0] + off), lds_read_b128(L.ka[m][1] + off));
  }
  // V^T operand of head-dim block dt, key group g (64 keys): row 32 dt + r, chunks
  // 4g + 2h + {0, 1} (keys 64g + 32h .. +32, in order).
  template <uint32_t SLOT>
  __device__ static i32x8 v_frag(const Lane &L, int dt, int g) {
    const uint32_t off = SLOT + (uint32_t)(32 * dt * KN);
    return cat8(lds_read_b128(L.va[g][0] + off), lds_read_b128(L.va[g][1] + off));
  }
};

// Next tile of the ring walk (chunks (start + t) mod P; inside a chunk, tiles stop at
// the last key visible to the block's last query).  t == P means done.
template <int KN>
__device__ __forceinline__ void ring_next_fp8(const FwdArgs &a, bool causal, int64_t vis_lim,
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

template <int D, bool CAUSAL, int KN, int NW, int WPE>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
attn_fwd_fp8_kernel(Fp8Args a) {
  using T = Fp8Tile<D, KN, NW>;
  constexpr int NMT = KN / 32;  // 32-key S^T blocks per tile
  constexpr int NG = KN / 64;   // 64-key PV groups per tile
  constexpr int BM = 32 * T::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * T::BUF];
  const FwdArgs &f = a.f;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int r32 = lane & 31;
  const int h = lane >> 5;

  const int HB = f.Hq * f.B;
  // Query tile: heaviest first; with a work counter (B*Hq not a multiple of 8) taken in
  // start order, so that faster XCDs take more tiles (same scheme as the bf16 kernel:
  // ticket mod grid, the last residue's holder restores the counter).
  __shared__ int s_job;
  int bid = blockIdx.x;
  if (f.sched != nullptr) {
    if (threadIdx.x == 0) {
      const unsigned long long g = gridDim.x;
      const unsigned long long tk = atomicAdd((unsigned long long *)f.sched, 1ull);
      const int job = (int)(tk % g);
      if (job == (int)g - 1) atomicAdd((unsigned long long *)f.sched, 0ull - g);
      s_job = job;
    }
    __syncthreads();
    bid = __builtin_amdgcn_readfirstlane(s_job);
  }
  const int trank = bid / HB;
  int j = bid - trank * HB;
  if ((HB & 7) == 0) j = (j & 7) * (HB >> 3) + (j >> 3);
  const int hq = j % f.Hq;
  const int b = j / f.Hq;
  const int qt = f.num_q_tiles - 1 - trank;
  const int hk = hq / f.group;

  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, f.Sq) - 1;
  const uint8_t *qbase = (const uint8_t *)f.q + b * f.q_sb + hq * f.q_sh;
  const uint8_t *kbase = (const uint8_t *)f.k + b * f.k_sb + hk * f.k_sh;
  const uint8_t *vbase = (const uint8_t *)f.v + b * f.v_sb + hk * f.v_sh;

  const int64_t wpos_first = f.q_offset + q0 + 32 * wave_u;
  const int64_t wpos_last = wpos_first + 31;
  const bool wave_active = (q0 + 32 * wave_u) < f.Sq;
  // (wave-uniform values: kept in scalar registers, which the compiler cannot prove for
  // loads that follow the work counter's atomic)
  auto uniform = [](float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
  };
  const float c = uniform(f.scale_log2 * a.q_desc[b * a.qd_sb + hq * a.qd_sh] *
                          a.k_desc[b * a.kd_sb + hk * a.kd_sh]);
  const float vdesc = uniform(a.v_desc[b * a.vd_sb + hk * a.vd_sh]);

  const uint32_t smem0 = lds_offset(smem);
  typename T::Lane L;
  T::setup(L, f, lane, wave, smem0);

  // Q as the B operand: head-dim slice m holds bytes 64m + 32h .. +32 of this row.
  i32x8 qf[D / 64];
  {
    const uint8_t *qr = qbase + (int64_t)min(q0 + 32 * wave + r32, f.Sq - 1) * f.q_ss;
#pragma unroll
    for (int m = 0; m < D / 64; ++m)
      qf[m] = cat8(*(const u32x4 *)(qr + 64 * m + 32 * h),
                   *(const u32x4 *)(qr + 64 * m + 32 * h + 16));
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  // exp2 offset -m_run + kP8Shift (kP8Shift while m_run is -inf) and the rescale test's
  // -(m_run + kLazyFp8), both changed only when m_run is
  float mneg = kP8Shift, nthr = INFINITY;
  float l_run = 0.f;

  const int64_t vis_lim = f.q_offset + qlast - f.kv_offset + 1;
  int t = -1, kb = 0, kend = 0, cend = 0;
  ring_next_fp8<KN>(f, CAUSAL, vis_lim, t, kb, kend, cend);
  if (t < f.num_chunks) T::load(L, a, kbase, vbase, kb, smem0, wave_u);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first tile have landed
  __syncthreads();

  // One tile: issue the next tile's loads into the other slot, then S^T, softmax and
  // O^T += V^T P'^T from slot CUR.  Returns false when the walk is done.  The loop runs
  // the two slots alternately so that every LDS operand offset is an immediate.
  auto tile = [&](auto cur_c) -> bool {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr uint32_t SLOT = (uint32_t)(CUR * T::BUF);
    const int kb_cur = kb, cend_cur = cend;
    ring_next_fp8<KN>(f, CAUSAL, vis_lim, t, kb, kend, cend);
    const bool has_next = t < f.num_chunks;
    if (has_next) T::load(L, a, kbase, vbase, kb, smem0 + (CUR ^ 1) * T::BUF, wave_u);

    const int64_t kpos0 = f.kv_offset + kb_cur;
    if (wave_active && !(CAUSAL && kpos0 > wpos_last)) {
      // S^T = K Q^T
      f32x16 s[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        s[mt] = mfma_fp8(T::template k_frag<SLOT>(L, mt, 0), qf[0], f32x16{});
#pragma unroll
        for (int m = 1; m < D / 64; ++m)
          s[mt] = mfma_fp8(T::template k_frag<SLOT>(L, mt, m), qf[m], s[mt]);
      }
      const int kvalid = min(KN, cend_cur - kb_cur);
      const bool need_mask = (kvalid < KN) || (CAUSAL && kpos0 + kvalid - 1 > wpos_first);
      if (need_mask) {
        // keys kk < lim are visible to this lane's row.  Row 32 wave + r sees
        // wpos_first + r - kpos0 + 1 keys of the tile; clamping the wave's term to
        // [-32, KN] changes no row's min(max(., 0), kvalid).
        const int ln = lane_index();
        int lim = kvalid;
        if (CAUSAL) {
          const int64_t w0 = wpos_first - kpos0 + 1;
          const int vis = (int)(w0 < -32 ? -32 : (w0 > KN ? KN : w0)) + (ln & 31);
          lim = min(lim, max(vis, 0));
        }
        lim -= 4 * (ln >> 5);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = 32 * mt + (i >> 2) * 8 + (i & 3);
            s[mt][i] = kk < lim ? s[mt][i] : -INFINITY;
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
      // c mx > m_run + kLazyFp8, as one FMA against the loop-carried -(m_run + kLazyFp8)
      if (__builtin_amdgcn_ballot_w64(fmaf(mx, c, nthr) > 0.f) != 0) {
        const float m_new = fmaxf(m_run, mx * c);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
        m_run = m_new;
        mneg = (m_new == -INFINITY ? 0.f : -m_new) + kP8Shift;
        nthr = -(m_new + kLazyFp8);
      }
      // P' -> e4m3, two values per conversion.  The first conversion of a dword fills its
      // low half and keeps the high half of its `old` operand, which the second
      // conversion overwrites: `old` is a score that is dead by then, so no register has
      // to be cleared or copied for it.
      // Dwords of block mt go straight into the P'^T operand of its 64-key group g = mt/2:
      // element 2 q4 + (mt & 1) holds the keys of registers 4 q4 .. 4 q4 + 3.
      i32x8 pf[NG];
      float acc0 = -0.f, acc1 = -0.f;  // x + -0 is x: the first additions fold away
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float p0 = fast_exp2(fmaf(s[mt][4 * q4 + 0], c, mneg));
          const float p1 = fast_exp2(fmaf(s[mt][4 * q4 + 1], c, mneg));
          const float p2 = fast_exp2(fmaf(s[mt][4 * q4 + 2], c, mneg));
          const float p3 = fast_exp2(fmaf(s[mt][4 * q4 + 3], c, mneg));
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[mt >> 1][2 * q4 + (mt & 1)],
                                                  false);
          pf[mt >> 1][2 * q4 + (mt & 1)] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
          acc0 += p0 + p1;
          acc1 += p2 + p3;
        }
      l_run += acc0 + acc1;
      // O^T += V^T P'^T, one 64-key group at a time.  The swap leaves half 0 with block
      // 2g's dword of its own and half 1's (keys 4w .. 4w+3 in dword w), half 1 with both
      // halves' block 2g+1 dwords: half h holds keys 32h .. 32h+31 in order.
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const auto sw = __builtin_amdgcn_permlane32_swap(pf[g][2 * q4], pf[g][2 * q4 + 1],
                                                           false, false);
          pf[g][2 * q4] = (int)sw[0];
          pf[g][2 * q4 + 1] = (int)sw[1];
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          o[dt] = mfma_fp8(T::template v_frag<SLOT>(L, dt, g), pf[g], o[dt]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile's direct loads landed
    __syncthreads();
    return has_next;
  };
  if (t < f.num_chunks) {
    while (tile(std::integral_constant<int, 0>{}) && tile(std::integral_constant<int, 1>{})) {
    }
  }

  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? vdesc / l_tot : 0.f;
  const int ln = lane_index();
  const int qrow = q0 + 32 * wave_u + (ln & 31);
  if (qrow < f.Sq) {
    const int he = ln >> 5;
    if (he == 0) {
      const float lse = l_tot > 0.f ? (m_run - kP8Shift + __log2f(l_tot)) * kLn2 : -INFINITY;
      f.lse[b * f.l_sb + hq * f.l_sh + qrow] = lse;
    }
    const int64_t orow = b * f.o_sb + hq * f.o_sh + (int64_t)qrow * f.o_ss;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * he;
        const float x0 = o[dt][4 * g4 + 0] * inv, x1 = o[dt][4 * g4 + 1] * inv;
        const float x2 = o[dt][4 * g4 + 2] * inv, x3 = o[dt][4 * g4 + 3] * inv;
        if (f.o_is_f32) {
          *(float4 *)((float *)f.o + orow + d) = float4{x0, x1, x2, x3};
        } else {
          const bf16x2 lo = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2){x2, x3}, bf16x2);
          *(u32x2 *)((uint16_t *)f.o + orow + d) =
              u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      }
  }
}

template <int D, bool CAUSAL>
int launch_fp8(const Fp8Args &args, hipStream_t stream) {
  Fp8Args a = args;
  constexpr int KN = RA_FP8_KN, NW = RA_FP8_NW;
  a.f.num_q_tiles = (a.f.Sq + 32 * NW - 1) / (32 * NW);
  const int64_t blocks = (int64_t)a.f.num_q_tiles * a.f.Hq * a.f.B;
  if (blocks <= 0) return RA_OK;
  if ((a.f.Hq * a.f.B) % 8 == 0) a.f.sched = nullptr;  // fixed XCD head map instead
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL, KN, NW, RA_FP8_WPE>), dim3((unsigned)blocks),
                     dim3(64 * NW), 0, stream, a);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace

int launch_attn_fwd_fp8(const Fp8Args &a, int D, int causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_fp8<128, true>(a, stream) : launch_fp8<128, false>(a, stream);
  if (D == 64) return causal ? launch_fp8<64, true>(a, stream) : launch_fp8<64, false>(a, stream);
  return RA_ERR_UNSUPPORTED;
}

}  // namespace ra
