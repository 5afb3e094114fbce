// lse_merge -- combine n partial attention results (o_i, lse_i) over disjoint key sets.
//
// [P1] "ms-swift支持Ulysses与Ring-Attention降低长文本显存占用" (bjdmk.com.cn), section
// "Ring-Attention：面向大规模部署的工程利器": each device keeps a local max and local
// exponential sum; the global max is the max of the local ones and the global
// normaliser sums every exponential shifted by the global max.  For partials that are
// already normalised by their own lse this is
//     m = max_i lse_i,  lse = m + ln sum_i exp(lse_i - m),  o = sum_i exp(lse_i - lse) o_i.
// [P2] "Ulysses与Ring-Attention序列并行技术详解" (cnvsn.com), ring_attention_forward listing:
// the same weighted average, folded one ring step at a time.
//
// Pure streaming (a few flops per element): bound by HBM bandwidth.  A group of lanes (a
// power of two, never straddling a wavefront) owns one query row, each lane 16 bytes of
// every part row (4 fp32 or 8 bf16 elements), so every part row is read once and the
// output row written once.  Parts are taken CH at a time (2, 4 or 8, the smallest that
// holds n up to 8) for 8 / CH rows per lane group: all their lse values and row pieces
// are loaded before any arithmetic, so a lane always has 8 independent 16-byte loads in
// flight; the chunks are folded with a running max (the same rescaling as the online
// softmax), so any number of parts is a single pass.  An empty part (lse = -inf)
// gets weight 0 by selection, whatever its o holds.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // 16-byte part loads in flight per lane (parts x rows)

// 16 bytes of a part row as fp32 values: 4 fp32 or 8 bf16 elements.
__device__ __forceinline__ void widen_f32(const u32x4 &x, float (&f)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = x[k];  // bit-cast a scalar copy: a cast of the element itself read lane 0
    f[k] = __builtin_bit_cast(float, u);
  }
}
__device__ __forceinline__ void widen_bf16(const u32x4 &x, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_bits_to_float(x[k] & 0xffffu);
    f[2 * k + 1] = bf16_bits_to_float(x[k] >> 16);
  }
}

template <bool PF32, bool OF32, int CH>
__global__ void __launch_bounds__(kThreads) lse_merge_kernel(MergeArgs a, int tpr_log2) {
  constexpr int EPL = PF32 ? 4 : 8;  // elements per lane
  constexpr int R = kInFlight / CH;   // rows per lane group and pass
  const int tpr = 1 << tpr_log2;
  const int groups = kThreads >> tpr_log2;  // lane groups (rows) per block and step
  const int sub = threadIdx.x & (tpr - 1);
  const int d0 = EPL * sub;
  const bool active = d0 < a.D;
  const int64_t nrows = (int64_t)a.B * a.H * a.S;
  for (int64_t row0 = (int64_t)blockIdx.x * groups * R + (threadIdx.x >> tpr_log2); row0 < nrows;
       row0 += (int64_t)gridDim.x * groups * R) {
    int64_t loff[R], poff[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + (int64_t)r * groups;
      ok[r] = row < nrows;
      const int64_t rr = ok[r] ? row : row0;
      const int s = (int)(rr % a.S);
      const int64_t bh = rr / a.S;
      const int hh = (int)(bh % a.H);
      const int b = (int)(bh / a.H);
      loff[r] = b * a.pl_sb + hh * a.pl_sh + s;
      poff[r] = (b * a.p_sb + hh * a.p_sh + (int64_t)s * a.p_ss + d0) * (PF32 ? 4 : 2);
    }

    float m[R], z[R], acc[R][EPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = -INFINITY;
      z[r] = 0.f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) acc[r][k] = 0.f;
    }
    for (int base = 0; base < a.n; base += CH) {
      const int cnt = min(CH, a.n - base);
      float li[R][CH];
      u32x4 x[R][CH];
#pragma unroll
      for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          li[r][j] = -INFINITY;
          x[r][j] = u32x4{0u, 0u, 0u, 0u};
          if (j < cnt) {
            li[r][j] = a.lse_parts[base + j][loff[r]];
            if (active) x[r][j] = *(const u32x4 *)((const char *)a.o_parts[base + j] + poff[r]);
          }
        }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float mc = m[r];
#pragma unroll
        for (int j = 0; j < CH; ++j) mc = fmaxf(mc, li[r][j]);
        if (mc == -INFINITY) continue;  // every part so far is empty
        const float sc = expf(m[r] - mc);  // 0 while m is still -inf
        z[r] *= sc;
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[r][k] *= sc;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const bool empty = li[r][j] == -INFINITY;
          const float w = empty ? 0.f : expf(li[r][j] - mc);
          z[r] += w;
          float f[EPL];
          if constexpr (PF32)
            widen_f32(x[r][j], f);
          else
            widen_bf16(x[r][j], f);
#pragma unroll
          for (int k = 0; k < EPL; ++k) acc[r][k] = empty ? acc[r][k] : fmaf(w, f[k], acc[r][k]);
        }
        m[r] = mc;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!ok[r] || !active) continue;
      const int64_t row = row0 + (int64_t)r * groups;
      const int s = (int)(row % a.S);
      const int64_t bh = row / a.S;
      const int hh = (int)(bh % a.H);
      const int b = (int)(bh / a.H);
      const float lse = z[r] > 0.f ? m[r] + logf(z[r]) : -INFINITY;
      const float inv = z[r] > 0.f ? 1.f / z[r] : 0.f;
      const int64_t ooff = b * a.o_sb + hh * a.o_sh + (int64_t)s * a.o_ss + d0;
      if constexpr (OF32) {
#pragma unroll
        for (int k = 0; k < EPL; k += 4)
          *(float4 *)((float *)a.o + ooff + k) = float4{acc[r][k] * inv, acc[r][k + 1] * inv,
                                                        acc[r][k + 2] * inv, acc[r][k + 3] * inv};
      } else if constexpr (EPL == 8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = pack_bf16x2(acc[r][2 * k] * inv, acc[r][2 * k + 1] * inv);
        *(u32x4 *)((uint16_t *)a.o + ooff) = w;
      } else {
        u32x2 w = {pack_bf16x2(acc[r][0] * inv, acc[r][1] * inv),
                   pack_bf16x2(acc[r][2] * inv, acc[r][3] * inv)};
        *(u32x2 *)((uint16_t *)a.o + ooff) = w;
      }
      if (sub == 0) a.lse[b * a.l_sb + hh * a.l_sh + s] = lse;
    }
  }
}

template <bool PF32, bool OF32, int CH>
void launch(const MergeArgs &a, hipStream_t stream) {
  constexpr int EPL = PF32 ? 4 : 8;
  constexpr int R = kInFlight / CH;
  int tpr_log2 = 0;
  while ((1 << tpr_log2) < a.D / EPL) ++tpr_log2;  // D <= 256 -> at most 64 lanes per row
  const int64_t rows_per_block = (int64_t)(kThreads >> tpr_log2) * R;
  const int64_t nrows = (int64_t)a.B * a.H * a.S;
  int64_t blocks = (nrows + rows_per_block - 1) / rows_per_block;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (blocks <= 0) return;
  hipLaunchKernelGGL((lse_merge_kernel<PF32, OF32, CH>), dim3((unsigned)blocks), dim3(kThreads),
                     0, stream, a, tpr_log2);
}

template <bool PF32, bool OF32>
void launch_n(const MergeArgs &a, hipStream_t stream) {
  if (a.n <= 2)
    launch<PF32, OF32, 2>(a, stream);
  else if (a.n <= 4)
    launch<PF32, OF32, 4>(a, stream);
  else
    launch<PF32, OF32, 8>(a, stream);
}

}  // namespace

int launch_lse_merge(const MergeArgs &a, hipStream_t stream) {
  if (a.parts_f32 && a.out_f32)
    launch_n<true, true>(a, stream);
  else if (a.parts_f32)
    launch_n<true, false>(a, stream);
  else if (a.out_f32)
    launch_n<false, true>(a, stream);
  else
    launch_n<false, false>(a, stream);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace ra
