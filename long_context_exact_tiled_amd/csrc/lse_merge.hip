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
// Pure streaming (a few flops per 4-byte element): bound by HBM bandwidth.  A group of
// lanes (a power of two, never straddling a wavefront) owns one query row, each lane 4
// consecutive head-dim elements, so every part row is read once with 8- or 16-byte
// accesses and the output row is written once.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

template <bool PF32, bool OF32>
__global__ void __launch_bounds__(kThreads) lse_merge_kernel(MergeArgs a, int tpr_log2) {
  const int tpr = 1 << tpr_log2;
  const int rows_per_block = kThreads >> tpr_log2;
  const int sub = threadIdx.x & (tpr - 1);
  const int d0 = 4 * sub;
  const int64_t nrows = (int64_t)a.B * a.H * a.S;
  for (int64_t row = (int64_t)blockIdx.x * rows_per_block + (threadIdx.x >> tpr_log2); row < nrows;
       row += (int64_t)gridDim.x * rows_per_block) {
    const int s = (int)(row % a.S);
    const int64_t bh = row / a.S;
    const int hh = (int)(bh % a.H);
    const int b = (int)(bh / a.H);
    const int64_t loff = b * a.pl_sb + hh * a.pl_sh + s;

    float m = -INFINITY;
    for (int i = 0; i < a.n; ++i) m = fmaxf(m, a.lse_parts[i][loff]);
    float lse = -INFINITY;
    if (m != -INFINITY) {
      float z = 0.f;
      for (int i = 0; i < a.n; ++i) z += expf(a.lse_parts[i][loff] - m);
      lse = m + logf(z);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const bool active = d0 < a.D;
    if (lse != -INFINITY && active) {
      const int64_t poff = b * a.p_sb + hh * a.p_sh + (int64_t)s * a.p_ss + d0;
      for (int i = 0; i < a.n; ++i) {
        const float li = a.lse_parts[i][loff];
        if (li == -INFINITY) continue;  // empty partial: zero weight
        const float w = expf(li - lse);
        if (PF32) {
          const float4 x = *(const float4 *)((const float *)a.o_parts[i] + poff);
          acc[0] = fmaf(w, x.x, acc[0]);
          acc[1] = fmaf(w, x.y, acc[1]);
          acc[2] = fmaf(w, x.z, acc[2]);
          acc[3] = fmaf(w, x.w, acc[3]);
        } else {
          const u32x2 x = *(const u32x2 *)((const uint16_t *)a.o_parts[i] + poff);
          acc[0] = fmaf(w, bf16_bits_to_float(x[0] & 0xffffu), acc[0]);
          acc[1] = fmaf(w, bf16_bits_to_float(x[0] >> 16), acc[1]);
          acc[2] = fmaf(w, bf16_bits_to_float(x[1] & 0xffffu), acc[2]);
          acc[3] = fmaf(w, bf16_bits_to_float(x[1] >> 16), acc[3]);
        }
      }
    }
    if (active) {
      const int64_t ooff = b * a.o_sb + hh * a.o_sh + (int64_t)s * a.o_ss + d0;
      if (OF32) {
        float4 w = {acc[0], acc[1], acc[2], acc[3]};
        *(float4 *)((float *)a.o + ooff) = w;
      } else {
        u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *(u32x2 *)((uint16_t *)a.o + ooff) = w;
      }
      if (sub == 0) a.lse[b * a.l_sb + hh * a.l_sh + s] = lse;
    }
  }
}

}  // namespace

int launch_lse_merge(const MergeArgs &a, hipStream_t stream) {
  int tpr_log2 = 0;
  while ((1 << tpr_log2) < a.D / 4) ++tpr_log2;  // D <= 256 -> at most 64 lanes per row
  const int rows_per_block = kThreads >> tpr_log2;
  const int64_t nrows = (int64_t)a.B * a.H * a.S;
  int64_t blocks = (nrows + rows_per_block - 1) / rows_per_block;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (blocks <= 0) return RA_OK;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (a.parts_f32 && a.out_f32)
    hipLaunchKernelGGL((lse_merge_kernel<true, true>), grid, block, 0, stream, a, tpr_log2);
  else if (a.parts_f32)
    hipLaunchKernelGGL((lse_merge_kernel<true, false>), grid, block, 0, stream, a, tpr_log2);
  else if (a.out_f32)
    hipLaunchKernelGGL((lse_merge_kernel<false, true>), grid, block, 0, stream, a, tpr_log2);
  else
    hipLaunchKernelGGL((lse_merge_kernel<false, false>), grid, block, 0, stream, a, tpr_log2);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace ra
