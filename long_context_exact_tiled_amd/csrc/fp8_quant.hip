// fp8_quantize -- bf16 [B, H, S, D] -> e4m3 codes with one fp32 scale per (batch, head),
// optionally transposed to [B, H, D, S_pad] (the V^T layout the FP8 attention reads).
//
// [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn), section
// "那么，FlashAttention-2 和 -3 又改进了什么？": FlashAttention-3 supports the FP8 data
// type, halving the key/value traffic.  The scaling rule is a reading (the pages give none):
// with a = max |x| over the head, codes = e4m3(clamp(x * (448 / a), -448, 448)) with an
// fp32 multiply and round-to-nearest-even conversion, descale = a / 448 (an all-zero
// head: 1, 1); the value of a code is decode(code) * descale.
//
// Two passes, both bound by HBM bandwidth and deterministic (a max does not depend on
// the order it is taken in): partial maxima per (head, row range) into the workspace,
// then every block folds its head's partials and converts its rows (or, transposed,
// a 64-token x D tile through LDS).  Up to four tensors (q, k and v of a layer) share the
// two launches: each tensor owns a contiguous range of either grid's blocks.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.f;

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // `red` may still be read from a previous call
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// max |x| of 8 bf16 values
__device__ __forceinline__ float absmax8(const u32x4 &x) {
  float m = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    m = fmaxf(m, fabsf(bf16_bits_to_float(x[w] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_bits_to_float(x[w] >> 16)));
  }
  return m;
}

// The tensors of one launch: tensor i owns blocks [amax0[i], amax0[i+1]) of the max pass
// and [conv0[i], conv0[i+1]) of the conversion pass.
constexpr int kMaxQuant = RA_MAX_QUANT_TENSORS;
struct QuantMulti {
  QuantArgs t[kMaxQuant];
  int32_t amax0[kMaxQuant + 1];
  int32_t conv0[kMaxQuant + 1];
  int32_t ntiles[kMaxQuant];  // transposed tensors: 64-token tiles per head
  int32_t n;
};

// the tensor owning block `bid` of a pass whose block ranges start at `base` (uniform)
__device__ __forceinline__ int owner(const int32_t *base, int n, int bid) {
  int i = 0;
  while (i + 1 < n && bid >= base[i + 1]) ++i;
  return i;
}

// Rows of a block's range go round its threads RPP = kThreads / ppr rows at a time
// (ppr 16-byte pieces per row, at most 32): thread x takes piece x % ppr of rows
// x / ppr, x / ppr + RPP, ... (threads past RPP * ppr idle), so the loop divides nothing.
__device__ __forceinline__ void amax_block(const QuantArgs &a, int blk, float *red) {
  const int bh = blk / a.nsplit, sp = blk % a.nsplit;
  const int b = bh / a.H, h = bh % a.H;
  const int r0 = sp * a.rows_per_split, r1 = min(a.S, r0 + a.rows_per_split);
  const int ppr = a.D / 8, rpp = kThreads / ppr;
  const int rl = threadIdx.x / ppr, c = threadIdx.x - rl * ppr;
  const uint16_t *src = a.src + b * a.s_sb + h * a.s_sh + 8 * c;
  float m = 0.f;
  if (rl < rpp) {
    int r = r0 + rl;
    for (; r + 3 * rpp < r1; r += 4 * rpp) {  // four loads in flight
      u32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *(const u32x4 *)(src + (int64_t)(r + u * rpp) * a.s_ss);
#pragma unroll
      for (int u = 0; u < 4; ++u) m = fmaxf(m, absmax8(x[u]));
    }
    for (; r < r1; r += rpp) m = fmaxf(m, absmax8(*(const u32x4 *)(src + (int64_t)r * a.s_ss)));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) a.partial[blk] = m;
}

__global__ void __launch_bounds__(kThreads) quant_amax_kernel(QuantMulti m) {
  __shared__ float red[4];
  const int i = owner(m.amax0, m.n, (int)blockIdx.x);
  amax_block(m.t[i], (int)blockIdx.x - m.amax0[i], red);
}

// The head's max from its partials; r = 448 / a (fp32, correctly rounded division).
__device__ __forceinline__ float head_ratio(const QuantArgs &a, int bh, bool write_descale,
                                            float *red) {
  float m = 0.f;
  for (int i = threadIdx.x; i < a.nsplit; i += kThreads) m = fmaxf(m, a.partial[bh * a.nsplit + i]);
  m = block_max(m, red);
  if (write_descale && threadIdx.x == 0) {
    const int b = bh / a.H, h = bh % a.H;
    a.descale[b * a.ds_sb + h * a.ds_sh] = m > 0.f ? m / kE4m3Max : 1.f;
  }
  return m > 0.f ? kE4m3Max / m : 1.f;
}

// Two values -> two e4m3 codes in the low (HI = false) or high 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ int cvt2(float x0, float x1, float r, int old) {
  const float y0 = fminf(fmaxf(x0 * r, -kE4m3Max), kE4m3Max);
  const float y1 = fminf(fmaxf(x1 * r, -kE4m3Max), kE4m3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, old, HI);
}

__device__ __forceinline__ u32x2 cvt8(const u32x4 &x, float r) {
  uint32_t out[2];
#pragma unroll
  for (int w2 = 0; w2 < 2; ++w2) {
    const uint32_t a0 = x[2 * w2], a1 = x[2 * w2 + 1];
    int v = cvt2<false>(bf16_bits_to_float(a0 & 0xffffu), bf16_bits_to_float(a0 >> 16), r, 0);
    v = cvt2<true>(bf16_bits_to_float(a1 & 0xffffu), bf16_bits_to_float(a1 >> 16), r, v);
    out[w2] = (uint32_t)v;
  }
  return u32x2{out[0], out[1]};
}

__device__ __forceinline__ void convert_block(const QuantArgs &a, int blk, float *red) {
  const int bh = blk / a.nsplit, sp = blk % a.nsplit;
  const int b = bh / a.H, h = bh % a.H;
  const float r = head_ratio(a, bh, sp == 0, red);
  const int r0 = sp * a.rows_per_split, r1 = min(a.S, r0 + a.rows_per_split);
  const int ppr = a.D / 8, rpp = kThreads / ppr;  // as in the max pass
  const int rl = threadIdx.x / ppr, c = threadIdx.x - rl * ppr;
  if (rl >= rpp) return;
  const uint16_t *src = a.src + b * a.s_sb + h * a.s_sh + 8 * c;
  uint8_t *dst = a.dst + b * a.d_sb + h * a.d_sh + 8 * c;
  int row = r0 + rl;
  for (; row + rpp < r1; row += 2 * rpp) {  // two rows in flight
    const u32x4 x0 = *(const u32x4 *)(src + (int64_t)row * a.s_ss);
    const u32x4 x1 = *(const u32x4 *)(src + (int64_t)(row + rpp) * a.s_ss);
    *(u32x2 *)(dst + (int64_t)row * a.d_s2) = cvt8(x0, r);
    *(u32x2 *)(dst + (int64_t)(row + rpp) * a.d_s2) = cvt8(x1, r);
  }
  if (row < r1)
    *(u32x2 *)(dst + (int64_t)row * a.d_s2) = cvt8(*(const u32x4 *)(src + (int64_t)row * a.s_ss), r);
}

// Transposed: one block per (head, 64-token tile).  Codes go through LDS as
// [D][64 + 4] bytes; each output row piece is 16 consecutive tokens of one head dim.
// Tokens S .. S_pad-1 get code 0.
constexpr int kTT = 64;           // tokens per tile
constexpr int kTRow = kTT + 4;    // LDS row bytes (4-byte aligned, spreads banks)

__device__ __forceinline__ void convert_t_block(const QuantArgs &a, int blk, int ntiles,
                                                float *red, uint8_t *tile) {
  const int bh = blk / ntiles, tt = blk % ntiles;
  const int b = bh / a.H, h = bh % a.H;
  const float r = head_ratio(a, bh, tt == 0, red);
  const int t0 = tt * kTT;
  const int ppr = a.D / 8;
  const uint16_t *src = a.src + b * a.s_sb + h * a.s_sh;
  for (int p = threadIdx.x; p < kTT * ppr; p += kThreads) {
    const int tok = p / ppr, c = p % ppr;
    u32x2 codes = u32x2{0u, 0u};
    if (t0 + tok < a.S)
      codes = cvt8(*(const u32x4 *)(src + (int64_t)(t0 + tok) * a.s_ss + 8 * c), r);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      tile[(8 * c + i) * kTRow + tok] = (uint8_t)(codes[i >> 2] >> (8 * (i & 3)));
  }
  __syncthreads();
  uint8_t *dst = a.dst + b * a.d_sb + h * a.d_sh;
  for (int p = threadIdx.x; p < a.D * (kTT / 16); p += kThreads) {
    const int d = p / (kTT / 16), k16 = p % (kTT / 16);
    const int col = t0 + 16 * k16;
    if (col >= a.S_pad) continue;
    const uint32_t *src4 = (const uint32_t *)(tile + d * kTRow + 16 * k16);
    *(u32x4 *)(dst + (int64_t)d * a.d_s2 + col) = u32x4{src4[0], src4[1], src4[2], src4[3]};
  }
}

// second pass of every tensor of the launch, transposed or not (a block-uniform branch)
__global__ void __launch_bounds__(kThreads) quant_convert_kernel(QuantMulti m) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[256 * kTRow];
  const int i = owner(m.conv0, m.n, (int)blockIdx.x);
  const int blk = (int)blockIdx.x - m.conv0[i];
  if (m.t[i].transpose)
    convert_t_block(m.t[i], blk, m.ntiles[i], red, tile);
  else
    convert_block(m.t[i], blk, red);
}

}  // namespace

// Row ranges of both passes: about 128 KiB of bf16 per block, at most 1024 per head
// (64, 32 and 16 KiB measured within 3 %).
void quant_split(int64_t S, int64_t D, int32_t &nsplit, int32_t &rows_per_split) {
  constexpr int64_t kBytes = 128 << 10;
  int64_t n = (S * D * 2 + kBytes - 1) / kBytes;
  n = n < 1 ? 1 : (n > 1024 ? 1024 : n);
  int64_t rps = S > 0 ? (S + n - 1) / n : 1;
  nsplit = (int32_t)(S > 0 ? (S + rps - 1) / rps : 1);
  rows_per_split = (int32_t)rps;
}

int launch_fp8_quantize_n(const QuantArgs *a, int n, hipStream_t stream) {
  QuantMulti m{};
  int k = 0;
  int64_t na = 0, nc = 0;
  m.amax0[0] = m.conv0[0] = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t nbh = (int64_t)a[i].B * a[i].H;
    if (nbh == 0) continue;  // nothing to quantize, no descale to write
    m.t[k] = a[i];
    // transposed: at least one tile per head, so that an empty head gets its descale
    m.ntiles[k] = a[i].transpose ? (a[i].S_pad > 0 ? (a[i].S_pad + kTT - 1) / kTT : 1) : 0;
    na += nbh * a[i].nsplit;
    nc += nbh * (a[i].transpose ? m.ntiles[k] : a[i].nsplit);
    m.amax0[k + 1] = (int32_t)na;
    m.conv0[k + 1] = (int32_t)nc;
    ++k;
  }
  if (k == 0) return RA_OK;
  m.n = k;
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)na), dim3(kThreads), 0, stream, m);
  hipLaunchKernelGGL(quant_convert_kernel, dim3((unsigned)nc), dim3(kThreads), 0, stream, m);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

int launch_fp8_quantize(const QuantArgs &a, hipStream_t stream) {
  return launch_fp8_quantize_n(&a, 1, stream);
}

}  // namespace ra
