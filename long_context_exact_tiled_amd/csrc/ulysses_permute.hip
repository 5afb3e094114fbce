// ulysses_permute -- the local layout step of Ulysses sequence parallelism:
// sequence shards [P, S/P, H, D] <-> head shards [H/P, S, D] (per rank), bit-exact.
//
// [P4] "ms-swift集成FlashAttention 2/3，长文本训练更高效" (maplevalley.com.cn), section
// "Ulysses：强互联下的高速通路": the input is cut into per-device sequence shards; one
// all-to-all before attention gives each device the whole sequence (here: of its head
// subset), one after attention restores the sequence order of the output.  On one GPU
// this kernel is the pack/unpack that would bracket that all-to-all.
//
// A row is D contiguous elements (a multiple of 16 bytes); every row moves as whole
// 16-byte vectors.  Pure data movement, bound by HBM bandwidth -- provided the index
// arithmetic stays out of the way: the main kernel takes (shard, rank and head, token
// tile) from the grid and (row, 16-byte column) from the thread index, so no thread
// divides; every wavefront reads and writes whole rows.  Row sizes other than 128, 256
// or 512 bytes use a flat kernel that decodes each 16-byte chunk's position by division.
#include "common.h"
#include "internal.h"

namespace ra {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(kThreads) permute_kernel(PermuteArgs a, int64_t nchunks) {
  const int cpr = a.row_bytes / 16;  // 16-byte chunks per row
  const int64_t S = (int64_t)a.P * a.Sl;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; idx < nchunks; idx += stride * kUnroll) {
    u32x4 val[kUnroll];
    int64_t dst_off[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t id = idx + u * stride;
      ok[u] = id < nchunks;
      if (!ok[u]) continue;
      const int64_t row = id / cpr;
      const int c = (int)(id % cpr);
      int64_t rr, hh, s, t;
      if (a.dir == 0) {
        // destination order (rank, head, token)
        const int64_t j = row % S;
        const int64_t rh = row / S;
        hh = rh % a.Hl;
        rr = rh / a.Hl;
        s = j / a.Sl;
        t = j % a.Sl;
      } else {
        // destination order (shard, token, head) over the rank's head slice
        hh = row % a.Hl;
        const int64_t rst = row / a.Hl;
        t = rst % a.Sl;
        const int64_t rs = rst / a.Sl;
        s = rs % a.P;
        rr = rs / a.P;
      }
      const int64_t rank = a.rank0 + rr;
      const int64_t seq_off =
          s * a.seq_s0 + t * a.seq_s1 + (rank * a.Hl + hh) * a.seq_s2;
      const int64_t head_off = rr * a.head_s0 + hh * a.head_s1 + (s * a.Sl + t) * a.head_s2;
      const int64_t src_off = a.dir == 0 ? seq_off : head_off;
      dst_off[u] = a.dir == 0 ? head_off : seq_off;
      val[u] = *(const u32x4 *)((const unsigned char *)a.src + src_off * a.elem_bytes + 16 * c);
      dst_off[u] = dst_off[u] * a.elem_bytes + 16 * c;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (ok[u]) *(u32x4 *)((unsigned char *)a.dst + dst_off[u]) = val[u];
  }
}

// grid (token tiles, shard s, rank-and-head rr * Hl + hh); CPR 16-byte chunks per row
constexpr int kRowUnroll = 4;
template <int CPR>
__global__ void __launch_bounds__(kThreads) permute_rows_kernel(PermuteArgs a) {
  constexpr int RPB = kThreads / CPR;  // rows per pass of the block
  const int rl = threadIdx.x / CPR, c = threadIdx.x % CPR;
  const int s = blockIdx.y;
  const int rh = blockIdx.z;
  const int hh = rh % a.Hl, rr = rh / a.Hl;  // wave-uniform
  const int64_t rank = a.rank0 + rr;
  const int64_t seq_base = s * a.seq_s0 + (rank * a.Hl + hh) * a.seq_s2;
  const int64_t head_base = rr * a.head_s0 + hh * a.head_s1 + (int64_t)s * a.Sl * a.head_s2;
  const int64_t src_base = a.dir == 0 ? seq_base : head_base;
  const int64_t dst_base = a.dir == 0 ? head_base : seq_base;
  const int64_t src_rs = a.dir == 0 ? a.seq_s1 : a.head_s2;  // row strides (elements)
  const int64_t dst_rs = a.dir == 0 ? a.head_s2 : a.seq_s1;
  const unsigned char *src = (const unsigned char *)a.src + 16 * c;
  unsigned char *dst = (unsigned char *)a.dst + 16 * c;
  const int t0 = blockIdx.x * (RPB * kRowUnroll) + rl;
  u32x4 val[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int t = t0 + u * RPB;
    if (t < a.Sl) val[u] = *(const u32x4 *)(src + (src_base + t * src_rs) * a.elem_bytes);
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const int t = t0 + u * RPB;
    if (t < a.Sl) *(u32x4 *)(dst + (dst_base + t * dst_rs) * a.elem_bytes) = val[u];
  }
}

}  // namespace

int launch_ulysses_permute(const PermuteArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nranks * a.Hl * a.P * a.Sl;
  const int64_t nchunks = rows * (a.row_bytes / 16);
  if (nchunks <= 0) return RA_OK;
  const int cpr = a.row_bytes / 16;
  const int64_t rh = (int64_t)a.nranks * a.Hl;
  if ((cpr == 8 || cpr == 16 || cpr == 32) && a.P <= 65535 && rh <= 65535) {
    const int64_t rows_per_block = (int64_t)(kThreads / cpr) * kRowUnroll;
    const dim3 grid((unsigned)((a.Sl + rows_per_block - 1) / rows_per_block), (unsigned)a.P,
                    (unsigned)rh);
    if (cpr == 8)
      hipLaunchKernelGGL(permute_rows_kernel<8>, grid, dim3(kThreads), 0, stream, a);
    else if (cpr == 16)
      hipLaunchKernelGGL(permute_rows_kernel<16>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(permute_rows_kernel<32>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
  }
  int64_t blocks = (nchunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, nchunks);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace ra
