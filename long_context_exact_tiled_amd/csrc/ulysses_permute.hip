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
// 16-byte vectors.  Rows are enumerated in the DESTINATION's order so the writes of a
// wavefront are contiguous; the reads are contiguous within each source row.  Pure data
// movement: bound by HBM bandwidth.
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

}  // namespace

int launch_ulysses_permute(const PermuteArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nranks * a.Hl * a.P * a.Sl;
  const int64_t nchunks = rows * (a.row_bytes / 16);
  if (nchunks <= 0) return RA_OK;
  int64_t blocks = (nchunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, nchunks);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // namespace ra
