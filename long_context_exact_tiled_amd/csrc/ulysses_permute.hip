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
// Several tensors (q, k and v of a layer) can move in one launch: the grid's z axis
// runs over the (rank, head) ranges of every pair in turn.
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

// Up to this many (src, dst) pairs share one launch; the z extent of the grid is the
// concatenation of their (rank, head) ranges.
constexpr int kMaxPairs = RA_MAX_PERMUTE_TENSORS;
struct PairArgs {
  PermuteArgs t[kMaxPairs];
  int32_t zbase[kMaxPairs + 1];  // pair i owns grid z in [zbase[i], zbase[i+1])
  int32_t n;
};

// grid (token tiles, shard s, rank-and-head rr * Hl + hh of pair i, pairs concatenated);
// CPR 16-byte chunks per row, one chunk per thread: a block moves 4 KiB.  Small blocks
// spread a launch over the chip fastest; 2, 4 and 8 rows per thread measured 5 %, 8 %
// and 35 % slower from a cold cache.
constexpr int kRowThreads = 256;
template <int CPR>
__global__ void __launch_bounds__(kRowThreads) permute_rows_kernel(PairArgs m) {
  constexpr int RPB = kRowThreads / CPR;  // rows per block
  int i = 0;  // the pair of this block (wave-uniform)
  while (i + 1 < m.n && (int)blockIdx.z >= m.zbase[i + 1]) ++i;
  const PermuteArgs &a = m.t[i];
  const int t = blockIdx.x * RPB + threadIdx.x / CPR, c = threadIdx.x % CPR;
  if (t >= a.Sl) return;
  const int s = blockIdx.y;
  const int rh = blockIdx.z - m.zbase[i];
  const int hh = rh % a.Hl, rr = rh / a.Hl;  // wave-uniform
  const int64_t rank = a.rank0 + rr;
  const int64_t seq_off = s * a.seq_s0 + (rank * a.Hl + hh) * a.seq_s2 + t * a.seq_s1;
  const int64_t head_off = rr * a.head_s0 + hh * a.head_s1 + ((int64_t)s * a.Sl + t) * a.head_s2;
  const int64_t src_off = a.dir == 0 ? seq_off : head_off;  // elements
  const int64_t dst_off = a.dir == 0 ? head_off : seq_off;
  const u32x4 val = *(const u32x4 *)((const unsigned char *)a.src + src_off * a.elem_bytes + 16 * c);
  *(u32x4 *)((unsigned char *)a.dst + dst_off * a.elem_bytes + 16 * c) = val;
}

}  // namespace

namespace {

int launch_flat(const PermuteArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.nranks * a.Hl * a.P * a.Sl;
  const int64_t nchunks = rows * (a.row_bytes / 16);
  if (nchunks <= 0) return RA_OK;
  int64_t blocks = (nchunks + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, nchunks);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

// The row kernel serves pairs whose rows are 128, 256 or 512 bytes, all the same size.
bool rows_kernel_fits(const PermuteArgs *a, int n) {
  const int cpr = a[0].row_bytes / 16;
  if (cpr != 8 && cpr != 16 && cpr != 32) return false;
  int64_t z = 0;
  for (int i = 0; i < n; ++i) {
    if (a[i].row_bytes != a[0].row_bytes || a[i].P != a[0].P || a[i].P > 65535) return false;
    z += (int64_t)a[i].nranks * a[i].Hl;
  }
  return z <= 65535;
}

}  // namespace

int launch_ulysses_permute_n(const PermuteArgs *a, int n, hipStream_t stream) {
  // pairs with nothing to move drop out
  PairArgs m{};
  int k = 0;
  for (int i = 0; i < n; ++i)
    if ((int64_t)a[i].nranks * a[i].Hl * a[i].P * a[i].Sl > 0) m.t[k++] = a[i];
  if (k == 0) return RA_OK;
  if (!rows_kernel_fits(m.t, k)) {
    for (int i = 0; i < k; ++i) {
      const int rc = launch_flat(m.t[i], stream);
      if (rc != RA_OK) return rc;
    }
    return RA_OK;
  }
  m.n = k;
  int32_t max_sl = 0;
  m.zbase[0] = 0;
  for (int i = 0; i < k; ++i) {
    m.zbase[i + 1] = m.zbase[i] + m.t[i].nranks * m.t[i].Hl;
    max_sl = m.t[i].Sl > max_sl ? m.t[i].Sl : max_sl;
  }
  const int cpr = m.t[0].row_bytes / 16;
  const int64_t rows_per_block = kRowThreads / cpr;
  const dim3 grid((unsigned)((max_sl + rows_per_block - 1) / rows_per_block), (unsigned)m.t[0].P,
                  (unsigned)m.zbase[k]);
  if (cpr == 8)
    hipLaunchKernelGGL(permute_rows_kernel<8>, grid, dim3(kRowThreads), 0, stream, m);
  else if (cpr == 16)
    hipLaunchKernelGGL(permute_rows_kernel<16>, grid, dim3(kRowThreads), 0, stream, m);
  else
    hipLaunchKernelGGL(permute_rows_kernel<32>, grid, dim3(kRowThreads), 0, stream, m);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

int launch_ulysses_permute(const PermuteArgs &a, hipStream_t stream) {
  return launch_ulysses_permute_n(&a, 1, stream);
}

}  // namespace ra
