// KV-block-outer regrouping of the selection: per (sequence, group, block)
// the list of queries that selected the block.
//
// The Main Branch runs with the KV block as the outer loop, gathering the
// queries that hit each block, so every block is read once (tnkblog.net
// MiniMax M3 MSA post, section "MSA の実装"; wiki repost of the CSDN article,
// section "MiniMax Sparse Attention（MSA）", item 3).  This file builds those
// lists as a stable counting sort of the selection by bucket
// u = (b * G + g) * nb_max + beta:
//
//   1. count:   per (sequence, 128-query tile, group) an LDS histogram over
//               blocks, written as one row of a dense count matrix;
//   2. colscan: exclusive prefix of every bucket's column over the tiles of
//               its sequence, plus the bucket total;
//   3. scan:    exclusive prefix of the bucket totals -> CSR offsets
//               (three-kernel reduce / scan / add);
//   4. scatter: per (sequence, tile, group) one wave walks its rows in
//               ascending order and places (row * 32 + slot) at the running
//               position of each block, so every list is ascending in row.
#include "msa_common.h"

namespace msa {

constexpr int kListTile = 128;   // query rows per counting tile

// grid: x = (sequence, group), y = 128-query tile
__global__ __launch_bounds__(256) void lists_count_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cu_q, int G, int top_k,
    int nqt_max, int nb_max, int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];
  const int t = blockIdx.y;
  const int b = blockIdx.x / G;
  const int g = blockIdx.x % G;
  for (int i = threadIdx.x; i < nb_max; i += 256) hist[i] = 0;
  __syncthreads();
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int ra = qoff + t * kListTile;
  const int rz = min(qoff + lq, ra + kListTile);
  const int n = max(0, rz - ra) * top_k;
  for (int e = threadIdx.x; e < n; e += 256) {
    int row = ra + e / top_k, s = e % top_k;
    int beta = sel[((size_t)row * G + g) * top_k + s];
    if (beta >= 0 && beta < nb_max) atomicAdd(&hist[beta], 1);
  }
  __syncthreads();
  int32_t* out = cnt + (((size_t)b * nqt_max + t) * G + g) * nb_max;
  for (int i = threadIdx.x; i < nb_max; i += 256) out[i] = hist[i];
}

// one thread per bucket column; cnt rows are (b, t, g), columns beta
__global__ __launch_bounds__(256) void lists_colscan_kernel(int32_t* __restrict__ cnt, int batch,
                                                            int G, int nqt_max, int nb_max,
                                                            int32_t* __restrict__ tot) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long ncol = (long long)batch * G * nb_max;
  if (c >= ncol) return;
  const long long gnb = (long long)G * nb_max;
  const long long b = c / gnb, rem = c % gnb;
  int32_t* base = cnt + (size_t)b * nqt_max * gnb + rem;
  int run = 0;
  int t = 0;
  for (; t + 8 <= nqt_max; t += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = base[(size_t)(t + i) * gnb];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      base[(size_t)(t + i) * gnb] = run;
      run += v[i];
    }
  }
  for (; t < nqt_max; ++t) {
    int v = base[(size_t)t * gnb];
    base[(size_t)t * gnb] = run;
    run += v;
  }
  tot[c] = run;
}

// --- exclusive scan of n int32 values into out[0..n] (out[n] = total) -------
constexpr int kScanItems = 1024;   // per workgroup: 256 threads x 4

__device__ inline int block_exclusive_scan_256(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int x = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  int incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void scan_reduce_kernel(const int32_t* __restrict__ in, long long n,
                                                          int32_t* __restrict__ part) {
  __shared__ int sh[256];
  const long long base = (long long)blockIdx.x * kScanItems + threadIdx.x * 4;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (base + i < n) s += in[base + i];
  int total;
  block_exclusive_scan_256(s, sh, &total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// single workgroup: exclusive scan of nparts partial sums in place; writes the total to *total_out
__global__ __launch_bounds__(256) void scan_top_kernel(int32_t* __restrict__ part, int nparts,
                                                       int32_t* __restrict__ total_out) {
  __shared__ int sh[256];
  int carry = 0;
  for (int base = 0; base < nparts; base += 256) {
    int i = base + threadIdx.x;
    int v = i < nparts ? part[i] : 0;
    int total;
    int ex = block_exclusive_scan_256(v, sh, &total);
    if (i < nparts) part[i] = ex + carry;
    carry += total;
  }
  if (threadIdx.x == 0) *total_out = carry;
}

__global__ __launch_bounds__(256) void scan_add_kernel(const int32_t* __restrict__ in, long long n,
                                                       const int32_t* __restrict__ part,
                                                       int32_t* __restrict__ out) {
  __shared__ int sh[256];
  const long long base = (long long)blockIdx.x * kScanItems + threadIdx.x * 4;
  int v[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (base + i < n) ? in[base + i] : 0;
    s += v[i];
  }
  int total;
  int ex = block_exclusive_scan_256(s, sh, &total) + part[blockIdx.x];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (base + i < n) out[base + i] = ex;
    ex += v[i];
  }
}

// one wave per (sequence, tile, group); grid as lists_count_kernel
__global__ __launch_bounds__(64) void lists_scatter_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int G, int top_k, int nqt_max, int nb_max,
    const int32_t* __restrict__ cnt_prefix, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ entries) {
  extern __shared__ int smem[];
  int* run = smem;                    // nb_max
  int* sl = smem + nb_max;            // kListTile * top_k
  const int t = blockIdx.y;
  const int b = blockIdx.x / G;
  const int g = blockIdx.x % G;
  const int lane = threadIdx.x;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int lk = cu_k[b + 1] - cu_k[b];
  const int ra = qoff + t * kListTile;
  const int rz = min(qoff + lq, ra + kListTile);
  if (ra >= rz) return;
  // blocks any row of this tile can select: 0 .. beta(p of the last row)
  const int p_last = lk - lq + (rz - 1 - qoff);
  const int nbt = min(nb_max, max(0, p_last / kBlock + 1));
  const int32_t* pre = cnt_prefix + (((size_t)b * nqt_max + t) * G + g) * nb_max;
  const int32_t* off = offsets + ((size_t)b * G + g) * nb_max;
  const int n = (rz - ra) * top_k;
  for (int e = lane; e < n; e += 64) {
    int row = ra + e / top_k, s = e % top_k;
    sl[e] = sel[((size_t)row * G + g) * top_k + s];
  }
  // each block's first position: for all blocks the tile can select when they
  // are fewer than its selections, else only for the selected ones (a long
  // context's late tiles can select thousands of blocks but hold at most
  // kListTile * top_k selections); lanes that share a block write the same value
  if (nbt <= n) {
    for (int i = lane; i < nbt; i += 64) run[i] = off[i] + pre[i];
  } else {
    __syncthreads();
    for (int e = lane; e < n; e += 64) {
      const int beta = sl[e];
      if (beta >= 0 && beta < nbt) run[beta] = off[beta] + pre[beta];
    }
  }
  __syncthreads();
  for (int i = 0; i < rz - ra; ++i) {
    if (lane < top_k) {
      int beta = sl[i * top_k + lane];
      if (beta >= 0 && beta < nbt) {
        int pos = run[beta];
        run[beta] = pos + 1;
        entries[pos] = ((ra + i) << kEntrySlotBits) | lane;
      }
    }
  }
}

// ---------------------------------------------------------------------------
size_t lists_workspace_bytes(int batch, int G, int nqt_max, int nb_max) {
  size_t U = (size_t)batch * G * nb_max;
  size_t cnt = (size_t)batch * nqt_max * G * nb_max * sizeof(int32_t);
  size_t nparts = (U + kScanItems - 1) / kScanItems;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(cnt) + al(U * sizeof(int32_t)) + al((nparts + 1) * sizeof(int32_t));
}

int list_tile_rows() { return kListTile; }

hipError_t launch_build_lists(const int32_t* sel, const int32_t* cu_q, const int32_t* cu_k,
                              int batch, int G, int top_k, int nqt_max, int nb_max,
                              int32_t* offsets, int32_t* entries, void* ws, hipStream_t st) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t U = (size_t)batch * G * nb_max;
  char* p = (char*)ws;
  int32_t* cnt = (int32_t*)p;
  p += al((size_t)batch * nqt_max * G * nb_max * sizeof(int32_t));
  int32_t* tot = (int32_t*)p;
  p += al(U * sizeof(int32_t));
  int32_t* part = (int32_t*)p;
  size_t nparts = (U + kScanItems - 1) / kScanItems;

  // zero-size grids are skipped (no queries, or no blocks).  (sequence, group)
  // pairs run along x, which holds any count the host accepts; query tiles
  // along y (at most the per-sequence block limit of the LDS lists)
  dim3 g1((unsigned)(batch * G), nqt_max);
  if (nqt_max > 0 && U > 0)
    hipLaunchKernelGGL(lists_count_kernel, g1, dim3(256), nb_max * sizeof(int), st, sel, cu_q, G,
                       top_k, nqt_max, nb_max, cnt);
  if (U > 0) {
    dim3 g2((unsigned)((U + 255) / 256));
    hipLaunchKernelGGL(lists_colscan_kernel, g2, dim3(256), 0, st, cnt, batch, G, nqt_max, nb_max, tot);
    hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)nparts), dim3(256), 0, st, tot, (long long)U, part);
  }
  hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(256), 0, st, part, (int)nparts, offsets + U);
  if (U > 0)
    hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)nparts), dim3(256), 0, st, tot, (long long)U,
                       part, offsets);
  size_t lds = (size_t)(nb_max + kListTile * top_k) * sizeof(int);
  if (nqt_max > 0 && U > 0)
    hipLaunchKernelGGL(lists_scatter_kernel, g1, dim3(64), lds, st, sel, cu_q, cu_k, G, top_k,
                       nqt_max, nb_max, cnt, offsets, entries);
  return hipGetLastError();
}

}  // namespace msa
