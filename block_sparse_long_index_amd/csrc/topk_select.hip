// Index Branch, step 3: top-k block selection with the forced local block.
//
// Per (query, group): the query's own block beta(p) is always selected
// (MSA guide, ai-tool-zukan.com/minimax-msa-guide, section
// "クエリを含むローカルブロックの強制取り込み"; zhaixingw.cn ai-news/10, section
// "这套注意力到底怎么省的") and counts toward top_k, so the other top_k - 1
// are the best earlier blocks by block score (section "2段階構造の中身"; the
// budget of top_k * 128 tokens in the table of section
// "ブロック単位選択の数値設計").  Equal scores: the lower block id wins.  The
// output is ascending, -1 padded; one selection per group, shared by the
// group's heads (section "GQAグループ単位の選択共有とは").
//
// Each (score, block) pair is one 64-bit key: order-preserving float bits in
// the high word, bitwise-not of the block id in the low word, so "better"
// is one unsigned compare and ties resolve to the lower id.  Each lane keeps
// a descending list of the KCAP best keys of its candidate stream in
// registers (KCAP = next power of two >= top_k - 1).  With W lanes per row
// the lanes split the row's blocks and merge their lists in top_k - 1
// max-reduction rounds.
#include "msa_common.h"

namespace msa {

__device__ inline uint64_t make_key(float s, int beta) {
  return ((uint64_t)float_order_key(s) << 32) | (uint64_t)(~(uint32_t)beta);
}
__device__ inline int key_block(uint64_t k) { return (int)(~(uint32_t)k); }
__device__ inline float key_score(uint64_t k) { return float_from_order_key((uint32_t)(k >> 32)); }

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor((uint32_t)v, mask, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Insert `key` into a descending list of N keys (0 = empty), dropping the smallest.
template <int N>
__device__ inline void list_insert(uint64_t (&list)[N], uint64_t key) {
  if (key > list[N - 1]) {
#pragma unroll
    for (int i = N - 1; i >= 0; --i) {
      uint64_t prev = (i > 0) ? list[i - 1] : ~0ull;
      bool gt_i = key > list[i];
      bool gt_prev = key > prev;
      list[i] = gt_i ? (gt_prev ? prev : key) : list[i];
    }
  }
}

// Ascending sort of N values (bitonic network, static indices).
template <int N>
__device__ inline void sort_ascending(uint64_t (&a)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        int l = i ^ j;
        if (l > i) {
          bool up = (i & k) == 0;
          uint64_t x = a[i], y = a[l];
          bool sw = up ? (x > y) : (x < y);
          a[i] = sw ? y : x;
          a[l] = sw ? x : y;
        }
      }
    }
  }
}

// grid.x covers the chunk's rows (chunk row = (query - r0) * G + g), 256 / W rows per workgroup.
template <int KCAP, int W>
__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ S, long long ld, int r0, int r1, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int G, int top_k, int32_t* __restrict__ sel,
    float* __restrict__ sel_score) {
  const int rows_per_wg = 256 / W;
  const long long crow = (long long)blockIdx.x * rows_per_wg + threadIdx.x / W;
  const int w = threadIdx.x % W;
  const long long nrows = (long long)(r1 - r0) * G;
  const bool active = crow < nrows;
  const int km = top_k - 1;

  int r = r0, g = 0, beta_p = 0;
  if (active) {
    r = r0 + (int)(crow / G);
    g = (int)(crow % G);
    RowPos rp = locate_row(r, cu_q, cu_k, batch);
    beta_p = rp.p / kBlock;
  }

  uint64_t list[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) list[i] = 0;

  if (active && km > 0) {
    const float* col = S + crow;
    int beta = w;
    // two candidates per step to overlap the loads
    for (; beta + W < beta_p; beta += 2 * W) {
      float s0 = col[(size_t)beta * ld];
      float s1 = col[(size_t)(beta + W) * ld];
      if (s0 == s0) list_insert(list, make_key(s0, beta));
      if (s1 == s1) list_insert(list, make_key(s1, beta + W));
    }
    if (beta < beta_p) {
      float s0 = col[(size_t)beta * ld];
      if (s0 == s0) list_insert(list, make_key(s0, beta));
    }
  }

  uint64_t res[KCAP];
  if constexpr (W == 1) {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) res[i] = list[i];
  } else {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      res[i] = 0;
      if (i < km) {
        uint64_t head = list[0];
        uint64_t best = head;
#pragma unroll
        for (int off = W / 2; off >= 1; off >>= 1) {
          uint64_t o = shfl_xor_u64(best, off);
          best = o > best ? o : best;
        }
        if (best != 0 && head == best) {
#pragma unroll
          for (int j = 0; j < KCAP - 1; ++j) list[j] = list[j + 1];
          list[KCAP - 1] = 0;
        }
        res[i] = best;
      }
    }
  }
  if (!active || w != 0) return;

  // keep the km best, then order them by block id: (id << 32 | score key), empty -> max
  uint64_t byid[KCAP];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    bool real = (i < km) && res[i] != 0;
    cnt += real ? 1 : 0;
    byid[i] = real ? (((uint64_t)(uint32_t)key_block(res[i]) << 32) | (res[i] >> 32)) : ~0ull;
  }
  sort_ascending(byid);

  int32_t* so = sel + ((size_t)r * G + g) * top_k;
  float* sc = sel_score ? sel_score + ((size_t)r * G + g) * top_k : nullptr;
#pragma unroll
  for (int j = 0; j < KCAP + 1; ++j) {
    if (j < top_k) {
      int id;
      float s;
      if (j < cnt) {
        uint64_t v = (j < KCAP) ? byid[j < KCAP ? j : 0] : 0;
        id = (int)(v >> 32);
        s = float_from_order_key((uint32_t)v);
      } else if (j == cnt) {
        id = beta_p;
        s = INFINITY;
      } else {
        id = -1;
        s = __uint_as_float(0x7fc00000u);
      }
      so[j] = id;
      if (sc) sc[j] = s;
    }
  }
  // top_k beyond KCAP + 1 cannot occur (KCAP >= top_k - 1)
}

template <int KCAP>
static hipError_t launch_topk_kcap(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                                   const int32_t* cu_k, int batch, int G, int top_k, bool wide,
                                   int32_t* sel, float* sel_score, hipStream_t st) {
  long long nrows = (long long)(r1 - r0) * G;
  if (wide) {
    dim3 grid((unsigned)((nrows + 3) / 4));
    hipLaunchKernelGGL((topk_select_kernel<KCAP, 64>), grid, dim3(256), 0, st, S, ld, r0, r1, cu_q,
                       cu_k, batch, G, top_k, sel, sel_score);
  } else {
    dim3 grid((unsigned)((nrows + 255) / 256));
    hipLaunchKernelGGL((topk_select_kernel<KCAP, 1>), grid, dim3(256), 0, st, S, ld, r0, r1, cu_q,
                       cu_k, batch, G, top_k, sel, sel_score);
  }
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                              const int32_t* cu_k, int batch, int G, int top_k, bool wide,
                              int32_t* sel, float* sel_score, hipStream_t st) {
  int km = top_k - 1;
  if (km <= 1) return launch_topk_kcap<1>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 2) return launch_topk_kcap<2>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 4) return launch_topk_kcap<4>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 8) return launch_topk_kcap<8>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 16) return launch_topk_kcap<16>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  return launch_topk_kcap<32>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
}

}  // namespace msa
