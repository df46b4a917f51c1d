// Top-k helpers shared by the selection kernels.
//
// A (block score, block id) pair is one 64-bit key: order-preserving float
// bits in the high word and the bitwise-not of the block id in the low word,
// so "better" is one unsigned compare and equal scores rank the lower block
// id first.  Key 0 marks an empty slot.
#pragma once

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

// Running top list of one row whose candidate blocks arrive in increasing id
// order (the prefill kernels scan blocks 0, 1, 2, ...).  Then every listed id
// is smaller than a newcomer's, so under "equal scores: lower id first" a
// newcomer outranks an entry exactly when its score is strictly larger: the
// list keeps 32-bit order keys of the scores (descending, 0 = empty) beside
// the ids, and an insert is one 32-bit median per slot for the keys plus a
// compare and two selects per slot for the ids.
template <int N>
struct OrderedTopList {
  uint32_t key[N];
  int32_t id[N];

  __device__ inline void clear() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      key[i] = 0;
      id[i] = 0;
    }
  }
  // k = float_order_key(score) of block beta (> every listed id); k == 0 is a no-op
  __device__ inline void insert(uint32_t k, int beta) {
    if (k > key[N - 1]) {
      bool gt[N];
#pragma unroll
      for (int i = 0; i < N; ++i) gt[i] = k > key[i];
#pragma unroll
      for (int i = N - 1; i >= 1; --i) {
        id[i] = gt[i - 1] ? id[i - 1] : (gt[i] ? beta : id[i]);
        // the median of key[i-1] >= key[i] and k, written as the general median
        // so that it becomes one v_med3_u32
        key[i] = max(min(key[i - 1], key[i]), min(max(key[i - 1], key[i]), k));
      }
      id[0] = gt[0] ? beta : id[0];
      key[0] = max(key[0], k);
    }
  }
  // the same list as 64-bit keys (order key << 32 | ~id; 0 = empty)
  __device__ inline void to_keys(uint64_t (&out)[N]) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      out[i] = key[i] ? (((uint64_t)key[i] << 32) | (uint64_t)(~(uint32_t)id[i])) : 0ull;
  }
};

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

// Write one (query, group) selection: the km best earlier blocks of the
// descending key list `res` (first km entries) in ascending block order, then
// the local block beta_p, then -1 padding up to top_k.  sel_score (optional)
// gets each block's score, +inf for the local block and NaN for padding.
template <int KCAP>
__device__ inline void write_selection(const uint64_t (&res)[KCAP], int km, int beta_p, int top_k,
                                       int32_t* __restrict__ so, float* __restrict__ sc) {
  uint64_t byid[KCAP];   // (id << 32 | score key), empty -> max
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    bool real = (i < km) && res[i] != 0;
    cnt += real ? 1 : 0;
    byid[i] = real ? (((uint64_t)(uint32_t)key_block(res[i]) << 32) | (res[i] >> 32)) : ~0ull;
  }
  sort_ascending(byid);
#pragma unroll
  for (int j = 0; j < KCAP + 1; ++j) {   // top_k <= KCAP + 1
    if (j < top_k) {
      int id;
      float s;
      if (j < cnt) {
        const uint64_t v = byid[j < KCAP ? j : KCAP - 1];
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
}

}  // namespace msa
