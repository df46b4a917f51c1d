// Internal helpers shared by the MSA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;          // KV block size B_k
constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kEntrySlotBits = 5;    // list entries pack row * 32 + slot

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row geometry of one query row: its sequence, position and key offset.
struct RowPos {
  int b;       // sequence
  int p;       // position within the sequence (queries are the last Lq of Lk)
  int koff;    // first key row of the sequence
  int lk;      // keys of the sequence
  int qoff;    // first query row of the sequence
};

// Where the key rows of a sequence live (K, V and the index keys alike).
// Contiguous: sequence b owns rows cu_k[b] .. cu_k[b+1]-1.  Paged: block beta
// of sequence b is page table[b * max_blocks + beta], i.e. rows
// 128 * page .. 128 * page + 127 of the cache.
// E8M0 exponents of a quantised Main Branch's inputs: q per (row, head) of
// E4M3 codes; k and v per (block index, KV head) of E4M3 codes, or (kv4 != 0)
// per 32 elements of every (key, KV head) row of E2M1 codes.  All null for
// bf16 inputs.
struct MainFp8 {
  const uint8_t* qe;
  const uint8_t* ke;
  const uint8_t* ve;
  int kv4;
};

struct KvMap {
  const int32_t* table;   // nullptr: contiguous rows
  int max_blocks;         // row stride of the page table
  int pages;              // pages in the cache (paged only)

  // page of block beta of sequence b, clamped into the cache so that a
  // malformed table cannot make a kernel address outside it; beta is clamped
  // into the sequence's table row for the same reason
  __device__ inline size_t page(int b, int beta) const {
    const int pg = table[(size_t)b * max_blocks + min(max(beta, 0), max_blocks - 1)];
    return (size_t)min(max(pg, 0), pages - 1);
  }
  // the same page through the scalar cache (a read-only view of the table,
  // which no kernel writes): the load is counted by lgkmcnt, so waiting for
  // it never waits for vector loads in flight (b and beta wave-uniform)
  __device__ inline size_t page_uniform(int b, int beta) const {
    typedef const __attribute__((address_space(4))) int32_t ctable_t;
    ctable_t* t = (ctable_t*)table;
    const int j = __builtin_amdgcn_readfirstlane(b * max_blocks + min(max(beta, 0), max_blocks - 1));
    const int pg = t[j];
    return (size_t)min(max(pg, 0), pages - 1);
  }
  // first row of block beta of sequence b (koff = cu_k[b])
  __device__ inline size_t block_row(int b, int koff, int beta) const {
    return table ? page(b, beta) * 128u : (size_t)koff + (size_t)beta * 128u;
  }
  // row of key position j of sequence b
  __device__ inline size_t key_row(int b, int koff, int j) const {
    return block_row(b, koff, j >> 7) + (size_t)(j & 127);
  }
  // index of block beta's per-block exponent (fp8 index keys): per page when
  // paged, else [batch][nb_max]
  __device__ inline size_t block_index(int b, int beta, int nb_max) const {
    return table ? page(b, beta) : (size_t)b * nb_max + beta;
  }
};

// Sequence that owns global query row r (binary search over cu_seqlens_q).
__device__ inline RowPos locate_row(int r, const int32_t* __restrict__ cu_q,
                                    const int32_t* __restrict__ cu_k, int batch) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= r) lo = mid; else hi = mid - 1;
  }
  RowPos rp;
  rp.b = lo;
  rp.qoff = cu_q[lo];
  int lq = cu_q[lo + 1] - rp.qoff;
  rp.koff = cu_k[lo];
  rp.lk = cu_k[lo + 1] - rp.koff;
  rp.p = rp.lk - lq + (r - rp.qoff);
  return rp;
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Output layout: lane l holds column
// (l & 31) and, in register i, row 8*(i/4) + 4*(l/32) + (i%4).  The 16-wide
// contraction is split over lane halves: half h supplies elements 8h..8h+7.
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ inline uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Pack two floats as two bf16 (RNE) in one dword: lo in bits 0..15.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Same packing through the compiler's float -> __bf16 conversion, which on
// gfx950 is one v_cvt_pk_bf16_f32 per pair (round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack2_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Pack two floats as two fp16 (round to nearest even) in one dword: lo in bits 0..15.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack2_f16(float lo, float hi) {
  f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline float2 unpack2_f16(uint32_t w) {
  const f16x2_t v = __builtin_bit_cast(f16x2_t, w);
  return make_float2((float)v[0], (float)v[1]);
}
__device__ inline float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ inline uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float float_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ inline float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Block maxima of a lane's own row from per-lane partial maxima over the keys
// of its lane half (S^T layout: lane l and lane l ^ 32 hold the same query
// column, each for half of the keys).  RT == 2: half h owns row tile h, so
// one v_permlane32_swap hands each half the other half's partial of the tile
// it owns (lanes 0-31 receive rmax[0] of lanes 32-63, lanes 32-63 receive
// rmax[1] of lanes 0-31).  RT == 1: both halves own row tile 0.
template <int RT>
__device__ inline float row_tile_max(const float (&rmax)[RT], int half) {
  if constexpr (RT == 2) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax[0]),
                                                    __float_as_uint(rmax[1]), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    (void)half;
    return fmaxf(rmax[0], shfl_xor_f(rmax[0], 32));
  }
}

// v_permlane32_swap of x and y: x's lanes 32-63 trade places with y's lanes
// 0-31.  So lanes 0-31 receive x of lanes 32-63 (in .y) and lanes 32-63
// receive y of lanes 0-31 (in .x); the other halves keep their own values.
__device__ inline uint2 permlane32_swap_u32(uint32_t x, uint32_t y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  return make_uint2(r[0], r[1]);
}

// ds_read_b64_tr_b16 at an LDS byte address: the four 16-bit values this lane
// receives, as two dwords.  Within each 16 lanes, lane 4a + c receives element
// c of the 8-byte pieces addressed by lanes a, a + 4, a + 8, a + 12 (measured):
// if lane m addresses row k0 + m/4 at column d0 + 4 (m%4) of a row-major bf16
// tile, lane n receives rows k0 .. k0+3 of column d0 + n.
typedef short lds_tr_v4s __attribute__((ext_vector_type(4)));
__device__ inline uint2 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) lds_tr_v4s lds_v4s;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p));
}

// one 16-byte direct global->LDS load per lane; lane L writes lds_base + 16 L
// (lds_base wave-uniform)
__device__ inline void lds_load16(const uint8_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}
// the same with N = 1, 2 or 4 bytes per lane: lane L's N bytes land at
// lds_base + 4 L whatever N is
template <int N>
__device__ inline void lds_load_n(const uint8_t* src, uint8_t* lds_base) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 bytes per lane");
  if constexpr (N == 4) __builtin_amdgcn_global_load_lds(src, lds_base, 4, 0, 0);
  else if constexpr (N == 2) __builtin_amdgcn_global_load_lds(src, lds_base, 2, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, lds_base, 1, 0, 0);
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "small counts only");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace msa
