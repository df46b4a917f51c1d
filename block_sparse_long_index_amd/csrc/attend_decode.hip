// Main Branch for decode-shaped passes (a few new tokens per sequence).
//
// Same computation and the same partial format as attend_blocks_kernel (exact
// softmax over each selected block's visible keys; MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections "MiniMax MSAとは何か" and
// "2段階構造の中身"), but with one query per (sequence, group) a KV block is hit
// by that query alone, so "KV block outer, gather the queries that hit it"
// (tnkblog.net MiniMax M3 MSA post, section "MSA の実装") needs no list: each
// wave takes one (query, selected slot) straight from the selection and reads
// that block once.  Two kernels: bf16 inputs stage the block in LDS with
// whole-row loads (attend_decode_lds_kernel, one workgroup per item); 8-bit
// inputs (E4M3 codes with power-of-two scales), dequantised exactly into bf16
// operands while loading, take attend_decode_kernel, one wave per item: K from
// global memory straight into MFMA A fragments, V transposed through a
// per-wave LDS tile for O^T = V^T * P^T.  The query's HPG heads are MFMA
// columns (HPG <= 32).
#include "fp8_common.h"
#include "msa_common.h"

namespace msa {

constexpr int kDecodeWaves = 4;

template <int D, int HPG, bool Q8>
__global__ __launch_bounds__(kDecodeWaves * 64) void attend_decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint8_t* __restrict__ qe, const uint8_t* __restrict__ ke, const uint8_t* __restrict__ ve,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch, int G,
    int Hq, int top_k, int nb_max, const int32_t* __restrict__ sel, int r0, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml) {
  constexpr int KS = D / 16;      // k-steps of Q.K over the head dim
  constexpr int DT = D / 32;      // 32-row tiles of O^T
  constexpr int LDV = kBlock + 4; // 66-dword rows: 8-byte reads of 16 rows hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t Vt_all[kDecodeWaves][D * LDV];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  uint16_t* Vt = Vt_all[wave];
  const int r = r0 + (int)blockIdx.x;
  const int g = (int)blockIdx.z;
  const int slot = (int)blockIdx.y * kDecodeWaves + wave;

  // every wave runs to the end (no early exit), only the useful ones store
  const RowPos rp = locate_row(r, cu_q, cu_k, batch);
  int beta = -1;
  if (slot < top_k) beta = sel[((size_t)r * G + g) * top_k + slot];
  const int kb = beta * kBlock;
  const bool active = beta >= 0 && kb < rp.lk;
  const int kb_safe = active ? kb : 0;
  const size_t row0 = kv.block_row(rp.b, rp.koff, kb_safe >> 7);   // first cache row of the block

  // exponents of the block (8-bit inputs)
  int kexp = 0, vexp = 0;
  if constexpr (Q8) {
    const size_t xi = kv.block_index(rp.b, kb_safe >> 7, nb_max) * G + g;
    kexp = (int)ke[xi] - 127;
    vexp = (int)ve[xi] - 127;
  }

  // V^T of the block into this wave's LDS tile (keys past the sequence are zero)
  if constexpr (Q8) {
    for (int c = lane; c < kBlock * D / 16; c += 64) {
      const int key = c % kBlock, dc = c / kBlock;
      const bool in = active && kb_safe + key < rp.lk;
      const size_t row = (row0 + (in ? key : 0)) * G + g;
      uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(v) + row * D + dc * 16);
      vv = in ? vv : make_uint4(0, 0, 0, 0);
      const uint4 lo = dequant8_bf16(make_uint2(vv.x, vv.y), vexp);
      const uint4 hi = dequant8_bf16(make_uint2(vv.z, vv.w), vexp);
      const uint32_t vw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        Vt[(dc * 16 + i) * LDV + key] = (uint16_t)(vw[i >> 1] >> (16 * (i & 1)));
    }
  } else {
    for (int c = lane; c < kBlock * D / 8; c += 64) {
      const int key = c % kBlock, dc = c / kBlock;
      const bool in = active && kb_safe + key < rp.lk;
      const size_t row = (row0 + (in ? key : 0)) * G + g;
      uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(v) + row * D + dc * 8);
      vv = in ? vv : make_uint4(0, 0, 0, 0);
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        Vt[(dc * 8 + i) * LDV + key] = (uint16_t)(vw[i >> 1] >> (16 * (i & 1)));
    }
  }

  // Q^T fragments: MFMA column n = head (col) of query r; columns >= HPG are zero
  bf16x8 qf[KS];
  {
    const int hl = col < HPG ? col : 0;
    const size_t qrow = (size_t)r * Hq + g * HPG + hl;
    if constexpr (Q8) {
      const uint8_t* qs = static_cast<const uint8_t*>(q) + qrow * D + half * 8;
      const int e = (int)qe[qrow] - 127;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint2 x = *reinterpret_cast<const uint2*>(qs + ks * 16);
        qf[ks] = as_bf16x8(dequant8_bf16(col < HPG ? x : make_uint2(0, 0), e));
      }
    } else {
      const uint16_t* qs = static_cast<const uint16_t*>(q) + qrow * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 x = *reinterpret_cast<const uint4*>(qs + ks * 16);
        qf[ks] = as_bf16x8(x);   // columns >= HPG repeat head 0: never stored
      }
    }
  }

  // S^T = K * Q^T with K fragments read straight from global memory
  f32x16 sacc[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = kb_safe + kt * 32 + col;
    const bool in = active && key < rp.lk;
    const size_t krow = (row0 + (in ? key - kb_safe : 0)) * G + g;
    bf16x8 a[KS];
    if constexpr (Q8) {
      const uint8_t* ks_ptr = static_cast<const uint8_t*>(k) + krow * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint2 x = *reinterpret_cast<const uint2*>(ks_ptr + ks * 16);
        a[ks] = as_bf16x8(dequant8_bf16(in ? x : make_uint2(0, 0), kexp));
      }
    } else {
      const uint16_t* ks_ptr = static_cast<const uint16_t*>(k) + krow * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 x = *reinterpret_cast<const uint4*>(ks_ptr + ks * 16);
        a[ks] = as_bf16x8(in ? x : make_uint4(0, 0, 0, 0));
      }
    }
    sacc[kt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc[kt] = mfma32(a[ks], qf[ks], sacc[kt]);
  }

  // mask keys after the query (and past the sequence), softmax in log2 units
  const int pr = rp.p - kb_safe - 4 * half;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kt * 32 + 8 * (i >> 2) + (i & 3) > pr) sacc[kt][i] = -INFINITY;
  float mr = sacc[0][0];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mr = fmaxf(mr, sacc[kt][i]);
  mr = fmaxf(mr, shfl_xor_f(mr, 32));
  const float m = mr * scale_log2;
  const float nm = (mr == -INFINITY) ? 0.f : -m;
  float l = 0.f;
  uint4 pk[8];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * s2 + e], scale_log2, nm));
        l += x[e];
      }
      pk[2 * kt + s2] = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                                   pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7]));
    }
  l += shfl_xor_f(l, 32);

  // the wave's own V^T tile was written by this wave: wait for its LDS stores
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();

  // O^T = V^T * P^T: lane <-> head row, register i <-> d = 32dt + 8(i/4) + 4half + i%4
  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 pb = as_bf16x8(pk[ks]);
    const int kt = ks >> 1, s2 = ks & 1;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vr = Vt + (dt * 32 + col) * LDV + kt * 32 + 16 * s2 + 4 * half;
      uint2 lo = *reinterpret_cast<const uint2*>(vr);
      uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
      oacc[dt] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, oacc[dt]);
    }
  }

  if (active && col < HPG) {
    const int drow = (((r - r0) * G + g) * top_k + slot) * HPG + col;
    part_ml[drow] = make_float2(m, l);
    float* dst = part_acc + (size_t)drow * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(dst + dt * 32 + 8 * j) =
            make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs: the selected block staged in LDS.  One workgroup (4 waves) per
// (group, slot, query), groups fastest.  Fragment loads straight from global
// memory touch 32 key rows per instruction; here every load instruction reads
// whole rows (1 KiB of consecutive row bytes per wave).  K reaches LDS by
// direct global->LDS 16-byte loads; V is loaded into registers at the same
// time and written over K once the scores are done, so waiting for K never
// waits for V (the compiler cannot tell two direct-to-LDS streams apart), and
// the block needs 32 KiB of LDS.  Chunk positions are XOR-swizzled: K so that
// an A-fragment read (16 consecutive rows, one 16-byte chunk each) hits 16
// bank groups; V so that the transposed reads (ds_read_b64_tr_b16: within 16
// lanes, lane 4a + c receives element c of the 8-byte pieces addressed by
// lanes a, a + 4, a + 8, a + 12) of 4 rows x 4 chunks hit 16 bank groups.
// Those transposed reads give each lane four consecutive keys of one column:
// the V^T A fragment without a transposing store.  Wave w scores key tile w;
// the softmax maximum and sum combine through LDS; every key tile's bf16 P goes
// through LDS, and wave w then forms output columns 32w .. 32w + 31 (D = 64:
// waves 0 and 1).  Barriers are bare (s_barrier after lgkmcnt(0)): a
// workgroup fence would also wait for the loads still in flight.
// ---------------------------------------------------------------------------
typedef short lds_tr_v4s __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at an LDS byte address: the four 16-bit values this lane
// receives, as two dwords
__device__ inline uint2 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) lds_tr_v4s lds_v4s;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p));
}

// one 16-byte direct global->LDS load per lane; lane L writes lds_base + 16 L
__device__ inline void lds_load16(const uint16_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

template <int D, int HPG>
__global__ __launch_bounds__(256) void attend_decode_lds_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch, int G,
    int Hq, int top_k, const int32_t* __restrict__ sel, int r0, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml) {
  constexpr int RB = D * 2;                     // bytes per key row
  constexpr int CPR = RB / 16;                  // 16-byte chunks per row
  constexpr int R = 256 / RB;                   // rows per 256-byte bank line
  constexpr int ROWS_PER_PIECE = 1024 / RB;     // rows per wave load instruction
  constexpr int PER_WAVE = kBlock / ROWS_PER_PIECE / 4;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kBlock * RB];   // K, then V
  uint8_t* const Vs = Ks;
  __shared__ __attribute__((aligned(16))) uint4 Pl[4][2][64];
  __shared__ float red_m[4][32], red_l[4][32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int r = r0 + (int)blockIdx.z, slot = (int)blockIdx.y, g = (int)blockIdx.x;
  const RowPos rp = locate_row(r, cu_q, cu_k, batch);
  const int beta = sel[((size_t)r * G + g) * top_k + slot];
  if (beta < 0 || beta * kBlock >= rp.lk) return;   // the same for the whole workgroup
  const int kb = beta * kBlock;
  const int nvalid = min(kBlock, rp.lk - kb);       // rows of the block in the sequence
  const size_t row0 = kv.block_row(rp.b, rp.koff, beta);

  // Q^T fragments: MFMA column n = head n of the query's group; columns >= HPG are zero
  bf16x8 qf[KS];
  {
    const int hl = col < HPG ? col : 0;
    const uint16_t* qs = q + ((size_t)r * Hq + g * HPG + hl) * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = *reinterpret_cast<const uint4*>(qs + ks * 16);
      qf[ks] = as_bf16x8(x);   // columns >= HPG repeat head 0: never stored
    }
  }
  auto swz_k = [](int m) { return (m / R) % CPR; };
  auto swz_v = [](int m) { return 4 * ((m / R) % (CPR / 4)); };
  // this wave's pieces of K and V; rows past the sequence read its last row
  // (masked below, so they only need to be finite)
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int piece = wave * PER_WAVE + i;
    const int m = piece * ROWS_PER_PIECE + lane / CPR;
    const size_t src = ((row0 + min(m, nvalid - 1)) * G + g) * D;
    lds_load16(k + src + ((lane % CPR) ^ swz_k(m)) * 8, Ks + piece * 1024);
  }
  // V into registers (the same coalesced pieces), written to LDS over K once
  // the scores are done
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u vreg[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int piece = wave * PER_WAVE + i;
    const int m = piece * ROWS_PER_PIECE + lane / CPR;
    const size_t src = ((row0 + min(m, nvalid - 1)) * G + g) * D;
    vreg[i] = *reinterpret_cast<const v4u*>(v + src + (lane % CPR) * 8);
  }

  wait_vmcnt<PER_WAVE>();   // this wave's K pieces (its V pieces may still be in flight)
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // S^T = K * Q^T for keys 32 wave .. 32 wave + 31
  f32x16 sacc = f32x16{};
  {
    const int m = wave * 32 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(Ks + m * RB + (((2 * ks + half) ^ swz_k(m)) * 16));
      sacc = mfma32(as_bf16x8(a), qf[ks], sacc);
    }
  }
  // mask keys after the query, then the block maximum over the four waves
  const int pr = rp.p - kb - wave * 32 - 4 * half;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (8 * (i >> 2) + (i & 3) > pr) sacc[i] = -INFINITY;
  float mr = sacc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mr = fmaxf(mr, sacc[i]);
  mr = fmaxf(mr, shfl_xor_f(mr, 32));
  if (half == 0) red_m[wave][col] = mr;
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  mr = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
  const float m = mr * scale_log2;
  const float nm = (mr == -INFINITY) ? 0.f : -m;
  float l = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = __builtin_amdgcn_exp2f(fmaf(sacc[8 * s2 + e], scale_log2, nm));
      l += x[e];
    }
    Pl[wave][s2][lane] = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                                    pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7]));
  }
  l += shfl_xor_f(l, 32);
  if (half == 0) red_l[wave][col] = l;
  // every wave's K reads ended at the barrier above: V replaces K
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int piece = wave * PER_WAVE + i;
    const int m = piece * ROWS_PER_PIECE + lane / CPR;
    *reinterpret_cast<v4u*>(Vs + m * RB + (((lane % CPR) ^ swz_v(m)) * 16)) = vreg[i];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses are done
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (wave >= DT) return;

  // O^T = V^T * P^T for output columns 32 wave .. 32 wave + 31: lane <-> head,
  // register i <-> column 32 wave + 8(i/4) + 4 half + i%4
  f32x16 oacc = f32x16{};
  {
    const int grp = lane >> 4, mm = lane & 15;
    const int d0 = wave * 32 + 16 * (grp & 1);              // this 16-lane group's columns
    const int cb = (2 * d0 + 8 * (mm & 3)) >> 4;             // logical chunk of lane mm's piece
    const int cofs = 8 * (mm & 1);                           // byte offset inside the chunk
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kb1 = kt * 32 + 16 * s2 + 4 * (grp >> 1) + (mm >> 2);   // row this lane addresses
        const int kb2 = kb1 + 8;
        const uint2 lw = lds_read_tr16(Vs + kb1 * RB + ((cb ^ swz_v(kb1)) * 16) + cofs);
        const uint2 hw = lds_read_tr16(Vs + kb2 * RB + ((cb ^ swz_v(kb2)) * 16) + cofs);
        oacc = mfma32(as_bf16x8(make_uint4(lw.x, lw.y, hw.x, hw.y)), as_bf16x8(Pl[kt][s2][lane]), oacc);
      }
  }
  if (col < HPG) {
    const int drow = (((r - r0) * G + g) * top_k + slot) * HPG + col;
    if (wave == 0 && half == 0)
      part_ml[drow] = make_float2(m, red_l[0][col] + red_l[1][col] + red_l[2][col] + red_l[3][col]);
    float* dst = part_acc + (size_t)drow * D + wave * 32 + 4 * half;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(dst + 8 * j) =
          make_float4(oacc[4 * j], oacc[4 * j + 1], oacc[4 * j + 2], oacc[4 * j + 3]);
  }
}

template <int D, int HPG>
static void launch_decode_t(const void* q, const void* k, const void* v, MainFp8 f8,
                            const int32_t* cu_q, const int32_t* cu_k, KvMap kv, int batch, int G,
                            int Hq, int top_k, int nb_max, const int32_t* sel, int r0, int r1,
                            float scale_log2, float* part_acc, float2* part_ml, hipStream_t st) {
  if (!f8.qe && HPG <= 32) {
    hipLaunchKernelGGL((attend_decode_lds_kernel<D, HPG>), dim3(G, top_k, r1 - r0), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, cu_q, cu_k, kv,
                       batch, G, Hq, top_k, sel, r0, scale_log2, part_acc, part_ml);
    return;
  }
  dim3 grid(r1 - r0, (top_k + kDecodeWaves - 1) / kDecodeWaves, G);
  if (f8.qe)
    hipLaunchKernelGGL((attend_decode_kernel<D, HPG, true>), grid, dim3(kDecodeWaves * 64), 0, st, q,
                       k, v, f8.qe, f8.ke, f8.ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel,
                       r0, scale_log2, part_acc, part_ml);
  else
    hipLaunchKernelGGL((attend_decode_kernel<D, HPG, false>), grid, dim3(kDecodeWaves * 64), 0, st,
                       q, k, v, (const uint8_t*)nullptr, (const uint8_t*)nullptr,
                       (const uint8_t*)nullptr, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel, r0,
                       scale_log2, part_acc, part_ml);
}

template <int D>
static hipError_t launch_decode_d(int hpg, const void* q, const void* k, const void* v, MainFp8 f8,
                                  const int32_t* cu_q, const int32_t* cu_k, KvMap kv, int batch,
                                  int G, int Hq, int top_k, int nb_max, const int32_t* sel, int r0,
                                  int r1, float scale_log2, float* part_acc, float2* part_ml,
                                  hipStream_t st) {
#define MSA_DEC(H) launch_decode_t<D, H>(q, k, v, f8, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel, r0, r1, scale_log2, part_acc, part_ml, st)
  switch (hpg) {
    case 1: MSA_DEC(1); break;
    case 2: MSA_DEC(2); break;
    case 4: MSA_DEC(4); break;
    case 8: MSA_DEC(8); break;
    case 16: MSA_DEC(16); break;
    case 32: MSA_DEC(32); break;
    default: return hipErrorInvalidValue;
  }
#undef MSA_DEC
  return hipGetLastError();
}

hipError_t launch_attend_decode(int D, int hpg, const void* q, const void* k, const void* v,
                                MainFp8 f8, const int32_t* cu_q, const int32_t* cu_k, KvMap kv,
                                int batch, int G, int Hq, int top_k, int nb_max, const int32_t* sel,
                                int r0, int r1, float scale_log2, float* part_acc, float2* part_ml,
                                hipStream_t st) {
  if (D == 64)
    return launch_decode_d<64>(hpg, q, k, v, f8, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel,
                               r0, r1, scale_log2, part_acc, part_ml, st);
  if (D == 128)
    return launch_decode_d<128>(hpg, q, k, v, f8, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel,
                                r0, r1, scale_log2, part_acc, part_ml, st);
  return hipErrorInvalidValue;
}

}  // namespace msa
