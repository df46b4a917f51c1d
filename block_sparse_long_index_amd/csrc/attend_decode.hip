// Main Branch for decode-shaped passes (a few new tokens per sequence).
//
// Same computation and the same partial format as attend_blocks_kernel (exact
// softmax over each selected block's visible keys; MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections "MiniMax MSAとは何か" and
// "2段階構造の中身"), but with one query per (sequence, group) a KV block is hit
// by that query alone, so "KV block outer, gather the queries that hit it"
// (tnkblog.net MiniMax M3 MSA post, section "MSA の実装") needs no list: each
// wave takes one (query, selected slot) straight from the selection and reads
// that block once.  K goes from global memory straight into MFMA A
// fragments; V is transposed through a per-wave LDS tile for O^T = V^T * P^T.
// The tile holds the query's HPG heads as MFMA rows (HPG <= 32).  Q8: 8-bit
// inputs (E4M3 codes with power-of-two scales), dequantised exactly into the
// same bf16 operands while loading.
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
        qf[ks] = as_bf16x8(col < HPG ? x : make_uint4(0, 0, 0, 0));
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

template <int D, int HPG>
static void launch_decode_t(const void* q, const void* k, const void* v, MainFp8 f8,
                            const int32_t* cu_q, const int32_t* cu_k, KvMap kv, int batch, int G,
                            int Hq, int top_k, int nb_max, const int32_t* sel, int r0, int r1,
                            float scale_log2, float* part_acc, float2* part_ml, hipStream_t st) {
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
