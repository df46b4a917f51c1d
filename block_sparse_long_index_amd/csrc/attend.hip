// Main Branch: exact softmax attention over the selected blocks, run with the
// KV block as the outer loop.
//
// The Main Branch computes ordinary exact softmax attention, restricted to
// the blocks the Index Branch selected (MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections "MiniMax MSAとは何か" and
// "2段階構造の中身").  The access order is "KV block outer, gather the
// queries that hit it": each block's K/V is read once and serves all of its
// queries (tnkblog.net MiniMax M3 MSA post, section "MSA の実装").
//
// attend_blocks_kernel: one workgroup per (block, sequence, group) item, in
// block-major launch order (early blocks, which most queries select, start
// first).  It stages K (row-major) and V (transposed) of the block in LDS
// once, then its four waves walk the item's query list in tiles of 32 MFMA
// rows = (32 / heads-per-group) queries x heads-per-group heads:
//     S^T = K * Q^T                      (bf16 MFMA, fp32; lane <-> query row)
//     mask keys after the query (only where the block is not wholly visible)
//     m = max, P = 2^(z - m), l = sum P  (z in log2 units: scale * log2(e))
//     O = P * V                          (P cast to bf16, fp32 accumulate)
// and writes the unnormalised partial (m, l, O) of every (query, head, slot).
//
// merge_partials_kernel: per (query, head) the log-sum-exp merge of its
// partials -- M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L -- which equals one softmax over the union of
// the selected keys; lse = (M + log2 L) * ln 2.
#include "msa_common.h"

namespace msa {

template <int D, int HPG>
__global__ __launch_bounds__(256) void attend_blocks_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int G, int Hq,
    int top_k, int nb_max, const int32_t* __restrict__ offsets, const int32_t* __restrict__ entries,
    int r0, int r1, float scale_log2, float* __restrict__ part_acc, float2* __restrict__ part_ml) {
  constexpr int QPT = 32 / HPG;   // queries per 32-row tile
  constexpr int KS = D / 16;      // k-steps of Q.K over the head dim
  constexpr int DT = D / 32;      // 32-wide output column tiles
  constexpr int LDK = D + 8;
  constexpr int LDV = kBlock + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LDV];
  __shared__ int range[2];

  const int BG = batch * G;
  const int beta = blockIdx.x / BG;
  const int bg = blockIdx.x % BG;
  const int b = bg / G, g = bg % G;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  if (beta * kBlock >= lk) return;
  const size_t u = (size_t)bg * nb_max + beta;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int lo = offsets[u], hi = offsets[u + 1];
    const int keys[2] = {r0 << kEntrySlotBits, r1 << kEntrySlotBits};
    int a = lo;
    for (int w = 0; w < 2; ++w) {
      int l2 = a, h2 = hi;
      while (l2 < h2) {
        int mid = (l2 + h2) >> 1;
        if (entries[mid] < keys[w]) l2 = mid + 1; else h2 = mid;
      }
      range[w] = l2;
      a = l2;
    }
  }
  __syncthreads();
  const int e0 = range[0], e1 = range[1];
  if (e0 >= e1) return;

  // stage the block: K as [key][d], V as [d][key]; keys past the sequence are zero
  const int kb = beta * kBlock;
  for (int c = tid; c < kBlock * D / 8; c += 256) {
    int key = c / (D / 8), dc = c % (D / 8);
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (kb + key < lk) {
      size_t src = ((size_t)(koff + kb + key) * G + g) * D + dc * 8;
      kv = *reinterpret_cast<const uint4*>(k + src);
      vv = *reinterpret_cast<const uint4*>(v + src);
    }
    *reinterpret_cast<uint4*>(Ks + key * LDK + dc * 8) = kv;
    const uint16_t* ve = reinterpret_cast<const uint16_t*>(&vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) Vt[(dc * 8 + i) * LDV + key] = ve[i];
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int qi = col / HPG, hl = col % HPG;
  const int ntiles = (e1 - e0 + QPT - 1) / QPT;
  const int pshift = lk - lq - qoff;   // position of global row r is r + pshift

  for (int t = wave; t < ntiles; t += 4) {
    const int e = e0 + t * QPT + qi;
    const bool valid = e < e1;
    const int ent = valid ? entries[e] : 0;
    const int r = ent >> kEntrySlotBits, slot = ent & ((1 << kEntrySlotBits) - 1);
    const bool ok = valid && r >= r0 && r < r1 && slot < top_k;
    const int p = ok ? r + pshift : 0x7fffffff;

    bf16x8 qf[KS];
    {
      const uint16_t* qs = q + ((size_t)(ok ? r : 0) * Hq + g * HPG + hl) * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (ok) x = *reinterpret_cast<const uint4*>(qs + ks * 16);
        qf[ks] = as_bf16x8(x);
      }
    }

    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (kt * 32 + col) * LDK + ks * 16 + half * 8));
        sacc[kt] = mfma32(a, qf[ks], sacc[kt]);
      }
    }

    // softmax over this block's keys for the lane's query row
    const bool partial = kb + kBlock - 1 > p;   // some keys lie after the query
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float z = sacc[kt][i] * scale_log2;
        if (partial) {
          int key = kb + kt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key > p) z = -INFINITY;
        }
        sacc[kt][i] = z;
        m = fmaxf(m, z);
      }
    m = fmaxf(m, shfl_xor_f(m, 32));
    const float msafe = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = exp2f(sacc[kt][i] - msafe);
        sacc[kt][i] = x;
        l += x;
      }
    l += shfl_xor_f(l, 32);

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint4 pk;
        pk.x = pack_bf16x2(sacc[kt][8 * s2 + 0], sacc[kt][8 * s2 + 1]);
        pk.y = pack_bf16x2(sacc[kt][8 * s2 + 2], sacc[kt][8 * s2 + 3]);
        pk.z = pack_bf16x2(sacc[kt][8 * s2 + 4], sacc[kt][8 * s2 + 5]);
        pk.w = pack_bf16x2(sacc[kt][8 * s2 + 6], sacc[kt][8 * s2 + 7]);
        const bf16x8 pa = as_bf16x8(pk);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* vr = Vt + (dt * 32 + col) * LDV + kt * 32 + 16 * s2 + 4 * half;
          uint2 lo = *reinterpret_cast<const uint2*>(vr);
          uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
          const bf16x8 vb = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          oacc[dt] = mfma32(pa, vb, oacc[dt]);
        }
      }

    // destination partial row of the lane's query row; -1 if none
    const int drow = ok ? (((r - r0) * Hq + g * HPG + hl) * top_k + slot) : -1;
    if (half == 0 && ok) part_ml[drow] = make_float2(m, l);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mrow = 8 * (i >> 2) + 4 * half + (i & 3);
      const int dm = __shfl(drow, mrow, kWave);
      if (dm >= 0) {
        float* dst = part_acc + (size_t)dm * D + col;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dst[dt * 32] = oacc[dt][i];
      }
    }
  }
}

// one wave per (query row, head)
template <int D>
__global__ __launch_bounds__(256) void merge_partials_kernel(
    const float* __restrict__ part_acc, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ sel, int r0, int r1, int Hq, int G, int top_k,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long n = (long long)(r1 - r0) * Hq;
  if (w >= n) return;
  const int lane = threadIdx.x & 63;
  const int rr = (int)(w / Hq), h = (int)(w % Hq);
  const int r = r0 + rr;
  const int g = h / (Hq / G);
  const int32_t* srow = sel + ((size_t)r * G + g) * top_k;
  int ns = 0;
  for (int s = 0; s < top_k; ++s) ns += srow[s] >= 0 ? 1 : 0;
  const size_t base = ((size_t)rr * Hq + h) * top_k;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[base + s].x);
  float L = 0.f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float2 ml = part_ml[base + s];
    const float wgt = exp2f(ml.x - M);
    L += ml.y * wgt;
    const float* src = part_acc + (base + s) * D + lane * PER;
    if constexpr (PER == 2) {
      float2 x = *reinterpret_cast<const float2*>(src);
      acc[0] += wgt * x.x;
      acc[1] += wgt * x.y;
    } else {
      acc[0] += wgt * src[0];
    }
  }
  const float inv = 1.f / L;
  uint16_t* o = out + ((size_t)r * Hq + h) * D + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    o[0] = f32_to_bf16_bits(acc[0] * inv);
  }
  if (lse && lane == 0) lse[(size_t)r * Hq + h] = (M + log2f(L)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
template <int D, int HPG>
static void launch_attend_t(const void* q, const void* k, const void* v, const int32_t* cu_q,
                            const int32_t* cu_k, int batch, int G, int Hq, int top_k, int nb_max,
                            const int32_t* offsets, const int32_t* entries, int r0, int r1,
                            float scale_log2, float* part_acc, float2* part_ml, hipStream_t st) {
  dim3 grid((unsigned)((size_t)nb_max * batch * G));
  hipLaunchKernelGGL((attend_blocks_kernel<D, HPG>), grid, dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, cu_q, cu_k, batch, G, Hq, top_k,
                     nb_max, offsets, entries, r0, r1, scale_log2, part_acc, part_ml);
}

template <int D>
static hipError_t launch_attend_d(int hpg, const void* q, const void* k, const void* v,
                                  const int32_t* cu_q, const int32_t* cu_k, int batch, int G, int Hq,
                                  int top_k, int nb_max, const int32_t* offsets,
                                  const int32_t* entries, int r0, int r1, float scale_log2,
                                  float* part_acc, float2* part_ml, hipStream_t st) {
#define MSA_ATT(H) launch_attend_t<D, H>(q, k, v, cu_q, cu_k, batch, G, Hq, top_k, nb_max, offsets, entries, r0, r1, scale_log2, part_acc, part_ml, st)
  switch (hpg) {
    case 1: MSA_ATT(1); break;
    case 2: MSA_ATT(2); break;
    case 4: MSA_ATT(4); break;
    case 8: MSA_ATT(8); break;
    case 16: MSA_ATT(16); break;
    case 32: MSA_ATT(32); break;
    default: return hipErrorInvalidValue;
  }
#undef MSA_ATT
  return hipGetLastError();
}

hipError_t launch_attend_blocks(int D, int hpg, const void* q, const void* k, const void* v,
                                const int32_t* cu_q, const int32_t* cu_k, int batch, int G, int Hq,
                                int top_k, int nb_max, const int32_t* offsets,
                                const int32_t* entries, int r0, int r1, float scale_log2,
                                float* part_acc, float2* part_ml, hipStream_t st) {
  if (D == 64)
    return launch_attend_d<64>(hpg, q, k, v, cu_q, cu_k, batch, G, Hq, top_k, nb_max, offsets,
                               entries, r0, r1, scale_log2, part_acc, part_ml, st);
  if (D == 128)
    return launch_attend_d<128>(hpg, q, k, v, cu_q, cu_k, batch, G, Hq, top_k, nb_max, offsets,
                                entries, r0, r1, scale_log2, part_acc, part_ml, st);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int D, const float* part_acc, const float2* part_ml, const int32_t* sel,
                        int r0, int r1, int Hq, int G, int top_k, void* out, float* lse,
                        hipStream_t st) {
  long long n = (long long)(r1 - r0) * Hq;
  dim3 grid((unsigned)((n + 3) / 4));
  if (D == 64)
    hipLaunchKernelGGL(merge_partials_kernel<64>, grid, dim3(256), 0, st, part_acc, part_ml, sel, r0,
                       r1, Hq, G, top_k, (uint16_t*)out, lse);
  else if (D == 128)
    hipLaunchKernelGGL(merge_partials_kernel<128>, grid, dim3(256), 0, st, part_acc, part_ml, sel, r0,
                       r1, Hq, G, top_k, (uint16_t*)out, lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace msa
