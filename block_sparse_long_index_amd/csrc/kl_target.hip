// KL-alignment target of the Index Branch, forward only.
//
// The Index Branch is trained by pulling the distribution of its block scores
// towards the distribution of the blocks the Main Branch's exact attention
// relied on, through a KL divergence (MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections
// "非微分的な選択をどう学習させるか（KLダイバージェンス）" and "選択を学習可能にするKL損失").
// Computed here, per (query, group), over the selected blocks:
//   P(s)  = attention mass of the Main Branch on selected slot s, averaged over
//           the group's heads: l_s 2^(m_s - M) / L per head, from the same
//           (m, l) partials the log-sum-exp merge uses;
//   Q(s)  = softmax of the selected blocks' index scores (the local block
//           scored here on its visible tokens; the others come from the
//           selection's scores);
//   KL    = sum_s P(s) (log P(s) - log Q(s)).
#include "msa_common.h"

namespace msa {

// One lane per (query row of the pass, group, head): the HPG lanes of a
// (row, group) are adjacent, so each slot's (m, l) pairs of the group's heads
// are one coalesced read; every lane forms its head's softmax mass per slot,
// and a shuffle reduction over the HPG lanes averages them.
template <int HPG, int KMAX>
__global__ __launch_bounds__(256) void block_mass_kernel(const float2* __restrict__ part_ml,
                                                         const int32_t* __restrict__ sel, int r0,
                                                         int r1, int G, int top_k,
                                                         float* __restrict__ mass) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = (long long)(r1 - r0) * G * HPG;
  const bool active = i < n;
  const long long pair = active ? i / HPG : 0;        // (row - r0) * G + g
  const int h = (int)(i % HPG);
  const int rr = (int)(pair / G), g = (int)(pair % G);
  const size_t srow = ((size_t)(r0 + rr) * G + g) * top_k;
  int ns = 0;
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (s < top_k) ns += sel[srow + s] >= 0 ? 1 : 0;
  const float2* ml = part_ml + (size_t)pair * top_k * HPG + h;
  float2 v[KMAX];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    v[s] = make_float2(-INFINITY, 0.f);
    if (s < ns) v[s] = ml[(size_t)s * HPG];
    M = fmaxf(M, v[s].x);
  }
  float w[KMAX];
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    w[s] = s < ns ? v[s].y * exp2f(v[s].x - M) : 0.f;
    L += w[s];
  }
  const float inv = 1.f / (L * HPG);
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    float x = w[s] * inv;
#pragma unroll
    for (int off = HPG / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    w[s] = x;
  }
  if (!active) return;
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (s < top_k && s % HPG == h) mass[srow + s] = w[s];   // 0 for padding slots
}

template <int HPG>
static hipError_t launch_mass_h(const float2* part_ml, const int32_t* sel, int r0, int r1, int G,
                                int top_k, float* mass, hipStream_t st) {
  const long long n = (long long)(r1 - r0) * G * HPG;
  dim3 grid((unsigned)((n + 255) / 256));
#define MSA_MASS(K) hipLaunchKernelGGL((block_mass_kernel<HPG, K>), grid, dim3(256), 0, st, part_ml, sel, r0, r1, G, top_k, mass)
  if (top_k <= 4) MSA_MASS(4);
  else if (top_k <= 8) MSA_MASS(8);
  else if (top_k <= 16) MSA_MASS(16);
  else MSA_MASS(32);
#undef MSA_MASS
  return hipGetLastError();
}

hipError_t launch_block_mass(int hpg, const float2* part_ml, const int32_t* sel, int r0, int r1,
                             int G, int top_k, float* mass, hipStream_t st) {
  switch (hpg) {
    case 1: return launch_mass_h<1>(part_ml, sel, r0, r1, G, top_k, mass, st);
    case 2: return launch_mass_h<2>(part_ml, sel, r0, r1, G, top_k, mass, st);
    case 4: return launch_mass_h<4>(part_ml, sel, r0, r1, G, top_k, mass, st);
    case 8: return launch_mass_h<8>(part_ml, sel, r0, r1, G, top_k, mass, st);
    case 16: return launch_mass_h<16>(part_ml, sel, r0, r1, G, top_k, mass, st);
    case 32: return launch_mass_h<32>(part_ml, sel, r0, r1, G, top_k, mass, st);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Local block scores and the KL.  Workgroup per (query block, sequence): the
// block's index keys are staged in LDS; for each tile of 32 (query, group)
// rows whose queries lie in the block, S^T = K . Q^T on bf16 MFMA with keys
// after the query (or past the sequence) masked, and the row max is the local
// block's score.  The lane that owns a row then forms log Q over the row's
// selection and the KL against its Main-Branch masses.
// ---------------------------------------------------------------------------
template <int DI, int KMAX>
__global__ __launch_bounds__(256) void index_kl_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int G, int top_k,
    const int32_t* __restrict__ sel, const float* __restrict__ sel_score,
    const float* __restrict__ mass, float* __restrict__ log_q, float* __restrict__ kl) {
  constexpr int KS = DI / 16;
  constexpr int LD = DI + 8;           // padded row: 16-byte reads of 32 rows spread over banks
  __shared__ __attribute__((aligned(16))) uint16_t kt[kBlock * LD];

  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  if (lq <= 0) return;
  const int first = lk - lq;                          // position of the first query
  const int beta = first / kBlock + (int)blockIdx.x;  // this workgroup's block
  const int pa = max(beta * kBlock, first), pz = min((beta + 1) * kBlock, lk);
  if (pa >= pz) return;
  const int nrows = (pz - pa) * G;                    // (query, group) rows of the block
  const int tid = threadIdx.x;

  // the block's keys (rows past the sequence are zero and masked below)
  const size_t row0 = kv.block_row(b, koff, beta);
  for (int c = tid; c < kBlock * DI / 8; c += 256) {
    const int row = c / (DI / 8), cc = c % (DI / 8);
    const int key = beta * kBlock + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (key < lk) v = *reinterpret_cast<const uint4*>(k_idx + (row0 + row) * DI + cc * 8);
    *reinterpret_cast<uint4*>(kt + row * LD + cc * 8) = v;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  for (int t0 = wave * 32; t0 < nrows; t0 += 4 * 32) {
    const int n = t0 + col;
    const bool valid = n < nrows;
    const int nn = valid ? n : nrows - 1;
    const int p = pa + nn / G, g = nn % G;
    const int r = qoff + (p - first);
    bf16x8 qf[KS];
    const uint16_t* src = q_idx + ((size_t)r * G + g) * DI + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(src + ks * 16));
    float mx = -INFINITY;
#pragma unroll
    for (int ktile = 0; ktile < 4; ++ktile) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(kt + (ktile * 32 + col) * LD + ks * 16 + half * 8));
        acc = mfma32(a, qf[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = beta * kBlock + ktile * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (key <= p) mx = fmaxf(mx, acc[i]);       // key <= p < lk: visible
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (!valid || half != 0) continue;

    // log Q over the row's selection and the KL against the Main-Branch masses
    const size_t so = ((size_t)r * G + g) * top_k;
    float sc[KMAX];
    int ns = 0;
    float smax = -INFINITY;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      sc[s] = -INFINITY;
      if (s < top_k) {
        const int blk = sel[so + s];
        if (blk >= 0) {
          ++ns;
          sc[s] = blk == beta ? mx : sel_score[so + s];
          smax = fmaxf(smax, sc[s]);
        }
      }
    }
    float z = 0.f;
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      if (s < ns) z += expf(sc[s] - smax);
    const float lse = smax + logf(z);
    float div = 0.f;
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (s < top_k) {
        const float lqs = s < ns ? sc[s] - lse : __uint_as_float(0x7fc00000u);
        if (log_q) log_q[so + s] = lqs;
        if (s < ns) {
          const float pm = mass[so + s];
          if (pm > 0.f) div += pm * (logf(pm) - lqs);
        }
      }
    }
    kl[(size_t)r * G + g] = div;
  }
}

template <int DI>
static hipError_t launch_kl_di(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                               const int32_t* cu_k, KvMap kv, int batch, int G, int top_k,
                               int max_q_len,
                               const int32_t* sel, const float* sel_score, const float* mass,
                               float* log_q, float* kl, hipStream_t st) {
  // a sequence's queries span at most ceil(Lq / 128) + 1 blocks
  dim3 grid((max_q_len + kBlock - 1) / kBlock + 1, batch);
#define MSA_KL(K) hipLaunchKernelGGL((index_kl_kernel<DI, K>), grid, dim3(256), 0, st, (const uint16_t*)q_idx, (const uint16_t*)k_idx, cu_q, cu_k, kv, G, top_k, sel, sel_score, mass, log_q, kl)
  if (top_k <= 4) MSA_KL(4);
  else if (top_k <= 8) MSA_KL(8);
  else if (top_k <= 16) MSA_KL(16);
  else MSA_KL(32);
#undef MSA_KL
  return hipGetLastError();
}

hipError_t launch_index_kl(int DI, const void* q_idx, const void* k_idx, const int32_t* cu_q,
                           const int32_t* cu_k, KvMap kv, int batch, int G, int top_k,
                           int max_q_len, const int32_t* sel, const float* sel_score,
                           const float* mass, float* log_q, float* kl, hipStream_t st) {
  switch (DI) {
    case 32: return launch_kl_di<32>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, top_k, max_q_len, sel, sel_score, mass, log_q, kl, st);
    case 64: return launch_kl_di<64>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, top_k, max_q_len, sel, sel_score, mass, log_q, kl, st);
    case 128: return launch_kl_di<128>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, top_k, max_q_len, sel, sel_score, mass, log_q, kl, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
