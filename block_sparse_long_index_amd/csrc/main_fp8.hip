// Quantised Main Branch inputs: 8-bit queries, keys and values.
//
// The pages state that the production model runs both the sparse-attention
// indexer and the Main Branch with 8-bit queries and 8-bit keys/values
// (dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
// "MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開", on the model card's
// quantisation notes).  As for the index branch, codes are OCP FP8 E4M3 with
// power-of-two (E8M0) scales: one per (query row, head) of q, and one per
// (sequence block, KV head) of k and of v -- the unit the Main Branch stages.
// The attention kernels dequantise while loading (exactly, into bf16) and
// then compute what the bf16 path computes.
#include "fp8_common.h"

namespace msa {

// K or V [rows, G, D] of one (block beta, sequence b, head g) per workgroup:
// the block's maximum over its keys in the sequence, its exponent, its codes.
// Exponents: [block index][G] (block index b * nb_max + beta, or the page);
// blocks past a contiguous sequence's end get the neutral 127.
template <int D>
__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ cu_k, KvMap kv,
                                                          int nb_max, int G, uint8_t* __restrict__ x8,
                                                          uint8_t* __restrict__ xe) {
  constexpr int LPR = D / 8;                     // 16-byte bf16 chunks per key row
  constexpr int PER = kBlock * LPR / 256;        // chunks per thread
  __shared__ float red[4];
  const int beta = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int n = min(kBlock, lk - beta * kBlock);   // keys of this block in the sequence
  const int tid = threadIdx.x;
  if (n <= 0) {
    if (tid == 0 && !kv.table) xe[((size_t)b * nb_max + beta) * G + g] = 127;
    return;
  }
  const size_t row0 = kv.block_row(b, koff, beta);
  const size_t ld = (size_t)G * D;                 // elements between consecutive keys
  const uint16_t* src = x + row0 * ld + (size_t)g * D;
  float v[PER][8];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256, row = c / LPR, col = c % LPR;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (row < n) w = *reinterpret_cast<const uint4*>(src + row * ld + col * 8);
    unpack8_bf16(w, v[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[i][j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, shfl_xor_f(a, off));
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = fp8_scale_exponent(a);
  uint8_t* dst = x8 + row0 * ld + (size_t)g * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256, row = c / LPR, col = c % LPR;
    const uint2 w = quantize8(v[i], e);
    if (row < n) *reinterpret_cast<uint2*>(dst + row * ld + col * 8) = w;
  }
  if (tid == 0) xe[kv.block_index(b, beta, nb_max) * G + g] = (uint8_t)(e + 127);
}

// 4-bit keys or values: E2M1 codes with one E8M0 exponent per 32 elements of
// every (key, KV head) row (the same rule as the 4-bit index keys: e is the
// smallest integer with amax * 2^-e <= 6, clamped to [-127, 127]; nearest
// E2M1 value of x * 2^-e, ties to the even code, with x's sign bit).  One
// workgroup per (block beta, sequence b): the block's keys are n * G rows of D
// elements, 8 per lane; the four lanes of a 32-element group share its
// maximum through two shuffles.  Codes [rows][G][D/2] (element 2i in the low
// nibble), exponents [rows][G][D/32]; rows past the sequence are not written.
template <int D>
__global__ __launch_bounds__(256) void quantize_kv4_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ cu_k, KvMap kv,
                                                           int G, uint8_t* __restrict__ x4,
                                                           uint8_t* __restrict__ xe) {
  constexpr int LPR = D / 8;    // 8-element chunks per (key, head) row
  const int beta = blockIdx.x, b = blockIdx.y;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int n = min(kBlock, lk - beta * kBlock);
  if (n <= 0) return;
  const size_t r0 = kv.block_row(b, koff, beta) * G;      // first (key, head) row of the block
  const int chunks = n * G * LPR;                          // a multiple of 4: whole groups
  const int iters = (kBlock * G * LPR + 255) / 256;        // the same count for every lane
  for (int it = 0; it < iters; ++it) {
    const int c = (int)threadIdx.x + it * 256;
    const bool ok = c < chunks;
    const int row = c / LPR, col = c % LPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4*>(x + (r0 + row) * D + col * 8);
    float f[8];
    unpack8_bf16(v, f);
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
    a = fmaxf(a, shfl_xor_f(a, 1));
    a = fmaxf(a, shfl_xor_f(a, 2));
    const int e = fp4_scale_exponent(a);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_code(ldexpf(f[j], -e)) << (4 * j);
    if (ok) {
      *reinterpret_cast<uint32_t*>(x4 + (r0 + row) * (D / 2) + col * 4) = w;
      if ((col & 3) == 0) xe[(r0 + row) * (D / 32) + col / 4] = (uint8_t)(e + 127);
    }
  }
}

template <int D>
static hipError_t launch_main_quantize_kv4_d(const void* q, const void* k, const void* v,
                                             const int32_t* cu_k, KvMap kv, int batch, int G,
                                             int nb_max, long long q_rows, void* q8, uint8_t* qe,
                                             void* k4, uint8_t* ke, void* v4, uint8_t* ve,
                                             hipStream_t st) {
  if (q && q_rows > 0) {
    const long long threads = q_rows * (D / 8);
    hipLaunchKernelGGL(quantize_q_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, (const uint16_t*)q, q_rows, (uint8_t*)q8, qe);
  }
  const dim3 grid(nb_max, batch);
  if (k && nb_max > 0)
    hipLaunchKernelGGL(quantize_kv4_kernel<D>, grid, dim3(256), 0, st, (const uint16_t*)k, cu_k, kv,
                       G, (uint8_t*)k4, ke);
  if (v && nb_max > 0)
    hipLaunchKernelGGL(quantize_kv4_kernel<D>, grid, dim3(256), 0, st, (const uint16_t*)v, cu_k, kv,
                       G, (uint8_t*)v4, ve);
  return hipGetLastError();
}

hipError_t launch_main_quantize_q8kv4(int D, const void* q, const void* k, const void* v,
                                      const int32_t* cu_k, KvMap kv, int batch, int G, int nb_max,
                                      long long q_rows, void* q8, uint8_t* qe, void* k4,
                                      uint8_t* ke, void* v4, uint8_t* ve, hipStream_t st) {
  switch (D) {
    case 64: return launch_main_quantize_kv4_d<64>(q, k, v, cu_k, kv, batch, G, nb_max, q_rows, q8, qe, k4, ke, v4, ve, st);
    case 128: return launch_main_quantize_kv4_d<128>(q, k, v, cu_k, kv, batch, G, nb_max, q_rows, q8, qe, k4, ke, v4, ve, st);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_main_quantize_d(const void* q, const void* k, const void* v,
                                         const int32_t* cu_k, KvMap kv, int batch, int G,
                                         int nb_max, long long q_rows, void* q8, uint8_t* qe,
                                         void* k8, uint8_t* ke, void* v8, uint8_t* ve,
                                         hipStream_t st) {
  if (q && q_rows > 0) {
    const long long threads = q_rows * (D / 8);
    hipLaunchKernelGGL(quantize_q_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, (const uint16_t*)q, q_rows, (uint8_t*)q8, qe);
  }
  const dim3 grid(nb_max, batch, G);
  if (k && nb_max > 0)
    hipLaunchKernelGGL(quantize_kv_kernel<D>, grid, dim3(256), 0, st, (const uint16_t*)k, cu_k, kv,
                       nb_max, G, (uint8_t*)k8, ke);
  if (v && nb_max > 0)
    hipLaunchKernelGGL(quantize_kv_kernel<D>, grid, dim3(256), 0, st, (const uint16_t*)v, cu_k, kv,
                       nb_max, G, (uint8_t*)v8, ve);
  return hipGetLastError();
}

hipError_t launch_main_quantize_fp8(int D, const void* q, const void* k, const void* v,
                                    const int32_t* cu_k, KvMap kv, int batch, int G, int nb_max,
                                    long long q_rows, void* q8, uint8_t* qe, void* k8, uint8_t* ke,
                                    void* v8, uint8_t* ve, hipStream_t st) {
  switch (D) {
    case 64: return launch_main_quantize_d<64>(q, k, v, cu_k, kv, batch, G, nb_max, q_rows, q8, qe, k8, ke, v8, ve, st);
    case 128: return launch_main_quantize_d<128>(q, k, v, cu_k, kv, batch, G, nb_max, q_rows, q8, qe, k8, ke, v8, ve, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
