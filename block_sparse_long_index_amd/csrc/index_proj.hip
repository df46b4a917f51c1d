// Index projections: q_idx = x W_q^T (one index-query head per GQA group) and
// k_idx = x W_k^T (one shared index-key head), the two projection matrices the
// Index Branch adds to a GQA layer (MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, section "Index BranchとMain Branchの役割分担").
//
// One bf16 GEMM over the concatenated weights [W_q; W_k] (F = (G + 1) * d_idx
// output features, K = the layer width D), computed transposed,
// C^T = [W_q; W_k] x^T, so that as in the index-score kernel each lane owns
// one token: its 4-feature runs go straight to that token's q_idx row or, for
// the key head, to the key row the token occupies in its sequence.
//
// Workgroup tile: 128 features x 256 tokens, 4 waves of 128 x 64; K in steps
// of 32 through a three-stage LDS ring filled by direct global->LDS loads two
// steps ahead.  Tile order is XCD-aware: the feature tiles of one token tile
// run on one XCD, so each x tile is fetched into one L2 and reused there.
#include <algorithm>

#include "msa_common.h"

namespace msa {

constexpr int kProjBF = 128;   // features per workgroup tile
constexpr int kProjBT = 256;   // tokens per workgroup tile
constexpr int kProjBK = 32;    // K per step
constexpr int kProjNW = 4;

// Rows of 32 bf16 (64 bytes, 4 chunks of 16 bytes); 4 rows share a 256-byte
// bank line, so chunk c of row m is stored at c ^ ((m / 4) % 4): the 16 rows a
// fragment read serves at once land in 16 different 16-byte bank groups.
__device__ inline int proj_swz(int m) { return (m >> 2) & 3; }

__global__ __launch_bounds__(kProjNW * 64, 2) void index_project_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq,
    const uint16_t* __restrict__ wk, int D, int GD, int F, int T, int n_ft, int n_tiles,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch, int DI,
    uint16_t* __restrict__ q_idx, uint16_t* __restrict__ k_idx) {
  __shared__ __attribute__((aligned(1024))) uint16_t a0[kProjBF * kProjBK];
  __shared__ __attribute__((aligned(1024))) uint16_t a1[kProjBF * kProjBK];
  __shared__ __attribute__((aligned(1024))) uint16_t a2[kProjBF * kProjBK];
  __shared__ __attribute__((aligned(1024))) uint16_t b0[kProjBT * kProjBK];
  __shared__ __attribute__((aligned(1024))) uint16_t b1[kProjBT * kProjBK];
  __shared__ __attribute__((aligned(1024))) uint16_t b2[kProjBT * kProjBK];

  // XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin, so
  // block b runs on XCD b % 8; give each XCD a contiguous run of logical tiles
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = n_tiles >> 3, rem = n_tiles & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  const int ft = logical % n_ft, tt = logical / n_ft;
  const int f0 = ft * kProjBF, t0 = tt * kProjBT;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // this lane's source rows for its 6 pieces per stage (2 of the weight tile,
  // 4 of the token tile); rows past the end are clamped (never stored)
  const int prow = lane >> 2;                        // row within a 16-row piece
  const uint16_t* asrc[2];
  const uint16_t* bsrc[4];
  int apos[2], bpos[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (wave * 2 + i) * 16 + prow;
    const int f = min(f0 + m, F - 1);
    const int lc = (lane & 3) ^ proj_swz(m);
    asrc[i] = (f < GD ? wq + (size_t)f * D : wk + (size_t)(f - GD) * D) + lc * 8;
    apos[i] = (wave * 2 + i) * 512;                  // bf16 elements: 1 KiB pieces
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (wave * 4 + i) * 16 + prow;
    const int t = min(t0 + m, T - 1);
    const int lc = (lane & 3) ^ proj_swz(m);
    bsrc[i] = x + (size_t)t * D + lc * 8;
    bpos[i] = (wave * 4 + i) * 512;
  }
  auto load = [&](int ks, uint16_t* sa, uint16_t* sb) __attribute__((always_inline)) {
    const int k0 = ks * kProjBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_global_load_lds(asrc[i] + k0, sa + apos[i], 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_global_load_lds(bsrc[i] + k0, sb + bpos[i], 16, 0, 0);
  };
  auto frag = [&](const uint16_t* s, int m, int lc) __attribute__((always_inline)) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(s + m * kProjBK + ((lc ^ proj_swz(m)) * 8)));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = D / kProjBK;
  load(0, a0, b0);
  if (nk > 1) load(1, a1, b1);

  auto step = [&](int ks, const uint16_t* ra, const uint16_t* rb, uint16_t* la, uint16_t* lb)
      __attribute__((always_inline)) {
    // this wave's pieces of step ks have landed (only step ks+1 may be younger);
    // the barrier publishes every wave's pieces and retires the reads of the
    // stage about to be refilled
    if (ks + 1 < nk) wait_vmcnt<6>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ks + 2 < nk) load(ks + 2, la, lb);
#pragma unroll
    for (int kk = 0; kk < kProjBK / 16; ++kk) {
      bf16x8 fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag(ra, i * 32 + col, 2 * kk + half);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = frag(rb, wave * 64 + j * 32 + col, 2 * kk + half);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
    }
  };
  for (int ks = 0; ks < nk; ks += 3) {
    step(ks, a0, b0, a2, b2);
    if (ks + 1 < nk) step(ks + 1, a1, b1, a0, b0);
    if (ks + 2 < nk) step(ks + 2, a2, b2, a1, b1);
  }

  // epilogue: lane <-> token; register 4j..4j+3 of tile i <-> features
  // f0 + 32i + 8j + 4half + 0..3, written as one 8-byte run
#pragma unroll
  for (int j2 = 0; j2 < 2; ++j2) {
    const int t = t0 + wave * 64 + j2 * 32 + col;
    if (t >= T) continue;
    const RowPos rp = locate_row(t, cu_q, cu_k, batch);
    const size_t krow = kv.key_row(rp.b, rp.koff, rp.p);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = f0 + 32 * i + 8 * j + 4 * half;
        if (f >= F) continue;
        const uint2 v = make_uint2(pack2_bf16(acc[i][j2][4 * j], acc[i][j2][4 * j + 1]),
                                   pack2_bf16(acc[i][j2][4 * j + 2], acc[i][j2][4 * j + 3]));
        uint16_t* dst = f < GD ? q_idx + (size_t)t * GD + f : k_idx + krow * DI + (f - GD);
        *reinterpret_cast<uint2*>(dst) = v;
      }
  }
}

// Few tokens (decode and verification steps): the work is reading the
// weights once, and 32 x 32 output tiles alone would give a few dozen
// workgroups, each walking all of K through a long chain of dependent loads.
// So K is split across workgroups as well: workgroup (feature tile, token
// tile, slice) multiplies its tile over one slice of K (a run of 64-element
// chunks; its 4 waves take every 4th chunk and load up to 4 chunks'
// fragments at once, straight from global memory), the waves' tiles are
// summed through LDS in a fixed order, and the fp32 tile goes to the
// workspace.  A second kernel sums the slices in order, rounds to bf16 and
// stores the outputs.  Nothing is accumulated with atomics, so results are
// deterministic.
constexpr int kProjSmallMaxT = 512;     // token counts up to this take the split path
constexpr int kProjSplitWaves = 4;
constexpr int kProjSplitChunks = 4;     // chunks a wave has in flight
constexpr int kProjSplitMax = 32;       // slices of K at most (sizes the workspace)
constexpr int kProjSplitTarget = 512;   // workgroups the split aims for at least

// slices of K for T tokens, F features and C chunks of 64: enough workgroups
// to fill the GPU, and few enough chunks per wave to load them in one go
static int project_split(int T, int F, int C) {
  const long long tiles = (long long)((F + 31) / 32) * ((T + 31) / 32);
  const long long want = std::max((kProjSplitTarget + tiles - 1) / tiles,
                                  (long long)(C + kProjSplitWaves * kProjSplitChunks - 1) /
                                      (kProjSplitWaves * kProjSplitChunks));
  // every wave keeps at least one chunk
  const long long cap = std::min<long long>(kProjSplitMax, std::max(1, C / kProjSplitWaves));
  return (int)std::max(1ll, std::min(want, cap));
}

size_t project_workspace_bytes(int T, int F) {
  if (T <= 0 || T > kProjSmallMaxT) return 0;
  return (size_t)kProjSplitMax * (size_t)((T + 31) / 32 * 32) * (size_t)((F + 31) / 32 * 32) *
         sizeof(float);
}

// part: fp32 [KS][Tp][Fp], Tp / Fp = T / F rounded up to 32 (padding rows and
// columns get values from clamped operands and are never read back)
__global__ __launch_bounds__(kProjSplitWaves * 64) void index_project_split_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq,
    const uint16_t* __restrict__ wk, int D, int GD, int F, int T, int n_ft, int n_tt, int KS,
    int Tp, int Fp, float* __restrict__ part) {
  __shared__ float red[kProjSplitWaves - 1][16][64];
  const int ft = blockIdx.x % n_ft;
  const int rest = blockIdx.x / n_ft;
  const int tt = rest % n_tt, ks = rest / n_tt;
  const int f0 = ft * 32, t0 = tt * 32;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int f = min(f0 + col, F - 1);
  const int t = min(t0 + col, T - 1);
  const uint16_t* arow = (f < GD ? wq + (size_t)f * D : wk + (size_t)(f - GD) * D) + 8 * half;
  const uint16_t* brow = x + (size_t)t * D + 8 * half;
  const int C = D / 64;                                   // 64-element chunks of K
  const int c0 = (int)((long long)ks * C / KS), c1 = (int)((long long)(ks + 1) * C / KS);
  f32x16 acc = f32x16{};
  constexpr int NC = kProjSplitChunks;
  for (int cb = c0 + wave; cb < c1; cb += NC * kProjSplitWaves) {
    uint4 a[NC][4], bb[NC][4];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = cb + u * kProjSplitWaves;
      if (c < c1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a[u][s] = *reinterpret_cast<const uint4*>(arow + (size_t)c * 64 + 16 * s);
          bb[u][s] = *reinterpret_cast<const uint4*>(brow + (size_t)c * 64 + 16 * s);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      if (cb + u * kProjSplitWaves < c1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma32(as_bf16x8(a[u][s]), as_bf16x8(bb[u][s]), acc);
      }
    }
  }
  if (wave != 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = acc[i];
#pragma unroll
    for (int w = 0; w < kProjSplitWaves - 1; ++w) v += red[w][i][lane];
    acc[i] = v;
  }
  // lane holds token t0 + col, features f0 + 8j + 4 half + (0..3)
  float* dst = part + ((size_t)ks * Tp + t0 + col) * Fp + f0 + 4 * half;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<float4*>(dst + 8 * j) =
        make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
}

// One thread per (token, run of 4 features): the slices summed in order,
// rounded to bf16 and stored to the token's q_idx row or its key row.
__global__ __launch_bounds__(256) void index_project_reduce_kernel(
    const float* __restrict__ part, int KS, int Tp, int Fp, int T, int F, int GD, int DI,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch,
    uint16_t* __restrict__ q_idx, uint16_t* __restrict__ k_idx) {
  const int F4 = F / 4;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)T * F4) return;
  const int tok = (int)(i / F4), ff = (int)(i % F4) * 4;
  const float* src = part + (size_t)tok * Fp + ff;
  const size_t slice = (size_t)Tp * Fp;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  // eight slices' loads in flight at a time, added in slice order
  for (int k0 = 0; k0 < KS; k0 += 8) {
    float4 u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < KS) u[j] = *reinterpret_cast<const float4*>(src + (size_t)(k0 + j) * slice);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (k0 + j < KS) {
        v.x += u[j].x;
        v.y += u[j].y;
        v.z += u[j].z;
        v.w += u[j].w;
      }
    }
  }
  const uint2 o = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
  if (ff < GD) {
    *reinterpret_cast<uint2*>(q_idx + (size_t)tok * GD + ff) = o;
  } else {
    const RowPos rp = locate_row(tok, cu_q, cu_k, batch);
    *reinterpret_cast<uint2*>(k_idx + kv.key_row(rp.b, rp.koff, rp.p) * DI + (ff - GD)) = o;
  }
}

hipError_t launch_index_project(const void* x, const void* wq, const void* wk, int D, int G, int DI,
                                int T, const int32_t* cu_q, const int32_t* cu_k, KvMap kv,
                                int batch, void* q_idx, void* k_idx, void* workspace,
                                hipStream_t st) {
  const int GD = G * DI, F = GD + DI;
  if (T <= 0) return hipSuccess;
  if (T <= kProjSmallMaxT) {
    const int n_ft = (F + 31) / 32, n_tt = (T + 31) / 32;
    const int Tp = n_tt * 32, Fp = n_ft * 32;
    // at least 4 chunks of 64 per slice, so that every wave has work
    const int KS = project_split(T, F, D / 64);
    float* part = reinterpret_cast<float*>(workspace);
    hipLaunchKernelGGL(index_project_split_kernel, dim3(n_ft * n_tt * KS), dim3(kProjSplitWaves * 64),
                       0, st, (const uint16_t*)x, (const uint16_t*)wq, (const uint16_t*)wk, D, GD, F,
                       T, n_ft, n_tt, KS, Tp, Fp, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long n = (long long)T * (F / 4);
    hipLaunchKernelGGL(index_project_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, (const float*)part, KS, Tp, Fp, T, F, GD, DI, cu_q, cu_k, kv, batch,
                       (uint16_t*)q_idx, (uint16_t*)k_idx);
    return hipGetLastError();
  }
  const int n_ft = (F + kProjBF - 1) / kProjBF;
  const long long n_tt = ((long long)T + kProjBT - 1) / kProjBT;
  const long long n_tiles = n_ft * n_tt;
  if (n_tiles <= 0) return hipSuccess;
  if (n_tiles >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(index_project_kernel, dim3((unsigned)n_tiles), dim3(kProjNW * 64), 0, st,
                     (const uint16_t*)x, (const uint16_t*)wq, (const uint16_t*)wk, D, GD, F, T,
                     n_ft, (int)n_tiles, cu_q, cu_k, kv, batch, DI, (uint16_t*)q_idx,
                     (uint16_t*)k_idx);
  return hipGetLastError();
}

}  // namespace msa
