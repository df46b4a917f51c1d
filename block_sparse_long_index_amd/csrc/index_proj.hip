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
// Workgroup tile: 128 features x 512 tokens, one wave per SIMD, each wave a
// 128 x 128 register tile (16 MFMA tiles, 256 accumulators), so every
// fragment read from LDS feeds four MFMAs.  K runs in stages of 32: the
// weight tile and each wave's own 128 token rows go through a four-stage LDS
// ring (160 KiB: all of a CU's LDS) filled by direct global->LDS loads.
// The barrier sits in the middle of a stage, so no fragment read is ever
// waited for right away: a stage issues its second half's reads, runs its
// first half's 16 MFMAs, waits for the next stage's loads and passes the
// barrier, refills its own buffer, issues the next stage's first-half reads
// and runs its second half's MFMAs.
// Tile order is XCD-aware: the feature tiles of one token tile run on one
// XCD, so each x tile is fetched into one L2 and reused there.
#include <algorithm>

#include "msa_common.h"

namespace msa {

constexpr int kProjBF = 128;   // features per workgroup tile
constexpr int kProjBT = 512;   // tokens per workgroup tile (128 per wave)
constexpr int kProjBK = 32;    // K per stage
constexpr int kProjNW = 4;

// Rows of 32 bf16 (64 bytes, 4 chunks of 16 bytes); 4 rows share a 256-byte
// bank line, so chunk c of row m is stored at c ^ ((m / 4) % 4): the 16 rows a
// fragment read serves at once land in 16 different 16-byte bank groups.
__device__ inline int proj_swz(int m) { return (m >> 2) & 3; }

// vmcnt(n) for n < 64 (gfx9 encoding: low four bits and bits 14-15)
template <int N>
__device__ inline void wait_vmcnt_wide() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N >> 4) << 14 | 0x0F70 | (N & 15));
}

// the fragments of one half-stage (16 of the stage's 32 K): 4 weight tiles
// and 4 token tiles of 32 rows
struct ProjFrags {
  bf16x8 a[4], b[4];
};

// PART: the workgroup sums one slice of K (kps stages; the last slice may be
// shorter) and stores its fp32 tile to part [slice][T][F], which
// index_project_reduce_kernel adds up; otherwise it sums all of K and stores
// the bf16 outputs.
template <bool PART>
__global__ __launch_bounds__(kProjNW * 64, 1) void index_project_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wq,
    const uint16_t* __restrict__ wk, int D, int GD, int F, int T, int n_ft, int n_tt, int n_tiles,
    int kps, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch,
    int DI, uint16_t* __restrict__ q_idx, uint16_t* __restrict__ k_idx, float* __restrict__ part) {
  // one array per stage: the weight tile [128 rows][32 elements], then the
  // token rows [wave][128 rows][32 elements]
  constexpr int kStageElems = (kProjBF + kProjBT) * kProjBK;
  __shared__ __attribute__((aligned(1024))) uint16_t s0[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t s1[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t s2[kStageElems];
  __shared__ __attribute__((aligned(1024))) uint16_t s3[kStageElems];

  // XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin, so
  // block b runs on XCD b % 8; give each XCD a contiguous run of logical tiles
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = n_tiles >> 3, rem = n_tiles & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  const int ft = logical % n_ft, rest = logical / n_ft;
  const int tt = rest % n_tt, slice = rest / n_tt;
  const int f0 = ft * kProjBF, t0 = tt * kProjBT;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // weight tile: 8 pieces of 16 rows per stage, 2 per wave; rows past F are
  // clamped (their outputs are never stored)
  const int prow = lane >> 2;                        // row within a 16-row piece
  const uint16_t* asrc[2];
  int apos[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = (wave * 2 + i) * 16 + prow;
    const int f = min(f0 + m, F - 1);
    const int lc = (lane & 3) ^ proj_swz(m);
    asrc[i] = (f < GD ? wq + (size_t)f * D : wk + (size_t)(f - GD) * D) + lc * 8;
    apos[i] = (wave * 2 + i) * 512;                  // bf16 elements: 1 KiB pieces
  }
  // this wave's token rows: 8 pieces of 16 rows per stage, laid out as the
  // weight tile; rows past T are clamped (never stored)
  const uint16_t* bsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = i * 16 + prow;
    const int t = min(t0 + wave * 128 + m, T - 1);
    bsrc[i] = x + (size_t)t * D + ((lane & 3) ^ proj_swz(m)) * 8;
  }
  const int bbase = kProjBF * kProjBK + wave * 128 * kProjBK;
  // this workgroup's stages of K: kps per slice, kps and D / kProjBK even, so
  // every slice has an even count >= 2
  const int kb = slice * kps;
  const int nk = min(kps, D / kProjBK - kb);
  // stage s of K into buf; a stage past the last is clamped to it (the copy
  // lands in a buffer no stage reads), so every stage issues the same loads
  // and the loop has no branch.  After a branch joins, the compiler can no
  // longer tell which buffer a direct load in flight writes and waits for all
  // of them before the next LDS read, which would drain the prefetch.
  auto load = [&](int s, uint16_t* buf) __attribute__((always_inline)) {
    const int k0 = (kb + min(s, nk - 1)) * kProjBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_global_load_lds(asrc[i] + k0, buf + apos[i], 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(bsrc[i] + k0, buf + bbase + i * 512, 16, 0, 0);
  };
  auto frag = [&](const uint16_t* buf, int m, int c) __attribute__((always_inline)) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(buf + m * kProjBK + ((c ^ proj_swz(m)) * 8)));
  };
  // half u of a stage: K elements 16u .. 16u + 15, lane half h holding 8h .. 8h + 7
  auto read = [&](const uint16_t* buf, int u, ProjFrags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = frag(buf + bbase, j * 32 + col, 2 * u + half);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = frag(buf, i * 32 + col, 2 * u + half);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  auto mfmas = [&](const ProjFrags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // prologue: stages 0 .. 3 in flight, stage 0 published, its first half read
  ProjFrags fa;
  load(0, s0);
  load(1, s1);
  load(2, s2);
  load(3, s3);
  wait_vmcnt_wide<30>();
  sync();
  read(s0, 0, fa);

  // a half-stage's 16 MFMAs with the 8 fragment reads of the next half
  // between its first 9, one at a time: a burst of reads fills the LDS
  // command queue and holds up the MFMAs behind it.  Each half starts with an
  // MFMA, so the wait the compiler puts before it covers only fragments read
  // a half-stage earlier.
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // an MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // a fragment read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);     // the other 8 MFMAs
  };

  // stage s: buffer rb holds it, nb the next; fa holds its first half
  auto stage = [&](int s, uint16_t* rb, const uint16_t* nb) __attribute__((always_inline)) {
    ProjFrags fb;
    read(rb, 1, fb);
    mfmas(fa);
    interleave();
    __builtin_amdgcn_sched_barrier(0);   // none of them may sink past the barrier
    // stage s + 1 has landed (stages s + 2 and s + 3, 10 loads each, may be
    // younger) and this wave's reads of stage s are done; the barrier
    // publishes every wave's pieces of stage s + 1 and frees rb for stage s + 4
    wait_vmcnt_wide<20>();
    sync();
    load(s + 4, rb);
    read(nb, 0, fa);
    mfmas(fb);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  int s = 0;
  for (; s + 4 <= nk; s += 4) {
    stage(s, s0, s1);
    stage(s + 1, s1, s2);
    stage(s + 2, s2, s3);
    stage(s + 3, s3, s0);
  }
  if (s < nk) {   // nk % 4 == 2
    stage(s, s0, s1);
    stage(s + 1, s1, s2);
  }
  wait_vmcnt_wide<0>();   // no direct load may still write LDS when the workgroup ends

  // epilogue: lane <-> token; register 4r..4r+3 of tile (i, j) <-> features
  // f0 + 32i + 8r + 4half + 0..3 of token t0 + 128 wave + 32 j + col, written
  // as one 8-byte bf16 run (or one 16-byte fp32 run of the slice's tile)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + wave * 128 + j * 32 + col;
    if (t >= T) continue;
    if constexpr (PART) {
      float* dst = part + ((size_t)slice * T + t) * F;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = f0 + 32 * i + 8 * r + 4 * half;
          if (f < F)
            *reinterpret_cast<float4*>(dst + f) =
                make_float4(acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]);
        }
      continue;
    }
    const RowPos rp = locate_row(t, cu_q, cu_k, batch);
    const size_t krow = kv.key_row(rp.b, rp.koff, rp.p);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = f0 + 32 * i + 8 * r + 4 * half;
        if (f >= F) continue;
        const uint2 v = make_uint2(pack2_bf16(acc[i][j][4 * r], acc[i][j][4 * r + 1]),
                                   pack2_bf16(acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]));
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

// Up to a few thousand tokens the large-tile kernel has fewer tiles than the
// GPU has CUs (one large-tile workgroup fits a CU), and its time is one
// workgroup's walk over all of K.  Then K is split into slices as well, as
// many as keep every workgroup in one round, each of at least 16 stages (512
// of K); the fp32 slice tiles go to the workspace and the reduce kernel adds
// them in slice order.  With at most 256 / tiles slices of T x F, the
// workspace stays under 256 x 512 x 128 x 4 B = 64 MiB.
constexpr int kProjCUs = 256;            // compute units of a gfx950 GPU
constexpr int kProjBigSplitMax = 16;
constexpr int kProjBigMinStages = 16;

// slices of K for n_tiles large tiles and nk stages of K (0: not known yet)
static int project_big_split(long long n_tiles, int nk) {
  if (n_tiles <= 0 || 2 * n_tiles > kProjCUs) return 1;
  int S = (int)std::min<long long>(kProjBigSplitMax, kProjCUs / n_tiles);
  if (nk > 0) S = std::min(S, nk / kProjBigMinStages);
  return std::max(S, 1);
}

static long long project_big_tiles(int T, int F) {
  return (long long)((F + kProjBF - 1) / kProjBF) * (((long long)T + kProjBT - 1) / kProjBT);
}

// what the fastest launch uses (the split of K, whenever it applies)
size_t project_workspace_bytes(int T, int F) {
  if (T <= 0) return 0;
  if (T <= kProjSmallMaxT)
    return (size_t)kProjSplitMax * (size_t)((T + 31) / 32 * 32) * (size_t)((F + 31) / 32 * 32) *
           sizeof(float);
  const int S = project_big_split(project_big_tiles(T, F), 0);
  return S >= 2 ? (size_t)S * (size_t)T * (size_t)F * sizeof(float) : 0;
}

// what a call must be given: the few-token path always splits K; above it the
// split is taken only when the workspace holds it
size_t project_workspace_required(int T, int F) {
  return T <= kProjSmallMaxT ? project_workspace_bytes(T, F) : 0;
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
                                size_t workspace_bytes, hipStream_t st) {
  const int GD = G * DI, F = GD + DI;
  if (T <= 0) return hipSuccess;
  float* part = reinterpret_cast<float*>(workspace);
  auto reduce = [&](int KS, int Tp, int Fp) {
    const long long n = (long long)T * (F / 4);
    hipLaunchKernelGGL(index_project_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       st, (const float*)part, KS, Tp, Fp, T, F, GD, DI, cu_q, cu_k, kv, batch,
                       (uint16_t*)q_idx, (uint16_t*)k_idx);
    return hipGetLastError();
  };
  if (T <= kProjSmallMaxT) {
    const int n_ft = (F + 31) / 32, n_tt = (T + 31) / 32;
    const int Tp = n_tt * 32, Fp = n_ft * 32;
    // at least 4 chunks of 64 per slice, so that every wave has work
    const int KS = project_split(T, F, D / 64);
    hipLaunchKernelGGL(index_project_split_kernel, dim3(n_ft * n_tt * KS), dim3(kProjSplitWaves * 64),
                       0, st, (const uint16_t*)x, (const uint16_t*)wq, (const uint16_t*)wk, D, GD, F,
                       T, n_ft, n_tt, KS, Tp, Fp, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return reduce(KS, Tp, Fp);
  }
  const int n_ft = (F + kProjBF - 1) / kProjBF;
  const long long n_tt = ((long long)T + kProjBT - 1) / kProjBT;
  const long long n_tiles = n_ft * n_tt;
  if (n_tiles <= 0) return hipSuccess;
  if (n_tiles >= (1ll << 31)) return hipErrorInvalidValue;
  const int nk = D / kProjBK;                      // even, >= 2
  int S = project_big_split(n_tiles, nk), kps = nk;
  if (S >= 2) {
    kps = (nk + S - 1) / S;
    kps += kps & 1;                                // even: every slice's stage count is even
    S = (nk + kps - 1) / kps;
  }
  if (S >= 2 && part && workspace_bytes >= (size_t)S * (size_t)T * (size_t)F * sizeof(float)) {
    hipLaunchKernelGGL(index_project_kernel<true>, dim3((unsigned)(n_tiles * S)), dim3(kProjNW * 64), 0,
                       st, (const uint16_t*)x, (const uint16_t*)wq, (const uint16_t*)wk, D, GD, F, T,
                       n_ft, (int)n_tt, (int)(n_tiles * S), kps, cu_q, cu_k, kv, batch, DI,
                       (uint16_t*)q_idx, (uint16_t*)k_idx, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return reduce(S, T, F);
  }
  hipLaunchKernelGGL(index_project_kernel<false>, dim3((unsigned)n_tiles), dim3(kProjNW * 64), 0, st,
                     (const uint16_t*)x, (const uint16_t*)wq, (const uint16_t*)wk, D, GD, F, T,
                     n_ft, (int)n_tt, (int)n_tiles, nk, cu_q, cu_k, kv, batch, DI, (uint16_t*)q_idx,
                     (uint16_t*)k_idx, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace msa
