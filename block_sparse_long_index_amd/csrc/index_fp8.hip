// Quantised Index Branch: 8-bit index queries and keys.
//
// The pages state that the production model runs the sparse-attention indexer
// (and Main Branch) with 8-bit queries and 8-bit keys, moving to 4-bit keys
// (dot-ai.myuuu.co.jp article on MiniMax M3.1 Flash, section
// "MiniMax M3.1 Flashとは？428BのMoEモデルがウェイト公開", on the model card's
// quantisation notes).  The format and scaling are not given; this
// file implements OCP FP8 E4M3 codes with power-of-two (E8M0) scales, one per
// (query row, group) of q_idx and one per (sequence, 128-token block) of
// k_idx.  The selection rule is the one of the bf16 path (token scores,
// block max-pool, forced local block, top_k - 1 others; MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections "2段階構造の中身" and
// "クエリを含むローカルブロックの強制取り込み"), evaluated on the dequantised values.
//
// Because a key block's scale 2^ek is one positive factor for all its keys,
// max_j (2^eq q8 . 2^ek k8_j) = 2^(eq + ek) max_j (q8 . k8_j): the kernels
// contract raw codes on the fp8 MFMA and apply the two exponents once per
// (row, block), exactly (ldexp).
//
// 4-bit index keys (the pages' move to 4-bit keys) are OCP E2M1 codes, two
// per byte (element 2i in the low nibble), with one E8M0 exponent per 32
// elements of a key row, the microscaling layout that gfx950's scaled MFMA
// consumes directly: the keys' exponents go to the MFMA as per-lane scales and
// the query's exponent is applied to the block maximum as before.  The prefill
// kernel reads them when instantiated with K4; decode steps have a kernel of
// their own (index_score_decode_k4_kernel).
#include "fp8_common.h"
#include "msa_common.h"
#include "topk_common.h"

namespace msa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 MFMA on OCP E4M3 operands (A and B format code 0), fp32
// accumulate, no block scaling.  Same output layout as mfma32; each lane half
// supplies 32 of the 64 contraction bytes of its row / column, with the same
// assignment in A and B.
__device__ inline f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32x32x64 MFMA of E2M1 keys (A, format code 4) against E4M3 queries (B,
// format 0) with per-lane E8M0 scales (2^(s - 127)).  Measured lane layout:
// A lane half h holds contraction elements 32h .. 32h+31 in its first 16 bytes
// (low nibble first); B lane half h holds elements 16h .. 16h+15 in bytes 0-15
// and 32+16h .. 32+16h+15 in bytes 16-31; lane half h's scale covers elements
// 32h .. 32h+31 of its row (A) or column (B).  Products are summed as for the
// fp8 MFMA (groups of 8 aligned to their largest product).
__device__ inline f32x16 mfma32_k4(i32x8 a, i32x8 b, f32x16 c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, 127);
}

__device__ inline i32x8 as_i32x8(uint4 lo, uint4 hi) {
  i32x8 r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// k blocks: one workgroup per (block beta, sequence b); block maximum over the
// block's keys that belong to the sequence; blocks past its end get 127.
template <int DI>
__global__ __launch_bounds__(256) void quantize_k_kernel(const uint16_t* __restrict__ k,
                                                         const int32_t* __restrict__ cu_k, KvMap kv,
                                                         int nb_max, uint8_t* __restrict__ k8,
                                                         uint8_t* __restrict__ ke) {
  constexpr int LPR = DI / 8;                      // 16-byte bf16 chunks per key row
  constexpr int PER = kBlock * LPR / 256;          // chunks per thread
  __shared__ float red[4];
  const int beta = blockIdx.x, b = blockIdx.y;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int n = min(kBlock, lk - beta * kBlock);   // keys of this block in the sequence
  const int tid = threadIdx.x;
  if (n <= 0) {   // past the sequence: a contiguous cache keeps the neutral exponent
    if (tid == 0 && !kv.table) ke[(size_t)b * nb_max + beta] = 127;
    return;
  }
  const size_t row0 = kv.block_row(b, koff, beta);
  const uint16_t* src = k + row0 * DI;
  float x[PER][8];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256, row = c / LPR, col = c % LPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < n) v = *reinterpret_cast<const uint4*>(src + (size_t)row * DI + col * 8);
    unpack8_bf16(v, x[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[i][j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, shfl_xor_f(a, off));
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = fp8_scale_exponent(a);
  uint8_t* dst = k8 + row0 * DI;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256, row = c / LPR, col = c % LPR;
    const uint2 w = quantize8(x[i], e);
    if (row < n) *reinterpret_cast<uint2*>(dst + (size_t)row * DI + col * 8) = w;
  }
  if (tid == 0) ke[kv.block_index(b, beta, nb_max)] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------
// 4-bit index keys (fp4_scale_exponent, e2m1_code: fp8_common.h)
// ---------------------------------------------------------------------------
// Key rows of one (block beta, sequence b) per workgroup, 8 elements per lane:
// the four lanes of a 32-element group share its maximum through shuffles.
// Codes: [rows][DI / 2] bytes; exponents: [rows][DI / 32], row as for k_idx.
// Rows past the sequence's end are not written.
template <int DI>
__global__ __launch_bounds__(256) void quantize_k4_kernel(const uint16_t* __restrict__ k,
                                                          const int32_t* __restrict__ cu_k, KvMap kv,
                                                          uint8_t* __restrict__ k4,
                                                          uint8_t* __restrict__ ke4) {
  constexpr int LPR = DI / 8;                      // 8-element chunks per key row
  constexpr int PER = kBlock * LPR / 256;          // chunks per thread
  static_assert(LPR % 4 == 0 && PER >= 1, "whole 32-element groups per row");
  const int beta = blockIdx.x, b = blockIdx.y;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int n = min(kBlock, lk - beta * kBlock);
  if (n <= 0) return;
  const size_t row0 = kv.block_row(b, koff, beta);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256, row = c / LPR, col = c % LPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < n) v = *reinterpret_cast<const uint4*>(k + (row0 + row) * DI + col * 8);
    float x[8];
    unpack8_bf16(v, x);
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
    a = fmaxf(a, shfl_xor_f(a, 1));
    a = fmaxf(a, shfl_xor_f(a, 2));
    const int e = fp4_scale_exponent(a);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_code(ldexpf(x[j], -e)) << (4 * j);
    if (row < n) {
      *reinterpret_cast<uint32_t*>(k4 + (row0 + row) * (DI / 2) + col * 4) = w;
      if ((col & 3) == 0) ke4[(row0 + row) * (DI / 32) + col / 4] = (uint8_t)(e + 127);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill scoring + selection on E4M3 codes.  Same organisation as the bf16
// prefill kernel: a workgroup owns RT * NW * 32 (query, group) rows of one
// sequence, waves hold their rows' index queries as MFMA B operands, key
// blocks stream through a three-buffer LDS ring filled by direct
// global->LDS loads, and every lane keeps its row's running top-(k-1) list.
// ---------------------------------------------------------------------------
// Ring of 128 x DI-byte key blocks.  One wave instruction fills 1 KiB (lane L
// -> bytes 16L..16L+15): 64 / CPR whole rows of CPR = DI / 16 chunks.  Chunk c
// of row m is stored at chunk position c ^ swz(m) (chosen through the source
// address).  The 64 four-byte banks span 256 bytes, i.e. R = 16 / CPR rows, and
// a fragment read serves 16 consecutive rows at a time; swz(m) = (m / R) % CPR
// gives those 16 rows 16 different 16-byte bank groups.
template <int DI, int NW>
struct KRing8 {
  static constexpr int CPR = DI / 16;
  static constexpr int R = 16 / CPR;                              // rows per 256-byte bank line
  static constexpr int ROWS_PER_INSTR = 64 / CPR;
  static constexpr int INSTR = kBlock / ROWS_PER_INSTR;          // 1 KiB pieces per block
  static constexpr int PER_WAVE = INSTR >= NW ? INSTR / NW : 1;  // loads per loading wave
  static constexpr int LOADERS = INSTR >= NW ? NW : INSTR;       // waves that load
  static_assert(INSTR < NW || INSTR % NW == 0, "block must split evenly over the waves");

  // issue this wave's loads of the key block whose first row is `blk_base` into `buf`
  __device__ static inline void load(const uint8_t* __restrict__ blk_base, uint8_t* buf,
                                     int wave, int lane) {
    // (only small blocks leave waves idle: a branch where every wave loads
    // would rejoin before the fragment reads and cost a wait for all loads)
    if constexpr (INSTR < NW) {
      if (wave >= LOADERS) return;
    }
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      const int m = piece * ROWS_PER_INSTR + lane / CPR;
      const int lc = (lane % CPR) ^ swz(m);
      const uint8_t* src = blk_base + (size_t)m * DI + lc * 16;
      __builtin_amdgcn_global_load_lds(src, buf + piece * 1024, 16, 0, 0);
    }
  }
  __device__ static inline int swz(int m) { return (m / R) % CPR; }
  __device__ static inline uint4 chunk(const uint8_t* buf, int m, int lc) {
    return *reinterpret_cast<const uint4*>(buf + m * DI + ((lc ^ swz(m)) * 16));
  }
  // A fragment of k-step ks for lane half h: logical chunks 4ks + 2h, +1
  // (DI = 32: chunk h and 16 zero bytes)
  __device__ static inline i32x8 frag(const uint8_t* buf, int m, int ks, int h) {
    if constexpr (DI == 32) {
      return as_i32x8(chunk(buf, m, h), make_uint4(0, 0, 0, 0));
    } else {
      return as_i32x8(chunk(buf, m, 4 * ks + 2 * h), chunk(buf, m, 4 * ks + 2 * h + 1));
    }
  }
};

// Ring of 4-bit key blocks: the block's codes (128 x DI/2 bytes, swizzled as in
// KRing8) followed by its exponents (128 x DI/32 bytes, in row order).  Every
// wave issues PER_WAVE code pieces and one exponent piece per block, so all
// waves count the same LOADS loads in flight.
template <int DI, int NW>
struct KRing4 {
  static constexpr int RB = DI / 2;                               // code bytes per key row
  static constexpr int CPR = RB / 16;                             // 16-byte chunks per row
  static constexpr int R = 16 / CPR;                              // rows per 256-byte bank line
  static constexpr int CODE_BYTES = kBlock * RB;
  static constexpr int PIECE = CODE_BYTES / NW < 1024 ? CODE_BYTES / NW : 1024;
  static constexpr int PER_WAVE = CODE_BYTES / PIECE / NW;
  static constexpr int ROWS_PER_PIECE = PIECE / RB;
  static constexpr int XB = DI / 32;                              // exponent bytes per key row
  static constexpr int EXP_PER_WAVE = kBlock * XB / NW;
  // every lane of a wave issues the exponent load (a branch on the lane would
  // rejoin before the next fragment reads, and the compiler would then wait
  // for all the loads in flight): the wave's EXP_PER_WAVE bytes, repeated, fill
  // a 1 KiB region per wave; rows 32w .. 32w + 31 read theirs from the first
  // EXP_PER_WAVE bytes of region w
  static constexpr int EXP_REGION = 1024;
  static constexpr int BYTES = CODE_BYTES + NW * EXP_REGION;
  static constexpr int LOADS = PER_WAVE + 1;
  static_assert(CODE_BYTES % (PIECE * NW) == 0 && EXP_PER_WAVE % 16 == 0 && PIECE % RB == 0,
                "block must split evenly over the waves");

  __device__ static inline void load(const uint8_t* __restrict__ codes,
                                     const uint8_t* __restrict__ exps, uint8_t* buf, int wave,
                                     int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      if (PIECE == 1024 || lane < PIECE / 16) {
        const int m = piece * ROWS_PER_PIECE + lane / CPR;
        const int lc = (lane % CPR) ^ swz(m);
        __builtin_amdgcn_global_load_lds(codes + (size_t)m * RB + lc * 16, buf + piece * PIECE, 16,
                                         0, 0);
      }
    }
    __builtin_amdgcn_global_load_lds(exps + wave * EXP_PER_WAVE + (lane % (EXP_PER_WAVE / 16)) * 16,
                                     buf + CODE_BYTES + wave * EXP_REGION, 16, 0, 0);
  }
  __device__ static inline int swz(int m) { return (m / R) % CPR; }
  // A fragment of k-step ks for lane half h: elements 64ks + 32h .. +31 of row
  // m, logical chunk 2ks + h (DI = 32: chunk 0 for half 0, zeros for half 1)
  __device__ static inline i32x8 frag(const uint8_t* buf, int m, int ks, int h) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (DI > 32 || h == 0) {
      const int lc = DI > 32 ? 2 * ks + h : 0;
      v = *reinterpret_cast<const uint4*>(buf + m * RB + ((lc ^ swz(m)) * 16));
    }
    return as_i32x8(v, make_uint4(0, 0, 0, 0));
  }
  // the XB exponent bytes of row m, byte j = elements 32j .. 32j+31
  __device__ static inline uint32_t exps(const uint8_t* buf, int m) {
    constexpr int ROWS_PER_WAVE = EXP_PER_WAVE / XB;
    const uint8_t* p = buf + CODE_BYTES + (m / ROWS_PER_WAVE) * EXP_REGION + (m % ROWS_PER_WAVE) * XB;
    if constexpr (XB == 4) return *reinterpret_cast<const uint32_t*>(p);
    else if constexpr (XB == 2) return *reinterpret_cast<const uint16_t*>(p);
    else return *p;
  }
};

// E8M0 scale for the A fragment of k-step ks, lane half h, from a row's
// exponent bytes (0, a factor 2^-127, for the zero half when DI = 32)
__device__ inline int k4_scale(uint32_t x, int ks, int h) { return (int)((x >> (8 * (2 * ks + h))) & 255u); }

// B fragment of k-step ks for lane half h from a query's E4M3 codes, in the
// order the MFMA pairs with the A layouts: fp8 keys take 32 contiguous bytes
// per half (both operands use the same assignment); fp4 keys need elements
// 16h .. 16h+15 and 32+16h .. 32+16h+15 of the k-step.
template <int DI, bool K4>
__device__ inline i32x8 q_frag(const uint8_t* src, int ks, int h) {
  uint4 lo, hi = make_uint4(0, 0, 0, 0);
  if constexpr (DI == 32) {
    lo = *reinterpret_cast<const uint4*>(src + h * 16);
  } else if constexpr (K4) {
    lo = *reinterpret_cast<const uint4*>(src + ks * 64 + h * 16);
    hi = *reinterpret_cast<const uint4*>(src + ks * 64 + 32 + h * 16);
  } else {
    lo = *reinterpret_cast<const uint4*>(src + ks * 64 + h * 32);
    hi = *reinterpret_cast<const uint4*>(src + ks * 64 + h * 32 + 16);
  }
  return as_i32x8(lo, hi);
}

constexpr int kFp8ExpLds = 16384;   // key blocks per sequence whose exponents fit on chip

// K4: 4-bit keys (codes k8 = [rows][DI/2], exponents ke = [rows][DI/32]);
// else E4M3 keys (k8 = [rows][DI], ke = one exponent per block index).
template <int DI, bool K4>
struct PrefillKeys {
  using Ring = KRing8<DI, 4>;
  static constexpr int BYTES = kBlock * DI;
  static constexpr int LOADS = Ring::PER_WAVE;
  static constexpr int EXP_LDS = kFp8ExpLds;
};
template <int DI>
struct PrefillKeys<DI, true> {
  using Ring = KRing4<DI, 4>;
  static constexpr int BYTES = Ring::BYTES;
  static constexpr int LOADS = Ring::LOADS;
  static constexpr int EXP_LDS = 1;
};

template <int DI, int RT, int NW, int KCAP, bool K4, bool PAGED>
__global__ __launch_bounds__(NW * 64, 2) void index_select_prefill_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ ke, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, KvMap kv, int G, int nb_max, int qt, int top_k,
    int32_t* __restrict__ sel, float* __restrict__ sel_score) {
  static_assert(RT == 1 || RT == 2, "a lane owns at most one row");
  static_assert(NW == 4, "rings are laid out for four waves");
  using Keys = PrefillKeys<DI, K4>;
  using Ring = typename Keys::Ring;
  constexpr int KS = DI >= 64 ? DI / 64 : 1;   // MFMA k-steps over the index dim
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[Keys::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[Keys::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[Keys::BYTES];
  __shared__ uint8_t kexp[Keys::EXP_LDS];

  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int tile = (int)(gridDim.x - 1 - blockIdx.x);   // latest query tiles first
  const int qa = qoff + tile * qt;
  const int qz = min(qoff + lq, qa + qt);
  if (qa >= qz) return;
  const int p_last = lk - lq + (qz - 1 - qoff);
  const int beta_hi = K4 ? p_last / kBlock : min(p_last / kBlock, kFp8ExpLds);
  const int nrows = (qz - qa) * G;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const bool owner = half < RT;
  const int n_own = (wave * RT + (owner ? half : 0)) * 32 + col;
  const bool own_valid = owner && n_own < nrows;
  const int q_own = qa + n_own / G, g_own = n_own % G;
  const int beta_own = own_valid ? (lk - lq + (q_own - qoff)) / kBlock : 0;
  const int eq_own = own_valid ? (int)qe[(size_t)q_own * G + g_own] - 127 : 0;
  OrderedTopList<KCAP> list;
  list.clear();

  if (beta_hi > 0) {
    // the sequence's key-block exponents (E4M3 keys), staged once
    if constexpr (!K4)
      for (int i = tid; i < beta_hi; i += NW * 64) kexp[i] = ke[kv.block_index(b, i, nb_max)];

    i32x8 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = (wave * RT + rt) * 32 + col;
      const uint8_t* src = q8 + ((size_t)qa * G + min(n, nrows - 1)) * DI;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[rt][ks] = q_frag<DI, K4>(src, ks, half);
        if (n >= nrows) qf[rt][ks] = i32x8{};
      }
    }
    __syncthreads();   // exponents visible; every earlier load has landed

    // issue this wave's loads of key block beta into buf.  Blocks past the
    // last earlier one are clamped to it, and every step issues its loads: a
    // branch around them (or on the page table: PAGED is a template argument)
    // would rejoin before the next fragment reads, and at such a join the
    // compiler loses track of which ring buffer the direct loads in flight
    // write and waits for all of them.
    // A page is read one step before its block's loads are issued, and
    // before the loads of the block in between: the wait for it then covers
    // no younger ring load.
    auto row_of = [&](int beta) __attribute__((always_inline)) {
      const int bc = min(beta, beta_hi - 1);
      return PAGED ? kv.page_uniform(b, bc) * kBlock : (size_t)koff + (size_t)bc * kBlock;
    };
    auto issue = [&](size_t row0, uint8_t* buf) __attribute__((always_inline)) {
      if constexpr (K4) Ring::load(k8 + row0 * (DI / 2), ke + row0 * (DI / 32), buf, wave, lane);
      else Ring::load(k8 + row0 * DI, buf, wave, lane);
    };
    uint32_t pending = 0;   // previous block's score key, inserted during the next block's MFMAs
    int pending_beta = 0;
    // blocks 0 and 1, and block 2 (which step 0 loads again): the loop is
    // entered with loads into all three buffers, as its back edge has them
    size_t next_row = row_of(2);   // the block step `beta` loads: beta + 2
    issue(row_of(0), ring0);
    issue(row_of(1), ring1);
    issue(next_row, ring2);

    auto step = [&](int beta, const uint8_t* rbuf, uint8_t* lbuf) __attribute__((always_inline)) {
      // this wave's pieces of block beta have landed (only beta+1 may be
      // younger); the barrier publishes every wave's pieces and retires the
      // reads of the buffer about to be refilled
      wait_vmcnt<Keys::LOADS>();   // (waits for one step more in steps 0 and 1)
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const size_t row2 = next_row;
      next_row = row_of(beta + 3);
      issue(row2, lbuf);

      // software pipeline: the MFMAs of key tile kt+1 are issued before the
      // row maxima of tile kt are taken, and the previous block's top-k
      // insert runs while tile 0's MFMAs execute
      float rmax[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) rmax[rt] = -INFINITY;
      f32x16 acc[2][RT];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        i32x8 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = Ring::frag(rbuf, kt * 32 + col, ks, half);
        uint32_t kx = 0;
        if constexpr (K4) kx = Ring::exps(rbuf, kt * 32 + col);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[kt & 1][rt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if constexpr (K4)
              acc[kt & 1][rt] = mfma32_k4(a[ks], qf[rt][ks], acc[kt & 1][rt], k4_scale(kx, ks, half));
            else
              acc[kt & 1][rt] = mfma32_fp8(a[ks], qf[rt][ks], acc[kt & 1][rt]);
          }
        if (kt == 0) {
          list.insert(pending, pending_beta);
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 16; ++i) rmax[rt] = fmaxf(rmax[rt], acc[(kt - 1) & 1][rt][i]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) rmax[rt] = fmaxf(rmax[rt], acc[1][rt][i]);
      const float mine = row_tile_max<RT>(rmax, half);
      const float score = ldexpf(mine, eq_own + (K4 ? 0 : (int)kexp[min(beta, beta_hi - 1)] - 127));
      // key 0 is never inserted
      pending = (beta < beta_own && score == score) ? float_order_key(score) : 0u;
      pending_beta = beta;
    };

    // Whole trips of three steps, none of them conditional (a conditional step
    // lets the compiler merge the steps' load code, and it then no longer
    // knows which buffer the loads write).  Steps past the last earlier block
    // score a reloaded copy of it and insert nothing: their beta is at or
    // above every row's own block.
    for (int beta = 0; beta < beta_hi; beta += 3) {
      step(beta, ring0, ring2);
      step(beta + 1, ring1, ring0);
      step(beta + 2, ring2, ring1);
    }
    wait_vmcnt<0>();   // no direct load may still write LDS when the workgroup ends
    list.insert(pending, pending_beta);
  }
  if (own_valid) {
    const size_t o = ((size_t)q_own * G + g_own) * top_k;
    uint64_t keys[KCAP];
    list.to_keys(keys);
    write_selection(keys, top_k - 1, beta_own, top_k, sel + o, sel_score ? sel_score + o : nullptr);
  }
}

// ---------------------------------------------------------------------------
// Decode scoring on E4M3 codes: at most 32 * RT rows per sequence; grid.x = key-block
// segment, grid.y = sequence; wave w computes keys 32w .. 32w+31 of each block.
// Writes S[beta * ld + row] = 2^(eq + ek) * max_j (q8 . k8_j) for the wide top-k.
// ---------------------------------------------------------------------------
// One 128 x DI-byte key block through registers into a padded LDS tile
// (row stride DI + 16 bytes).
template <int DI, int NT>
struct KTileStage8 {
  // a decode scan reads each key once: non-temporal loads
  typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
  static constexpr int kCpr = DI / 16;
  static constexpr int kChunks = kBlock * kCpr;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  static constexpr int kLd = DI + 16;
  uint4 r[kPer];

  __device__ inline void load(const uint8_t* __restrict__ src, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks)
        r[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(
                   src + (size_t)(c / kCpr) * DI + (c % kCpr) * 16)));
    }
  }
  __device__ inline void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks)
        *reinterpret_cast<uint4*>(lds + (c / kCpr) * kLd + (c % kCpr) * 16) = r[i];
    }
  }
};

template <int DI, int SEG, int RT>
__global__ __launch_bounds__(256) void index_score_decode_fp8_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ k8,
    const uint8_t* __restrict__ ke, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, KvMap kv, int G, int nb_max, int r0, int r1,
    float* __restrict__ S, long long ld) {
  constexpr int NT = 256;
  constexpr int KS = DI >= 64 ? DI / 64 : 1;
  constexpr int LD = KTileStage8<DI, NT>::kLd;
  constexpr int NR = 32 * RT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kBlock * LD];
  __shared__ float red[2][4][NR];

  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int qa = max(qoff, r0), qz = min(qoff + lq, r1);
  if (qa >= qz) return;
  const int p_last = lk - lq + (qz - 1 - qoff);
  const int beta_hi = p_last / kBlock;
  const int b0 = (int)blockIdx.x * SEG;
  const int b1 = min(beta_hi, b0 + SEG);
  if (b0 >= b1) return;
  const int nrows = min((qz - qa) * G, NR);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  i32x8 qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = rt * 32 + col;
    const uint8_t* src = q8 + ((size_t)qa * G + n) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[rt][ks] = n < nrows ? q_frag<DI, false>(src, ks, half) : i32x8{};
  }

  KTileStage8<DI, NT> stage;
  stage.load(k8 + kv.block_row(b, koff, b0) * DI, tid);
  stage.store(lds[0], tid);
  __syncthreads();

  // the four waves' partial maxima of block `blk`, scaled by 2^(eq + ek) -> S
  auto finish = [&](int it, int blk) __attribute__((always_inline)) {
    if (wave != 0) return;
    const size_t srow = (size_t)(qa - r0) * G;
    const int ek = (int)ke[kv.block_index(b, blk, nb_max)] - 127;
#pragma unroll
    for (int j = 0; j < (NR + 63) / 64; ++j) {
      const int n = j * 64 + lane;
      if (n < nrows) {
        const float* rr = &red[it & 1][0][0];
        const float m = fmaxf(fmaxf(rr[n], rr[NR + n]), fmaxf(rr[2 * NR + n], rr[3 * NR + n]));
        const int eq = (int)qe[(size_t)qa * G + n] - 127;
        S[(size_t)blk * ld + srow + n] = ldexpf(m, eq + ek);
      }
    }
  };

  for (int beta = b0; beta < b1; ++beta) {
    const int it = beta - b0;
    stage.load(k8 + kv.block_row(b, koff, min(beta + 1, b1 - 1)) * DI, tid);
    if (it > 0) finish(it - 1, beta - 1);
    const uint8_t* arow = lds[it & 1] + (wave * 32 + col) * LD;
    f32x16 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x8 a;
      if constexpr (DI == 32) {
        a = as_i32x8(*reinterpret_cast<const uint4*>(arow + half * 16), make_uint4(0, 0, 0, 0));
      } else {
        a = as_i32x8(*reinterpret_cast<const uint4*>(arow + ks * 64 + half * 32),
                     *reinterpret_cast<const uint4*>(arow + ks * 64 + half * 32 + 16));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_fp8(a, qf[rt][ks], acc[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float m = acc[rt][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, acc[rt][i]);
      m = fmaxf(m, shfl_xor_f(m, 32));
      if (half == 0) red[it & 1][wave][rt * 32 + col] = m;
    }
    stage.store(lds[(it + 1) & 1], tid);
    __syncthreads();
  }
  finish(b1 - 1 - b0, b1 - 1);
}

// ---------------------------------------------------------------------------
// Decode scoring on 4-bit keys without LDS.  A 4-bit key block is 128 x
// (DI/2 + DI/32) bytes, so per-block costs of a shared staging tile (the LDS
// round trip, a barrier, a cross-wave maximum) weigh twice as much as for 8-bit
// keys.  Here each wave scores whole blocks on its own: it loads its MFMA
// fragments straight from global memory, two of its blocks ahead, takes the
// block maximum in registers and writes S[beta * ld + row] = 2^eq * max_j
// (q8 . k_j).  Wave w of a workgroup owns blocks b0 + w, b0 + w + 4, ... of
// the workgroup's SEG, so the four waves stream adjacent blocks together.
// ---------------------------------------------------------------------------
template <int DI>
struct K4BlockFrags {
  // a decode scan reads each key once: non-temporal loads
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  static constexpr int KS = DI >= 64 ? DI / 64 : 1;
  v4u a[4][KS];     // tile kt, k-step ks: elements 64ks + 32h .. +31 of row 32kt + col
  uint32_t x[4];    // the row's exponent bytes, per tile

  __device__ inline void load(const uint8_t* __restrict__ k4, const uint8_t* __restrict__ ke4,
                              size_t row0, int col, int h) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const size_t row = row0 + kt * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (DI > 32 || h == 0)
          a[kt][ks] = __builtin_nontemporal_load(
              reinterpret_cast<const v4u*>(k4 + row * (DI / 2) + (DI > 32 ? (2 * ks + h) * 16 : 0)));
        else
          a[kt][ks] = v4u{0, 0, 0, 0};
      }
      const uint8_t* xp = ke4 + row * (DI / 32);
      if constexpr (DI == 128) x[kt] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(xp));
      else if constexpr (DI == 64) x[kt] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(xp));
      else x[kt] = __builtin_nontemporal_load(xp);
    }
  }
};

template <int DI, int SEG, int RT>
__global__ __launch_bounds__(256) void index_score_decode_k4_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ k4,
    const uint8_t* __restrict__ ke4, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, KvMap kv, int G, int r0, int r1, float* __restrict__ S,
    long long ld) {
  static_assert(SEG % 4 == 0, "whole rounds of four waves");
  constexpr int KS = K4BlockFrags<DI>::KS;
  constexpr int NR = 32 * RT;
  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int qa = max(qoff, r0), qz = min(qoff + lq, r1);
  if (qa >= qz) return;
  const int beta_hi = (lk - lq + (qz - 1 - qoff)) / kBlock;
  const int b0 = (int)blockIdx.x * SEG;
  const int b1 = min(beta_hi, b0 + SEG);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (b0 + wave >= b1) return;
  const int nrows = min((qz - qa) * G, NR);
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  i32x8 qf[RT][KS];
  int eq[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = rt * 32 + col;
    const uint8_t* src = q8 + ((size_t)qa * G + n) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = n < nrows ? q_frag<DI, true>(src, ks, half) : i32x8{};
    eq[rt] = n < nrows ? (int)qe[(size_t)qa * G + n] - 127 : 0;
  }
  const size_t srow = (size_t)(qa - r0) * G;

  auto score = [&](const K4BlockFrags<DI>& f, int beta) __attribute__((always_inline)) {
    float m[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m[rt] = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x8 a = as_i32x8(make_uint4(f.a[kt][ks].x, f.a[kt][ks].y, f.a[kt][ks].z, f.a[kt][ks].w),
                                 make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32_k4(a, qf[rt][ks], acc[rt], k4_scale(f.x[kt], ks, half));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) m[rt] = fmaxf(m[rt], acc[rt][i]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mm = fmaxf(m[rt], shfl_xor_f(m[rt], 32));
      const int n = rt * 32 + col;
      if (half == 0 && n < nrows) S[(size_t)beta * ld + srow + n] = ldexpf(mm, eq[rt]);
    }
  };

  // two fragment sets in flight: this wave's blocks beta and beta + 4
  K4BlockFrags<DI> f0, f1;
  int beta = b0 + wave;
  f0.load(k4, ke4, kv.block_row(b, koff, beta), col, half);
  if (beta + 4 < b1) f1.load(k4, ke4, kv.block_row(b, koff, beta + 4), col, half);
  for (; beta < b1; beta += 8) {
    score(f0, beta);
    if (beta + 8 < b1) f0.load(k4, ke4, kv.block_row(b, koff, beta + 8), col, half);
    if (beta + 4 < b1) {
      score(f1, beta + 4);
      if (beta + 12 < b1) f1.load(k4, ke4, kv.block_row(b, koff, beta + 12), col, half);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Four waves per workgroup: with 64 KiB of LDS two workgroups share a CU, and
// since they are not barrier-locked to each other one's top-k/epilogue VALU
// work overlaps the other's MFMAs (8 waves per workgroup leave one per CU).
constexpr int kFp8RT = 2;
constexpr int kFp8NW = 4;
constexpr int kFp8Rows = kFp8RT * kFp8NW * 32;
constexpr int kFp8DecodeSeg = 8;

int fp8_max_blocks_per_sequence() { return kFp8ExpLds; }
int fp8_prefill_rows_per_wg() { return kFp8Rows; }

template <int DI>
static hipError_t launch_quantize_di(const void* q, const void* k, const int32_t* cu_k, KvMap kv,
                                     int batch, int nb_max, long long q_rows, void* q8, uint8_t* qe,
                                     void* k8, uint8_t* ke, hipStream_t st) {
  if (q_rows > 0) {
    const long long threads = q_rows * (DI / 8);
    hipLaunchKernelGGL((quantize_q_kernel<DI>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, st, (const uint16_t*)q, q_rows, (uint8_t*)q8, qe);
  }
  if (nb_max > 0)
    hipLaunchKernelGGL((quantize_k_kernel<DI>), dim3(nb_max, batch), dim3(256), 0, st,
                       (const uint16_t*)k, cu_k, kv, nb_max, (uint8_t*)k8, ke);
  return hipGetLastError();
}

hipError_t launch_quantize_index_fp8(int DI, const void* q, const void* k, const int32_t* cu_k,
                                     KvMap kv, int batch, int nb_max, long long q_rows, void* q8,
                                     uint8_t* qe, void* k8, uint8_t* ke, hipStream_t st) {
  switch (DI) {
    case 32: return launch_quantize_di<32>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k8, ke, st);
    case 64: return launch_quantize_di<64>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k8, ke, st);
    case 128: return launch_quantize_di<128>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k8, ke, st);
  }
  return hipErrorInvalidValue;
}

template <int DI, int KCAP, bool K4>
static hipError_t launch_prefill8_t(const void* q8, const uint8_t* qe, const void* k8,
                                    const uint8_t* ke, const int32_t* cu_q, const int32_t* cu_k,
                                    KvMap kv, int batch, int G, int nb_max, int max_q_len, int top_k,
                                    int32_t* sel, float* sel_score, hipStream_t st) {
  const int qt = kFp8Rows / G;
  if (qt < 1) return hipErrorInvalidValue;
  dim3 grid((max_q_len + qt - 1) / qt, batch);
  if (kv.table)
    hipLaunchKernelGGL((index_select_prefill_fp8_kernel<DI, kFp8RT, kFp8NW, KCAP, K4, true>), grid,
                       dim3(kFp8NW * 64), 0, st, (const uint8_t*)q8, qe, (const uint8_t*)k8, ke, cu_q,
                       cu_k, kv, G, nb_max, qt, top_k, sel, sel_score);
  else
    hipLaunchKernelGGL((index_select_prefill_fp8_kernel<DI, kFp8RT, kFp8NW, KCAP, K4, false>), grid,
                       dim3(kFp8NW * 64), 0, st, (const uint8_t*)q8, qe, (const uint8_t*)k8, ke, cu_q,
                       cu_k, kv, G, nb_max, qt, top_k, sel, sel_score);
  return hipGetLastError();
}

template <int DI, bool K4>
static hipError_t launch_prefill8_di(const void* q8, const uint8_t* qe, const void* k8,
                                     const uint8_t* ke, const int32_t* cu_q, const int32_t* cu_k,
                                     KvMap kv, int batch, int G, int nb_max, int max_q_len,
                                     int top_k, int32_t* sel, float* sel_score, hipStream_t st) {
  const int km = top_k - 1;
#define MSA_PF8(K) launch_prefill8_t<DI, K, K4>(q8, qe, k8, ke, cu_q, cu_k, kv, batch, G, nb_max, max_q_len, top_k, sel, sel_score, st)
  if (km <= 1) return MSA_PF8(1);
  if (km <= 2) return MSA_PF8(2);
  if (km <= 4) return MSA_PF8(4);
  if (km <= 8) return MSA_PF8(8);
  if (km <= 16) return MSA_PF8(16);
  return MSA_PF8(32);
#undef MSA_PF8
}

hipError_t launch_index_select_prefill_fp8(const void* q8, const uint8_t* qe, const void* k8,
                                           const uint8_t* ke, bool k4, const int32_t* cu_q,
                                           const int32_t* cu_k, KvMap kv, int batch, int G, int DI,
                                           int nb_max, int max_q_len, int top_k, int32_t* sel,
                                           float* sel_score, hipStream_t st) {
#define MSA_PF8DI(D, K) launch_prefill8_di<D, K>(q8, qe, k8, ke, cu_q, cu_k, kv, batch, G, nb_max, max_q_len, top_k, sel, sel_score, st)
  switch (DI) {
    case 32: return k4 ? MSA_PF8DI(32, true) : MSA_PF8DI(32, false);
    case 64: return k4 ? MSA_PF8DI(64, true) : MSA_PF8DI(64, false);
    case 128: return k4 ? MSA_PF8DI(128, true) : MSA_PF8DI(128, false);
  }
#undef MSA_PF8DI
  return hipErrorInvalidValue;
}

// blocks per workgroup: one query row tile leaves each wave little work per
// block, so more, smaller workgroups; several tiles favour longer runs
constexpr int kK4DecodeSeg1 = 8;
constexpr int kK4DecodeSeg = 16;

template <int DI, bool K4>
static hipError_t launch_decode8_di(const void* q8, const uint8_t* qe, const void* k8,
                                    const uint8_t* ke, const int32_t* cu_q, const int32_t* cu_k,
                                    KvMap kv, int batch, int G, int nb_max, int rows, int r0, int r1,
                                    float* S, long long ld, hipStream_t st) {
  if constexpr (K4) {
#define MSA_DEC4(RT, SEG) hipLaunchKernelGGL((index_score_decode_k4_kernel<DI, SEG, RT>), dim3((nb_max + SEG - 1) / SEG, batch), dim3(256), 0, st, (const uint8_t*)q8, qe, (const uint8_t*)k8, ke, cu_q, cu_k, kv, G, r0, r1, S, ld)
    if (rows <= 32) MSA_DEC4(1, kK4DecodeSeg1);
    else if (rows <= 64) MSA_DEC4(2, kK4DecodeSeg);
    else if (rows <= 128) MSA_DEC4(4, kK4DecodeSeg);
    else return hipErrorInvalidValue;
#undef MSA_DEC4
  } else {
    dim3 grid((nb_max + kFp8DecodeSeg - 1) / kFp8DecodeSeg, batch);
#define MSA_DEC8(RT) hipLaunchKernelGGL((index_score_decode_fp8_kernel<DI, kFp8DecodeSeg, RT>), grid, dim3(256), 0, st, (const uint8_t*)q8, qe, (const uint8_t*)k8, ke, cu_q, cu_k, kv, G, nb_max, r0, r1, S, ld)
    if (rows <= 32) MSA_DEC8(1);
    else if (rows <= 64) MSA_DEC8(2);
    else if (rows <= 128) MSA_DEC8(4);
    else return hipErrorInvalidValue;
#undef MSA_DEC8
  }
  return hipGetLastError();
}

hipError_t launch_index_score_decode_fp8(const void* q8, const uint8_t* qe, const void* k8,
                                         const uint8_t* ke, bool k4, const int32_t* cu_q,
                                         const int32_t* cu_k, KvMap kv, int batch, int G, int DI,
                                         int nb_max, int rows, int r0, int r1, float* S,
                                         long long ld, hipStream_t st) {
#define MSA_D8DI(D, K) launch_decode8_di<D, K>(q8, qe, k8, ke, cu_q, cu_k, kv, batch, G, nb_max, rows, r0, r1, S, ld, st)
  switch (DI) {
    case 32: return k4 ? MSA_D8DI(32, true) : MSA_D8DI(32, false);
    case 64: return k4 ? MSA_D8DI(64, true) : MSA_D8DI(64, false);
    case 128: return k4 ? MSA_D8DI(128, true) : MSA_D8DI(128, false);
  }
#undef MSA_D8DI
  return hipErrorInvalidValue;
}

// 4-bit index keys: queries as for the 8-bit path, keys per 32-element group
template <int DI>
static hipError_t launch_quantize_q8k4_di(const void* q, const void* k, const int32_t* cu_k,
                                          KvMap kv, int batch, int nb_max, long long q_rows,
                                          void* q8, uint8_t* qe, void* k4, uint8_t* ke4,
                                          hipStream_t st) {
  if (q_rows > 0) {
    const long long threads = q_rows * (DI / 8);
    hipLaunchKernelGGL((quantize_q_kernel<DI>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, st, (const uint16_t*)q, q_rows, (uint8_t*)q8, qe);
  }
  if (nb_max > 0)
    hipLaunchKernelGGL((quantize_k4_kernel<DI>), dim3(nb_max, batch), dim3(256), 0, st,
                       (const uint16_t*)k, cu_k, kv, (uint8_t*)k4, ke4);
  return hipGetLastError();
}

hipError_t launch_quantize_index_q8k4(int DI, const void* q, const void* k, const int32_t* cu_k,
                                      KvMap kv, int batch, int nb_max, long long q_rows, void* q8,
                                      uint8_t* qe, void* k4, uint8_t* ke4, hipStream_t st) {
  switch (DI) {
    case 32: return launch_quantize_q8k4_di<32>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k4, ke4, st);
    case 64: return launch_quantize_q8k4_di<64>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k4, ke4, st);
    case 128: return launch_quantize_q8k4_di<128>(q, k, cu_k, kv, batch, nb_max, q_rows, q8, qe, k4, ke4, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
