// Index Branch, step 1+2: token scores q_idx . k_idx on bf16 MFMA, max-pooled
// per 128-token KV block.
//
// The Index Branch scores every visible key token with one index-query head
// per GQA group against one shared index-key head, then max-pools the token
// scores to block level (MSA guide, ai-tool-zukan.com/minimax-msa-guide,
// sections "Index BranchとMain Branchの役割分担" and "2段階構造の中身").
//
// Only earlier blocks (beta < beta(p)) are scored: the query's own block is
// always selected whatever its score, so its score is never needed for the
// choice.
//
// Prefill kernel: a workgroup owns the rows (query, group) of a run of
// queries in one sequence and streams the shared index keys block by block
// through LDS; every wave keeps its rows' index queries in registers as the
// MFMA B operand and computes S^T = K * Q^T so that each lane owns one row
// and the block max is a register reduction plus one cross-half exchange.
// The top-k selection is fused (see the kernel).
//
// Decode kernel: few rows per sequence and long contexts, so the key range
// is split over workgroups and the four waves split each block's 128 keys.
// It writes block scores S[beta * ld + row], row = (query - r0) * G + g, for
// the separate wide top-k kernel.
#include "msa_common.h"
#include "topk_common.h"

namespace msa {

// Copy one 128 x DI bf16 index-key block between global memory, registers and
// a padded LDS tile (row stride DI + 8 elements keeps 16-byte reads of 32
// consecutive rows on distinct banks).
template <int DI, int NT>
struct KTileStage {
  static constexpr int kChunks = kBlock * DI / 8;              // 16-byte chunks per block
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  static constexpr int kLd = DI + 8;
  uint4 r[kPer];

  __device__ inline void load(const uint16_t* __restrict__ src, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks) {
        int row = c / (DI / 8), col = c % (DI / 8);
        r[i] = *reinterpret_cast<const uint4*>(src + (size_t)row * DI + col * 8);
      }
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks) {
        int row = c / (DI / 8), col = c % (DI / 8);
        *reinterpret_cast<uint4*>(lds + row * kLd + col * 8) = r[i];
      }
    }
  }
};


// A key block staged in registers as clang vectors (plain values that stay in
// registers even when two stages are live; HIP's uint4 struct does not).  A
// decode scan reads each key once, so the loads are non-temporal.
template <int DI, int NT>
struct KTileRegs {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  static constexpr int kChunks = kBlock * DI / 8;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  static constexpr int kLd = DI + 8;
  v4u r[kPer];
  __device__ inline void load(const uint16_t* __restrict__ src, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks)
        r[i] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(src + (size_t)(c / (DI / 8)) * DI + (c % (DI / 8)) * 8));
    }
  }
  __device__ inline void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks)
        *reinterpret_cast<v4u*>(lds + (c / (DI / 8)) * kLd + (c % (DI / 8)) * 8) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------
// Prefill: scoring fused with the selection.  RT (1 or 2) row tiles of 32 rows
// per wave, NW waves per workgroup; grid.x = query tiles (latest first),
// grid.y = sequence.  After each key block a lane holds the block score of
// one row (lanes 32 * rt .. 32 * rt + 31 own row tile rt) and inserts it into
// that row's running top-(k-1) list (KCAP keys in registers); at the end the
// lane writes the row's selection.  No block-score buffer is needed.
// ---------------------------------------------------------------------------
// Index-key blocks reach LDS by direct global->LDS 16-byte loads: one wave
// instruction fills 1 KiB (lane L -> bytes 16L..16L+15), i.e. 64 / CPR whole
// rows of CPR = DI / 8 chunks.  Rows are not padded; instead chunk c of row m
// is stored at chunk position c ^ swz(m) (the swizzle is applied by choosing
// each lane's source address).  The 64 four-byte banks span 256 bytes, i.e.
// R = 16 / CPR rows (1 for DI = 128), and an A-fragment read serves 16
// consecutive rows at one logical chunk at a time: swz(m) = (m / R) % CPR
// gives those rows 16 different 16-byte bank groups.
template <int DI, int NW>
struct KRing {
  static constexpr int CPR = DI / 8;                  // 16-byte chunks per key row
  static constexpr int R = 16 / CPR;                  // rows per 256-byte bank line
  static constexpr int ROWS_PER_INSTR = 64 / CPR;
  static constexpr int INSTR = kBlock / ROWS_PER_INSTR;   // 1 KiB pieces per block
  static constexpr int PER_WAVE = INSTR / NW;          // loads per wave per block
  static_assert(INSTR % NW == 0, "block must split evenly over the waves");

  // issue this wave's loads of the key block whose first row is `blk_base` into `buf`
  __device__ static inline void load(const uint16_t* __restrict__ blk_base, uint16_t* buf,
                                     int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      const int m = piece * ROWS_PER_INSTR + lane / CPR;
      const int lc = (lane % CPR) ^ swz(m);
      const uint16_t* src = blk_base + (size_t)m * DI + lc * 8;
      __builtin_amdgcn_global_load_lds(src, buf + piece * 512, 16, 0, 0);
    }
  }
  __device__ static inline int swz(int m) { return (m / R) % CPR; }
  // A fragment: row m, logical chunk lc
  __device__ static inline bf16x8 frag(const uint16_t* buf, int m, int lc) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(buf + m * DI + ((lc ^ swz(m)) * 8)));
  }
};

template <int DI, int RT, int NW, int KCAP, bool PAGED>
__global__ __launch_bounds__(NW * 64) void index_select_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int G, int qt,
    int top_k, int32_t* __restrict__ sel, float* __restrict__ sel_score) {
  static_assert(RT == 1 || RT == 2, "a lane owns at most one row");
  using Ring = KRing<DI, NW>;
  constexpr int KS = DI / 16;          // MFMA k-steps over the index dim
  // three key-block buffers: block beta is scored while beta+1 and beta+2 load.
  // Separate arrays named statically in each step let the compiler see that
  // the direct loads into one buffer cannot alias reads of another, so it
  // does not drain the younger loads before reading.
  __shared__ __attribute__((aligned(1024))) uint16_t ring0[kBlock * DI];
  __shared__ __attribute__((aligned(1024))) uint16_t ring1[kBlock * DI];
  __shared__ __attribute__((aligned(1024))) uint16_t ring2[kBlock * DI];

  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  // later query tiles score more blocks (causal triangle): dispatch them first
  const int tile = (int)(gridDim.x - 1 - blockIdx.x);
  const int qa = qoff + tile * qt;
  const int qz = min(qoff + lq, qa + qt);
  if (qa >= qz) return;
  const int p_last = lk - lq + (qz - 1 - qoff);
  const int beta_hi = p_last / kBlock;   // blocks 0 .. beta_hi-1 are earlier blocks for the last row
  const int nrows = (qz - qa) * G;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // the row this lane selects for
  const bool owner = half < RT;
  const int n_own = (wave * RT + (owner ? half : 0)) * 32 + col;
  const bool own_valid = owner && n_own < nrows;
  const int q_own = qa + n_own / G, g_own = n_own % G;
  const int beta_own = own_valid ? (lk - lq + (q_own - qoff)) / kBlock : 0;
  OrderedTopList<KCAP> list;
  list.clear();

  if (beta_hi > 0) {
    // index queries of this wave's rows, as MFMA B operands (k = 16ks + 8half + e)
    bf16x8 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = (wave * RT + rt) * 32 + col;
      const uint16_t* src = q_idx + ((size_t)qa * G + min(n, nrows - 1)) * DI;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = *reinterpret_cast<const uint4*>(src + ks * 16 + half * 8);
        qf[rt][ks] = as_bf16x8(n < nrows ? v : make_uint4(0, 0, 0, 0));
      }
    }

    // First row of key block beta, clamped to the last earlier block.  PAGED
    // is a template argument: a branch on the table here would join right
    // before the next fragment reads, and at such a join the compiler loses
    // track of which ring buffer the direct loads in flight write, so it
    // waits for all of them.  A page is read one step before its block's
    // loads are issued, and before the loads of the block in between: the
    // wait for it then covers no younger ring load.
    auto row_of = [&](int beta) __attribute__((always_inline)) {
      const int bc = min(beta, beta_hi - 1);
      return PAGED ? kv.page_uniform(b, bc) * kBlock : (size_t)koff + (size_t)bc * kBlock;
    };
    uint32_t pending = 0;   // previous block's score key, inserted during the next block's MFMAs
    int pending_beta = 0;
    // blocks 0 and 1, and block 2 (which step 0 loads again): every step
    // issues its loads, clamped to the last block past the end (a branch
    // around them would rejoin before the next fragment reads, and there the
    // compiler would wait for every load in flight), and the loop is entered
    // with loads into all three buffers, as its back edge has them
    size_t next_row = row_of(2);   // the block step `beta` loads: beta + 2
    Ring::load(k_idx + row_of(0) * DI, ring0, wave, lane);
    Ring::load(k_idx + row_of(1) * DI, ring1, wave, lane);
    Ring::load(k_idx + next_row * DI, ring2, wave, lane);

    // score block beta from `rbuf`; first start loading block beta+2 into `lbuf`
    auto step = [&](int beta, const uint16_t* rbuf, uint16_t* lbuf) __attribute__((always_inline)) {
      // this wave's pieces of block beta have landed (only block beta+1 may be
      // younger); the barrier makes every wave's pieces visible and retires
      // the buffer read in the previous step (a plain __syncthreads would also
      // drain the younger block's loads)
      wait_vmcnt<Ring::PER_WAVE>();   // (waits for one step more in steps 0 and 1)
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads are done
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const size_t row2 = next_row;
      next_row = row_of(beta + 3);
      Ring::load(k_idx + row2 * DI, lbuf, wave, lane);

      // the previous block's top-k insert runs while this block's first
      // fragments load
      list.insert(pending, pending_beta);
      float rmax[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) rmax[rt] = -INFINITY;
      // the block's 4 * KS fragments flow through a window of DEPTH registers:
      // a slot is refilled right after its MFMAs issue, so DEPTH fragments are
      // in flight.  Key tiles are scored in pairs, k-step by k-step, into two
      // accumulator sets (fragment f: pair f / (2 KS), k-step (f % (2 KS)) / 2,
      // tile 2 pair + f % 2), so each accumulator's next MFMA comes 2 * RT
      // MFMAs after its last one (RT independent chains per tile would leave
      // dependent MFMAs back to back)
      constexpr int NF = 4 * KS, DEPTH = 4;
      auto kt_of = [](int f) { return 2 * (f / (2 * KS)) + (f & 1); };
      auto ks_of = [](int f) { return (f % (2 * KS)) >> 1; };
      bf16x8 win[DEPTH];
#pragma unroll
      for (int f = 0; f < DEPTH; ++f) win[f] = Ring::frag(rbuf, kt_of(f) * 32 + col, 2 * ks_of(f) + half);
      f32x16 acc[2][RT];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int ks = ks_of(f), set = f & 1;
        if (ks == 0) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[set][rt] = f32x16{};
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[set][rt] = mfma32(win[f % DEPTH], qf[rt][ks], acc[set][rt]);
        if (f + DEPTH < NF)
          win[f % DEPTH] = Ring::frag(rbuf, kt_of(f + DEPTH) * 32 + col, 2 * ks_of(f + DEPTH) + half);
        if (ks == KS - 1) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 16; ++i) rmax[rt] = fmaxf(rmax[rt], acc[set][rt][i]);
          // the tile's max is taken here, so its accumulators die here
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) asm volatile("" : "+v"(rmax[rt]));
        }
        __builtin_amdgcn_sched_barrier(0);   // keep this order: the window is the schedule
      }
      const float mine = row_tile_max<RT>(rmax, half);
      // key 0 is never inserted
      pending = (beta < beta_own && mine == mine) ? float_order_key(mine) : 0u;
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
// Decode-shaped steps: at most 32 * RT (query, group) rows per sequence (RT = 1,
// 2, 4 row tiles); grid.x = key-block segment, grid.y = sequence.  Wave w
// computes keys 32w .. 32w+31 of every block in the segment for all rows.
// ---------------------------------------------------------------------------
template <int DI, int SEG, int RT>
__global__ __launch_bounds__(256) void index_score_decode_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int G, int r0,
    int r1, float* __restrict__ S, long long ld) {
  constexpr int NT = 256;
  constexpr int KS = DI / 16;
  constexpr int LD = DI + 8;
  constexpr int NR = 32 * RT;              // (query, group) rows of one sequence, at most
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kBlock * LD];
  __shared__ float red[2][4][NR];

  const int b = blockIdx.y;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  int qa = max(qoff, r0), qz = min(qoff + lq, r1);
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

  // row tile rt holds rows 32 rt .. 32 rt + 31 as the MFMA B operand (lane <-> row)
  bf16x8 qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = rt * 32 + col;
    const uint16_t* src = q_idx + ((size_t)qa * G + n) * DI;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < nrows) v = *reinterpret_cast<const uint4*>(src + ks * 16 + half * 8);
      qf[rt][ks] = as_bf16x8(v);
    }
  }

  // two key blocks in flight: while block beta is scored from LDS, block beta+1
  // (issued one step earlier) and block beta+2 (issued now) are loading.  The
  // block loop is unrolled over the segment so that every stage index is a
  // compile-time constant (the stage registers then never touch scratch).
  KTileRegs<DI, NT> st[2];
  st[0].load(k_idx + kv.block_row(b, koff, b0) * DI, tid);
  st[0].store(lds[0], tid);
  st[1].load(k_idx + kv.block_row(b, koff, min(b0 + 1, b1 - 1)) * DI, tid);
  __syncthreads();

  // the four waves' partial maxima of block `blk` (kept in red[it & 1]) -> S
  auto finish = [&](int it, int blk) __attribute__((always_inline)) {
    if (wave != 0) return;
    const size_t srow = (size_t)(qa - r0) * G;
#pragma unroll
    for (int j = 0; j < (NR + 63) / 64; ++j) {
      const int n = j * 64 + lane;
      if (n < nrows) {
        const float* rr = &red[it & 1][0][0];
        const float m = fmaxf(fmaxf(rr[n], rr[NR + n]), fmaxf(rr[2 * NR + n], rr[3 * NR + n]));
        S[(size_t)blk * ld + srow + n] = m;
      }
    }
  };

#pragma unroll
  for (int it = 0; it < SEG; ++it) {
    const int beta = b0 + it;
    if (beta < b1) {
      // stage it&1 held block beta (now in LDS): it takes block beta+2
      st[it & 1].load(k_idx + kv.block_row(b, koff, min(beta + 2, b1 - 1)) * DI, tid);
      if (it > 0) finish(it - 1, beta - 1);
      const uint16_t* kt_lds = lds[it & 1];
      f32x16 acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(kt_lds + (wave * 32 + col) * LD + ks * 16 + half * 8));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma32(a, qf[rt][ks], acc[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float m = acc[rt][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, acc[rt][i]);
        m = fmaxf(m, shfl_xor_f(m, 32));
        if (half == 0) red[it & 1][wave][rt * 32 + col] = m;
      }
      // stage (it+1)&1 holds block beta+1
      if (beta + 1 < b1) st[(it + 1) & 1].store(lds[(it + 1) & 1], tid);
      __syncthreads();
    }
  }
  finish(b1 - 1 - b0, b1 - 1);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
constexpr int kPrefillRT = 2;
constexpr int kPrefillNW = 8;
constexpr int kPrefillRows = kPrefillRT * kPrefillNW * 32;   // rows per workgroup
constexpr int kDecodeSeg = 4;

int prefill_rows_per_wg() { return kPrefillRows; }

template <int DI, int KCAP>
static hipError_t launch_prefill_t(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                                   const int32_t* cu_k, KvMap kv, int batch, int G, int max_q_len,
                                   int top_k, int32_t* sel, float* sel_score, hipStream_t st) {
  const int qt = kPrefillRows / G;
  if (qt < 1) return hipErrorInvalidValue;
  dim3 grid((max_q_len + qt - 1) / qt, batch);
  if (kv.table)
    hipLaunchKernelGGL((index_select_prefill_kernel<DI, kPrefillRT, kPrefillNW, KCAP, true>), grid,
                       dim3(kPrefillNW * 64), 0, st, (const uint16_t*)q_idx, (const uint16_t*)k_idx,
                       cu_q, cu_k, kv, G, qt, top_k, sel, sel_score);
  else
    hipLaunchKernelGGL((index_select_prefill_kernel<DI, kPrefillRT, kPrefillNW, KCAP, false>), grid,
                       dim3(kPrefillNW * 64), 0, st, (const uint16_t*)q_idx, (const uint16_t*)k_idx,
                       cu_q, cu_k, kv, G, qt, top_k, sel, sel_score);
  return hipGetLastError();
}

template <int DI>
static hipError_t launch_prefill_di(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                                    const int32_t* cu_k, KvMap kv, int batch, int G, int max_q_len,
                                    int top_k, int32_t* sel, float* sel_score, hipStream_t st) {
  const int km = top_k - 1;
#define MSA_PF(K) launch_prefill_t<DI, K>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, max_q_len, top_k, sel, sel_score, st)
  if (km <= 1) return MSA_PF(1);
  if (km <= 2) return MSA_PF(2);
  if (km <= 4) return MSA_PF(4);
  if (km <= 8) return MSA_PF(8);
  if (km <= 16) return MSA_PF(16);
  return MSA_PF(32);
#undef MSA_PF
}

hipError_t launch_index_select_prefill(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                                       const int32_t* cu_k, KvMap kv, int batch, int G, int DI,
                                       int max_q_len, int top_k, int32_t* sel, float* sel_score,
                                       hipStream_t st) {
  switch (DI) {
    case 32: return launch_prefill_di<32>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, max_q_len, top_k, sel, sel_score, st);
    case 64: return launch_prefill_di<64>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, max_q_len, top_k, sel, sel_score, st);
    case 128: return launch_prefill_di<128>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, max_q_len, top_k, sel, sel_score, st);
  }
  return hipErrorInvalidValue;
}

template <int DI>
static hipError_t launch_decode_di(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                                   const int32_t* cu_k, KvMap kv, int batch, int G, int nb_max,
                                   int rows, int r0, int r1, float* S, long long ld, hipStream_t st) {
  dim3 grid((nb_max + kDecodeSeg - 1) / kDecodeSeg, batch);
#define MSA_DEC(RT) hipLaunchKernelGGL((index_score_decode_kernel<DI, kDecodeSeg, RT>), grid, dim3(256), 0, st, (const uint16_t*)q_idx, (const uint16_t*)k_idx, cu_q, cu_k, kv, G, r0, r1, S, ld)
  if (rows <= 32) MSA_DEC(1);
  else if (rows <= 64) MSA_DEC(2);
  else if (rows <= 128) MSA_DEC(4);
  else return hipErrorInvalidValue;
#undef MSA_DEC
  return hipGetLastError();
}

hipError_t launch_index_score_decode(const void* q_idx, const void* k_idx, const int32_t* cu_q,
                                     const int32_t* cu_k, KvMap kv, int batch, int G, int DI,
                                     int nb_max, int rows, int r0, int r1, float* S, long long ld,
                                     hipStream_t st) {
  switch (DI) {
    case 32: return launch_decode_di<32>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, nb_max, rows, r0, r1, S, ld, st);
    case 64: return launch_decode_di<64>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, nb_max, rows, r0, r1, S, ld, st);
    case 128: return launch_decode_di<128>(q_idx, k_idx, cu_q, cu_k, kv, batch, G, nb_max, rows, r0, r1, S, ld, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
