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
// Partials are laid out [query][group][slot][head-in-group][d], so the
// heads of one (query, slot) form one contiguous run of HPG * D floats.
//
// Q8: the Main Branch's inputs are E4M3 codes with power-of-two scales (one per
// (query row, head) of q, one per (block, KV head) of k and v); KV4 (with Q8):
// k and v are E2M1 codes with one power-of-two scale per 32 elements of every
// (key, KV head) row.  Q fragments and the staged K/V are dequantised on
// load, exactly, into the same bf16 operands, so everything after the loads
// is the bf16 path.
//
// merge_partials_kernel: per (query, head) the log-sum-exp merge of its
// partials -- M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L -- which equals one softmax over the union of
// the selected keys; lse = (M + log2 L) * ln 2.
//
// Compact partials (an option of the lists path; fp32 is the default): the
// same partial as (w, E, o) with w = m + log2 l (the block's log-sum-exp in
// log2 units), E the exponent with max_d |O_d| / l in [2^(E-1), 2^E), and
// o = O / l * 2^-E in fp16 (|o| < 1, 11 significant bits): 2 * D + 8 bytes
// per row instead of 4 * D + 8.  The merge is then M = max w_s,
// L = sum 2^(w_s - M), out = 2^Emax * sum o_s 2^(w_s - M + E_s - Emax) / L.
#include "fp8_common.h"
#include "msa_common.h"

namespace msa {

// One 32-row tile's queries: the Q fragments (MFMA B operand, lane <-> query
// row), the destination partial row (-1 for padding) and the query position.
template <int D, int HPG, bool Q8>
struct TileQ {
  static constexpr int KS = D / 16;
  bf16x8 qf[KS];
  int drow;   // (((r - r0) * G + g) * top_k + slot) * HPG + head-in-group; spare row if padding
  int p;      // query position (for the causal mask)
  bool ok;

  // `ent` is the tile's list entry for this lane's query (-1: none).  Every
  // load is issued unconditionally (padding lanes read row 0 and zero it),
  // so the compiler can count outstanding memory operations exactly.
  __device__ inline void load(const void* __restrict__ q, const uint8_t* __restrict__ qe, int ent,
                              int r0, int r1, int top_k, int Hq, int G, int g, int hl, int half,
                              int pshift, int spare_row) {
    const int r = ent >> kEntrySlotBits, slot = ent & ((1 << kEntrySlotBits) - 1);
    ok = ent >= 0 && r >= r0 && r < r1 && slot < top_k;
    drow = ok ? ((((r - r0) * G + g) * top_k + slot) * HPG + hl) : spare_row;
    p = ok ? r + pshift : 0x7fffffff;
    const size_t qrow = (size_t)(ok ? r : 0) * Hq + g * HPG + hl;
    if constexpr (Q8) {
      const uint8_t* qs = static_cast<const uint8_t*>(q) + qrow * D + half * 8;
      const int e = (int)qe[qrow] - 127;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint2 x = *reinterpret_cast<const uint2*>(qs + ks * 16);
        x = ok ? x : make_uint2(0, 0);
        qf[ks] = as_bf16x8(dequant8_bf16(x, e));
      }
    } else {
      const uint16_t* qs = static_cast<const uint16_t*>(q) + qrow * D + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 x = *reinterpret_cast<const uint4*>(qs + ks * 16);
        x = ok ? x : make_uint4(0, 0, 0, 0);
        qf[ks] = as_bf16x8(x);
      }
    }
  }
};

// list entry of position e of this item's range [.., e1), or -1 past its end
// (the load is clamped into the range so it is always issued)
__device__ inline int tile_entry(const int32_t* __restrict__ entries, int e, int e1) {
  const int v = entries[min(e, e1 - 1)];
  return e < e1 ? v : -1;
}

// First index in [lo, hi) of a sorted int array whose value is >= key, found
// by one wave with 64-way splitting (a few dependent loads instead of log2 n).
__device__ inline int wave_lower_bound(const int32_t* __restrict__ a, int lo, int hi, int key,
                                       int lane) {
  while (hi - lo > 64) {
    const int span = hi - lo;
    const int pos = lo + (int)(((long long)span * lane) >> 6);
    const bool below = a[pos] < key;
    const unsigned long long m = __ballot(below);
    const int nb = __popcll(m);             // samples below the key (a prefix of the lanes)
    const int nlo = nb == 0 ? lo : lo + (int)(((long long)span * (nb - 1)) >> 6) + 1;
    const int nhi = nb == 64 ? hi : lo + (int)(((long long)span * nb) >> 6);
    lo = nlo;
    hi = max(nhi, nlo);
  }
  const int pos = lo + lane;
  const bool below = pos < hi && a[pos] < key;
  return lo + __popcll(__ballot(below));
}

// One (block, sequence, group) item: stage its K/V block, then attend every
// gathered query of this pass.  Called by the whole workgroup; every exit is
// workgroup-uniform.
template <int D, int HPG, bool Q8, bool KV4, bool COMPACT>
__device__ __forceinline__ void attend_item(
    long long item, const void* __restrict__ q, const void* __restrict__ k,
    const void* __restrict__ v, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ ke,
    const uint8_t* __restrict__ ve, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, KvMap kv, int batch, int G, int Hq, int top_k, int nb_max,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ entries, int r0, int r1,
    int total_q, float scale_log2, void* __restrict__ part_acc, float2* __restrict__ part_ml,
    int spare_row, uint16_t* Ks, uint16_t* Vt, int* range) {
  constexpr int QPT = 32 / HPG;   // queries per 32-row tile
  constexpr int KS = D / 16;      // k-steps of Q.K over the head dim
  constexpr int DT = D / 32;      // 32-row tiles of the transposed output
  constexpr int LDK = D + 8;
  constexpr int LDV = kBlock + 4;   // 66-dword rows: 8-byte reads of 16 rows hit distinct banks

  const int BG = batch * G;
  const int beta = (int)(item / BG);
  const int bg = (int)(item % BG);
  const int b = bg / G, g = bg % G;
  const int koff = cu_k[b], lk = cu_k[b + 1] - koff;
  const int qoff = cu_q[b], lq = cu_q[b + 1] - qoff;
  if (beta * kBlock >= lk) return;
  const size_t u = (size_t)bg * nb_max + beta;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // this pass's rows [r0, r1) are a contiguous run of the ascending list
    const int lo = offsets[u], hi = offsets[u + 1];
    const int a = (r0 == 0) ? lo : wave_lower_bound(entries, lo, hi, r0 << kEntrySlotBits, tid);
    const int z = (r1 >= total_q) ? hi : wave_lower_bound(entries, a, hi, r1 << kEntrySlotBits, tid);
    if (tid == 0) {
      range[0] = a;
      range[1] = z;
    }
  }
  __syncthreads();
  const int e0 = range[0], e1 = range[1];
  if (e0 >= e1) return;

  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int qi = col / HPG, hl = col % HPG;
  const int ntiles = (e1 - e0 + QPT - 1) / QPT;
  const int pshift = lk - lq - qoff;   // position of global row r is r + pshift

  // Software pipeline over this wave's tiles t = wave, wave + 4, ...: list
  // entries two tiles ahead and Q one tile ahead, ping-ponging two tile
  // buffers; every load is issued before the current tile's stores (stores
  // share the memory counter on this GPU, so a load issued after them could
  // not be waited for on its own).
  TileQ<D, HPG, Q8> A, B;
  A.load(q, qe, tile_entry(entries, e0 + wave * QPT + qi, e1), r0, r1, top_k, Hq, G, g, hl, half,
         pshift, spare_row);
  int ent_next = tile_entry(entries, e0 + (wave + 4) * QPT + qi, e1);

  // stage the block: K as [key][d], V as [d][key]; keys past the sequence are zero.
  // K: consecutive threads take consecutive 16-byte chunks of a key row.
  // V: consecutive threads take consecutive keys, so the transposed 2-byte LDS
  //    writes of a wave land on consecutive addresses.
  const int kb = beta * kBlock;
  const size_t row0 = kv.block_row(b, koff, beta);   // first cache row of the block
  if constexpr (KV4) {
    // 32 codes (16 bytes) and their exponent per chunk: chunk gc of key row
    // `key` holds elements 32 gc .. 32 gc + 31
    const uint8_t* k4 = static_cast<const uint8_t*>(k);
    const uint8_t* v4 = static_cast<const uint8_t*>(v);
    for (int c = tid; c < kBlock * D / 32; c += 256) {
      const int key = c / (D / 32), gc = c % (D / 32);
      const size_t rr = (row0 + key) * G + g;
      uint4 kk = make_uint4(0, 0, 0, 0);
      int e = 0;
      if (kb + key < lk) {
        kk = *reinterpret_cast<const uint4*>(k4 + rr * (D / 2) + gc * 16);
        e = (int)ke[rr * (D / 32) + gc] - 127;
      }
      uint16_t* dst = Ks + key * LDK + gc * 32;
      *reinterpret_cast<uint4*>(dst) = dequant4_bf16(kk.x, e);
      *reinterpret_cast<uint4*>(dst + 8) = dequant4_bf16(kk.y, e);
      *reinterpret_cast<uint4*>(dst + 16) = dequant4_bf16(kk.z, e);
      *reinterpret_cast<uint4*>(dst + 24) = dequant4_bf16(kk.w, e);
    }
    for (int c = tid; c < kBlock * D / 32; c += 256) {
      const int key = c % kBlock, gc = c / kBlock;
      const size_t rr = (row0 + key) * G + g;
      uint4 vv = make_uint4(0, 0, 0, 0);
      int e = 0;
      if (kb + key < lk) {
        vv = *reinterpret_cast<const uint4*>(v4 + rr * (D / 2) + gc * 16);
        e = (int)ve[rr * (D / 32) + gc] - 127;
      }
      const uint4 d0 = dequant4_bf16(vv.x, e), d1 = dequant4_bf16(vv.y, e);
      const uint4 d2 = dequant4_bf16(vv.z, e), d3 = dequant4_bf16(vv.w, e);
      const uint32_t vw[16] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w,
                               d2.x, d2.y, d2.z, d2.w, d3.x, d3.y, d3.z, d3.w};
#pragma unroll
      for (int i = 0; i < 32; ++i)
        Vt[(gc * 32 + i) * LDV + key] = (uint16_t)(vw[i >> 1] >> (16 * (i & 1)));
    }
  } else if constexpr (Q8) {
    // 16 codes per 16-byte chunk, dequantised with the block's exponents
    const size_t xi = kv.block_index(b, beta, nb_max) * G + g;
    const int kexp = (int)ke[xi] - 127, vexp = (int)ve[xi] - 127;
    const uint8_t* k8 = static_cast<const uint8_t*>(k);
    const uint8_t* v8 = static_cast<const uint8_t*>(v);
    for (int c = tid; c < kBlock * D / 16; c += 256) {
      const int key = c / (D / 16), dc = c % (D / 16);
      uint4 kk = make_uint4(0, 0, 0, 0);
      if (kb + key < lk) kk = *reinterpret_cast<const uint4*>(k8 + ((row0 + key) * G + g) * D + dc * 16);
      *reinterpret_cast<uint4*>(Ks + key * LDK + dc * 16) = dequant8_bf16(make_uint2(kk.x, kk.y), kexp);
      *reinterpret_cast<uint4*>(Ks + key * LDK + dc * 16 + 8) = dequant8_bf16(make_uint2(kk.z, kk.w), kexp);
    }
    for (int c = tid; c < kBlock * D / 16; c += 256) {
      const int key = c % kBlock, dc = c / kBlock;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (kb + key < lk) vv = *reinterpret_cast<const uint4*>(v8 + ((row0 + key) * G + g) * D + dc * 16);
      const uint4 lo = dequant8_bf16(make_uint2(vv.x, vv.y), vexp);
      const uint4 hi = dequant8_bf16(make_uint2(vv.z, vv.w), vexp);
      const uint32_t vw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int i = 0; i < 16; ++i)
        Vt[(dc * 16 + i) * LDV + key] = (uint16_t)(vw[i >> 1] >> (16 * (i & 1)));
    }
  } else {
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    for (int c = tid; c < kBlock * D / 8; c += 256) {
      const int key = c / (D / 8), dc = c % (D / 8);
      uint4 kk = make_uint4(0, 0, 0, 0);
      if (kb + key < lk) kk = *reinterpret_cast<const uint4*>(k16 + ((row0 + key) * G + g) * D + dc * 8);
      *reinterpret_cast<uint4*>(Ks + key * LDK + dc * 8) = kk;
    }
    for (int c = tid; c < kBlock * D / 8; c += 256) {
      const int key = c % kBlock, dc = c / kBlock;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (kb + key < lk) vv = *reinterpret_cast<const uint4*>(v16 + ((row0 + key) * G + g) * D + dc * 8);
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        Vt[(dc * 8 + i) * LDV + key] = (uint16_t)(vw[i >> 1] >> (16 * (i & 1)));
    }
  }
  __syncthreads();


  auto tile = [&](const TileQ<D, HPG, Q8>& T) __attribute__((always_inline)) {
    // The block's K/V fragments do not change across tiles; an opaque zero
    // offset keeps their LDS reads inside the loop instead of letting the
    // compiler hoist all of them into (spilled) registers.
    int lo = 0;
    asm volatile("" : "+v"(lo));
    const uint16_t* Kl = Ks + lo;
    const uint16_t* Vl = Vt + lo;
    // S^T = K * Q^T: lane <-> query row, registers <-> keys
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Kl + (kt * 32 + col) * LDK + ks * 16 + half * 8));
        sacc[kt] = mfma32(a, T.qf[ks], sacc[kt]);
      }
    }
    const int drow = T.drow, p = T.p;

    // softmax over this block's keys for the lane's query row, in log2 units:
    // m = c * max(s), P = 2^(c*s - m) with c = scale * log2(e) > 0
    const bool partial = kb + kBlock - 1 > p;   // some keys lie after the query
    if (partial) {
      // key kb + kt*32 + 8(i/4) + 4half + i%4 is after the query when its
      // constant part exceeds p - kb - 4half
      const int pr = p - kb - 4 * half;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + 8 * (i >> 2) + (i & 3) > pr) sacc[kt][i] = -INFINITY;
    }
    float mr = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mr = fmaxf(mr, sacc[kt][i]);
    mr = fmaxf(mr, shfl_xor_f(mr, 32));
    const float m = mr * scale_log2;
    const float nm = (mr == -INFINITY) ? 0.f : -m;
    float l = 0.f;
    uint4 pk[8];   // P as bf16, MFMA B operand of O^T = V^T * P^T (k-step 2kt + s2)
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

    // O^T = V^T * P^T: lane <-> query row, register i <-> d = 32dt + 8(i/4) + 4half + i%4
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 pb = as_bf16x8(pk[ks]);
      const int kt = ks >> 1, s2 = ks & 1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = Vl + (dt * 32 + col) * LDV + kt * 32 + 16 * s2 + 4 * half;
        uint2 lo = *reinterpret_cast<const uint2*>(vr);
        uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        const bf16x8 va = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        oacc[dt] = mfma32(va, pb, oacc[dt]);
      }
    }

    // write the partial (m, l, O) of the lane's row: stores of 4 consecutive d
    // (padding lanes write the spare row; stores are unconditional for the
    // same exact-counting reason as the loads; both lane halves hold the
    // row's m and l and write the same value)
    if constexpr (COMPACT) {
      // the row's largest |O_d| (this lane holds half of the row's d, its
      // partner lane ^ 32 the other half), then (w, E) and fp16 O / l * 2^-E
      float a = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(oacc[dt][i]));
      a = fmaxf(a, shfl_xor_f(a, 32));
      const float inv_l = l > 0.f ? 1.f / l : 0.f;
      int E = 0;
      (void)frexpf(a * inv_l, &E);
      part_ml[drow] = make_float2(m + log2f(l), (float)E);
      // O / l first (no larger than the largest |v|), then the exact power-of-two
      // scaling into (-1, 1]: no intermediate overflows whatever E is
      auto sc = [&](float x) __attribute__((always_inline)) { return ldexpf(x * inv_l, -E); };
      // A lane holds its row's d = 32 dt + 8 j + 4 half + (0..3), j = 0..3.  For each
      // 16-value run 32 dt + 16 m the two lane halves trade one 4-value group, so that
      // half 0 holds d 0..7 and half 1 holds d 8..15 of the run: every store is then
      // 16 contiguous bytes per lane (32 per row), as for fp32 partials.
      uint16_t* dst = static_cast<uint16_t*>(part_acc) + (size_t)drow * D + 8 * half;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int i = 8 * m;
          // group j = 2m: d 16m + 4 half + 0..3; group j = 2m + 1: d 16m + 8 + 4 half + 0..3
          const uint32_t a0 = pack2_f16(sc(oacc[dt][i]), sc(oacc[dt][i + 1]));
          const uint32_t a1 = pack2_f16(sc(oacc[dt][i + 2]), sc(oacc[dt][i + 3]));
          const uint32_t b0 = pack2_f16(sc(oacc[dt][i + 4]), sc(oacc[dt][i + 5]));
          const uint32_t b1 = pack2_f16(sc(oacc[dt][i + 6]), sc(oacc[dt][i + 7]));
          // half 0 receives half 1's group 2m (d 16m + 4..7), half 1 receives half 0's
          // group 2m + 1 (d 16m + 8..11)
          const uint2 s0 = permlane32_swap_u32(a0, b0);
          const uint2 s1 = permlane32_swap_u32(a1, b1);
          const uint4 v = half == 0 ? make_uint4(a0, a1, s0.y, s1.y) : make_uint4(s0.x, s1.x, b0, b1);
          *reinterpret_cast<uint4*>(dst + dt * 32 + 16 * m) = v;
        }
    } else {
      part_ml[drow] = make_float2(m, l);
      float* dst = static_cast<float*>(part_acc) + (size_t)drow * D + 4 * half;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(dst + dt * 32 + 8 * j) =
              make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
    }
  };

  for (int t = wave; t < ntiles; t += 8) {
    {
      const int ea = tile_entry(entries, e0 + (t + 8) * QPT + qi, e1);
      B.load(q, qe, ent_next, r0, r1, top_k, Hq, G, g, hl, half, pshift, spare_row);
      ent_next = ea;
      tile(A);
    }
    if (t + 4 >= ntiles) break;
    {
      const int ea = tile_entry(entries, e0 + (t + 12) * QPT + qi, e1);
      A.load(q, qe, ent_next, r0, r1, top_k, Hq, G, g, hl, half, pshift, spare_row);
      ent_next = ea;
      tile(B);
    }
  }
}

// Items in block-major order (blocks that most queries select start first).
// items_per_wg == 1: one item per workgroup.  items_per_wg in 2..64 (sparse
// selections, e.g. decode): the workgroup finds which of its items have any
// query with one coalesced load and processes only those.
template <int D, int HPG, bool Q8, bool KV4, bool COMPACT>
__global__ __launch_bounds__(256, 2) void attend_blocks_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint8_t* __restrict__ qe, const uint8_t* __restrict__ ke, const uint8_t* __restrict__ ve,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch, int G,
    int Hq, int top_k, int nb_max, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ entries, int r0, int r1, int total_q, float scale_log2,
    void* __restrict__ part_acc, float2* __restrict__ part_ml, int spare_row, int items_per_wg) {
  constexpr int LDK = D + 8;
  constexpr int LDV = kBlock + 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlock * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LDV];
  __shared__ int range[2];
  __shared__ unsigned long long todo;
  const long long BG = (long long)batch * G;
  const long long n_items = (long long)nb_max * BG;
  const long long first = (long long)blockIdx.x * items_per_wg;
  if (items_per_wg == 1) {
    attend_item<D, HPG, Q8, KV4, COMPACT>(first, q, k, v, qe, ke, ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets,
                        entries, r0, r1, total_q, scale_log2, part_acc, part_ml, spare_row, Ks, Vt,
                        range);
    return;
  }
  const int tid = threadIdx.x;
  if (tid < 64) {
    const long long it = first + tid;
    bool busy = false;
    if (tid < items_per_wg && it < n_items) {
      const long long u = (it % BG) * nb_max + it / BG;
      busy = offsets[u + 1] > offsets[u];
    }
    const unsigned long long m = __ballot(busy);
    if (tid == 0) todo = m;
  }
  __syncthreads();
  unsigned long long m = todo;
  while (m) {
    const int i = __ffsll((long long)m) - 1;
    m &= m - 1;
    attend_item<D, HPG, Q8, KV4, COMPACT>(first + i, q, k, v, qe, ke, ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets,
                        entries, r0, r1, total_q, scale_log2, part_acc, part_ml, spare_row, Ks, Vt,
                        range);
    __syncthreads();   // LDS and range are reused by the next item
  }
}

// Merge: each lane owns one 16-byte chunk of one (query row, head)'s partial
// rows -- 4 fp32 values, or 8 fp16 values with compact partials -- so a wave
// covers 64 * 16 bytes of one slot per load instruction (2 heads at D = 128 with
// fp32 partials, 4 with compact ones; heads of one (row, group) are contiguous
// in every slot).  KMAX >= top_k, so every slot load is issued up front.
constexpr int kMergeWaves = 4;
template <int D, int KMAX, bool COMPACT>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_partials_kernel(
    const void* __restrict__ part_acc, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ sel, int r0, int r1, int Hq, int G, int top_k,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int VPL = COMPACT ? 8 : 4;   // values per lane: 16 bytes
  constexpr int LPH = D / VPL;           // lanes per head
  constexpr int HPW = 64 / LPH;          // heads per wave
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long n = (long long)(r1 - r0) * Hq;
  const long long hh = ((long long)blockIdx.x * kMergeWaves + wv) * HPW + lane / LPH;
  if (hh >= n) return;
  const int c = lane % LPH;              // this lane's chunk of the row
  const int rr = (int)(hh / Hq), h = (int)(hh % Hq);
  const int r = r0 + rr;
  const int hpg = Hq / G;
  const int g = h / hpg;
  const int32_t* srow = sel + ((size_t)r * G + g) * top_k;
  int ns = 0;
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (s < top_k) ns += srow[s] >= 0 ? 1 : 0;
  // partial rows of (row, group, slot) hold the group's heads contiguously
  const size_t base = ((size_t)rr * G + g) * top_k * hpg + (h - g * hpg);
  float2 ml[KMAX];
  uint4 a[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    ml[s] = make_float2(-INFINITY, 0.f);
    a[s] = make_uint4(0, 0, 0, 0);
    if (s < ns) {
      const size_t row = base + (size_t)s * hpg;
      ml[s] = part_ml[row];
      // non-temporal: each partial is read once (measured against ordinary
      // loads on the same buffers: within 1% either way)
      typedef unsigned v4u_nt __attribute__((ext_vector_type(4)));
      const v4u_nt* src = COMPACT
          ? reinterpret_cast<const v4u_nt*>(static_cast<const uint16_t*>(part_acc) + row * D + c * VPL)
          : reinterpret_cast<const v4u_nt*>(static_cast<const float*>(part_acc) + row * D + c * VPL);
      const v4u_nt v = __builtin_nontemporal_load(src);
      a[s] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  float acc[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = 0.f;
  float M = -INFINITY, L = 0.f;
  int e_out = 0;
  if constexpr (COMPACT) {
    // ml[s] = (w_s, E_s): weights 2^(w_s - M), values o_s 2^E_s
    float Em = -INFINITY;
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      if (s < ns) {
        M = fmaxf(M, ml[s].x);
        Em = fmaxf(Em, ml[s].y);
      }
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (s < ns) {
        L += exp2f(ml[s].x - M);
        const float wgt = exp2f(ml[s].x - M + (ml[s].y - Em));
        // the packed words pass through an empty asm so that each slot is
        // unpacked only here: converting every slot's fp16 values up front
        // would hold 8 * KMAX floats (175 registers at KMAX 16 instead of 111)
        // and halve the waves that keep loads in flight
        uint4 av = a[s];
        asm volatile("" : "+v"(av.x), "+v"(av.y), "+v"(av.z), "+v"(av.w));
        const uint32_t w4[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float2 v = unpack2_f16(w4[q]);
          acc[2 * q] += wgt * v.x;
          acc[2 * q + 1] += wgt * v.y;
        }
      }
    }
    e_out = (int)Em;
  } else {
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      if (s < ns) M = fmaxf(M, ml[s].x);
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (s < ns) {
        const float wgt = exp2f(ml[s].x - M);
        L += ml[s].y * wgt;
        acc[0] += wgt * __uint_as_float(a[s].x);
        acc[1] += wgt * __uint_as_float(a[s].y);
        acc[2] += wgt * __uint_as_float(a[s].z);
        acc[3] += wgt * __uint_as_float(a[s].w);
      }
    }
  }
  const float inv = 1.f / L;
  uint16_t* o = out + ((size_t)r * Hq + h) * D + c * VPL;
  uint32_t packed[VPL / 2];
#pragma unroll
  for (int q = 0; q < VPL / 2; ++q)
    packed[q] = pack2_bf16(ldexpf(acc[2 * q] * inv, e_out), ldexpf(acc[2 * q + 1] * inv, e_out));
  if constexpr (VPL == 8)
    *reinterpret_cast<uint4*>(o) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  else
    *reinterpret_cast<uint2*>(o) = make_uint2(packed[0], packed[1]);
  if (lse && c == 0) lse[(size_t)r * Hq + h] = (M + log2f(L)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------------------
template <int D, int HPG, bool COMPACT>
static void launch_attend_t(const void* q, const void* k, const void* v, MainFp8 f8,
                            const int32_t* cu_q,
                            const int32_t* cu_k, KvMap kv, int batch, int G, int Hq, int top_k,
                            int nb_max,
                            const int32_t* offsets, const int32_t* entries, int r0, int r1,
                            int total_q, float scale_log2, void* part_acc, float2* part_ml,
                            hipStream_t st) {
  // sparse selections (few queries per item on average): scan items in runs of 64
  const long long n_items = (long long)nb_max * batch * G;
  const double per_item = (double)(r1 - r0) * G * top_k / (double)n_items;
  const int ipw = per_item >= 4.0 ? 1 : 64;
  dim3 grid((unsigned)((n_items + ipw - 1) / ipw));
  if (f8.qe && f8.kv4)
    hipLaunchKernelGGL((attend_blocks_kernel<D, HPG, true, true, COMPACT>), grid, dim3(256), 0, st, q, k, v,
                       f8.qe, f8.ke, f8.ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets,
                       entries, r0, r1, total_q, scale_log2, part_acc, part_ml,
                       (r1 - r0) * Hq * top_k, ipw);
  else if (f8.qe)
    hipLaunchKernelGGL((attend_blocks_kernel<D, HPG, true, false, COMPACT>), grid, dim3(256), 0, st, q, k, v, f8.qe,
                       f8.ke, f8.ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets, entries,
                       r0, r1, total_q, scale_log2, part_acc, part_ml, (r1 - r0) * Hq * top_k, ipw);
  else
    hipLaunchKernelGGL((attend_blocks_kernel<D, HPG, false, false, COMPACT>), grid, dim3(256), 0, st, q, k, v,
                       (const uint8_t*)nullptr, (const uint8_t*)nullptr, (const uint8_t*)nullptr,
                       cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets, entries, r0, r1,
                       total_q, scale_log2, part_acc, part_ml, (r1 - r0) * Hq * top_k, ipw);
}

template <int D, bool COMPACT>
static hipError_t launch_attend_d(int hpg, const void* q, const void* k, const void* v, MainFp8 f8,
                                  const int32_t* cu_q, const int32_t* cu_k, KvMap kv, int batch,
                                  int G, int Hq,
                                  int top_k, int nb_max, const int32_t* offsets,
                                  const int32_t* entries, int r0, int r1, int total_q,
                                  float scale_log2, void* part_acc, float2* part_ml,
                                  hipStream_t st) {
#define MSA_ATT(H) launch_attend_t<D, H, COMPACT>(q, k, v, f8, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets, entries, r0, r1, total_q, scale_log2, part_acc, part_ml, st)
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

hipError_t launch_attend_blocks(int D, int hpg, bool compact, const void* q, const void* k,
                                const void* v, MainFp8 f8, const int32_t* cu_q, const int32_t* cu_k,
                                KvMap kv, int batch, int G, int Hq, int top_k, int nb_max,
                                const int32_t* offsets, const int32_t* entries, int r0, int r1,
                                int total_q, float scale_log2, void* part_acc, float2* part_ml,
                                hipStream_t st) {
#define MSA_ATD(DD, C) launch_attend_d<DD, C>(hpg, q, k, v, f8, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, offsets, entries, r0, r1, total_q, scale_log2, part_acc, part_ml, st)
  if (D == 64) return compact ? MSA_ATD(64, true) : MSA_ATD(64, false);
  if (D == 128) return compact ? MSA_ATD(128, true) : MSA_ATD(128, false);
#undef MSA_ATD
  return hipErrorInvalidValue;
}

template <int D, int KMAX, bool COMPACT>
static void launch_merge_t(dim3 grid, const void* part_acc, const float2* part_ml, const int32_t* sel,
                           int r0, int r1, int Hq, int G, int top_k, void* out, float* lse,
                           hipStream_t st) {
  hipLaunchKernelGGL((merge_partials_kernel<D, KMAX, COMPACT>), grid, dim3(kMergeWaves * 64), 0, st,
                     part_acc, part_ml, sel, r0, r1, Hq, G, top_k, (uint16_t*)out, lse);
}

template <int D, bool COMPACT>
static void launch_merge_d(dim3 grid, const void* part_acc, const float2* part_ml, const int32_t* sel,
                           int r0, int r1, int Hq, int G, int top_k, void* out, float* lse,
                           hipStream_t st) {
#define MSA_MRG(K) launch_merge_t<D, K, COMPACT>(grid, part_acc, part_ml, sel, r0, r1, Hq, G, top_k, out, lse, st)
  if (top_k <= 4) MSA_MRG(4);
  else if (top_k <= 8) MSA_MRG(8);
  else if (top_k <= 16) MSA_MRG(16);
  else MSA_MRG(32);
#undef MSA_MRG
}

hipError_t launch_merge(int D, bool compact, const void* part_acc, const float2* part_ml,
                        const int32_t* sel, int r0, int r1, int Hq, int G, int top_k, void* out,
                        float* lse, hipStream_t st) {
  // heads per wave: 64 lanes of 16 bytes over one head's row of D fp32 or fp16 values
  const long long hpw = 64 / (D / (compact ? 8 : 4));
  const long long n = (long long)(r1 - r0) * Hq;
  const long long waves = (n + hpw - 1) / hpw;
  dim3 grid((unsigned)((waves + kMergeWaves - 1) / kMergeWaves));
#define MSA_MRD(DD, C) launch_merge_d<DD, C>(grid, part_acc, part_ml, sel, r0, r1, Hq, G, top_k, out, lse, st)
  if (D == 64) {
    if (compact) MSA_MRD(64, true); else MSA_MRD(64, false);
  } else if (D == 128) {
    if (compact) MSA_MRD(128, true); else MSA_MRD(128, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef MSA_MRD
  return hipGetLastError();
}

}  // namespace msa
