// Main Branch for decode-shaped passes (a few new tokens per sequence).
//
// Same computation and the same partial format as attend_blocks_kernel (exact
// softmax over each selected block's visible keys; MSA guide,
// ai-tool-zukan.com/minimax-msa-guide, sections "MiniMax MSAとは何か" and
// "2段階構造の中身"), but with one query per (sequence, group) a KV block is hit
// by that query alone, so "KV block outer, gather the queries that hit it"
// (tnkblog.net MiniMax M3 MSA post, section "MSA の実装") needs no list: each
// workgroup takes one (group, selected slot, query) straight from the
// selection and reads that block once.
//
// One workgroup (4 waves) per item, groups fastest.  Fragment loads straight
// from global memory would touch 32 key rows per instruction; here every load
// instruction reads whole rows (1 KiB of consecutive row bytes per wave).  K
// (bf16 values or 8-bit codes) reaches LDS by direct global->LDS 16-byte
// loads; V is loaded into registers at the same time and written over K, as
// bf16, once the scores are done, so waiting for K never waits for V (the
// compiler cannot tell two direct-to-LDS streams apart) and the block needs
// one bf16 tile of LDS (32 KiB at D = 128).  8-bit inputs (E4M3 codes with
// power-of-two scales) are dequantised exactly into bf16: K fragments as they
// leave LDS, V as it enters.  4-bit K and V (E2M1 codes, one exponent per 32
// elements) are small enough to come in together: codes and exponents of
// both land inside the tile's bytes, V's codes move to registers before the
// barrier that ends the score phase, and V enters the tile as bf16 after it.
// Chunk positions are XOR-swizzled: K so that an A-fragment read (16
// consecutive rows, one 16-byte chunk each) hits 16 bank groups; V so that the
// transposed reads (ds_read_b64_tr_b16: within 16 lanes, lane 4a + c receives
// element c of the 8-byte pieces addressed by lanes a, a + 4, a + 8, a + 12)
// of 4 rows x 4 chunks hit 16 bank groups.  Those transposed reads give each
// lane four consecutive keys of one column: the V^T A fragment without a
// transposing store.  Wave w scores key tile w; the softmax maximum and sum
// combine through LDS; every key tile's bf16 P goes through LDS (the group's
// head columns only: with 8 heads a workgroup needs 35 KiB of LDS at D = 128,
// so 4 fit on a CU), and wave w then forms output columns 32w .. 32w + 31
// (D = 64: waves 0 and 1).  Barriers
// are bare (s_barrier after lgkmcnt(0)): a workgroup fence would also wait for
// the loads still in flight.
#include <algorithm>

#include "fp8_common.h"
#include "msa_common.h"

namespace msa {

template <int D, int HPG, bool Q8, bool KV4>
__global__ __launch_bounds__(256) void attend_decode_lds_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const uint8_t* __restrict__ qe, const uint8_t* __restrict__ ke, const uint8_t* __restrict__ ve,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, KvMap kv, int batch, int G,
    int Hq, int top_k, int nb_max, const int32_t* __restrict__ sel, int r0, int rz, float scale_log2,
    float* __restrict__ part_acc, float2* __restrict__ part_ml) {
  constexpr int RB = D * 2;                     // bytes per bf16 row (the V tile)
  constexpr int CPR = RB / 16;                  // 16-byte chunks per bf16 row
  constexpr int R = 256 / RB;                   // bf16 rows per 256-byte bank line
  constexpr int RBS = KV4 ? D / 2 : Q8 ? D : 2 * D;   // bytes per stored row (codes or bf16)
  constexpr int CPRS = RBS / 16;
  constexpr int RS = 256 / RBS;
  constexpr int ROWS_PER_PIECE = 1024 / RBS;    // rows per wave load instruction
  constexpr int PER_WAVE = kBlock / ROWS_PER_PIECE / 4;
  constexpr int XB = D / 32;                    // 4-bit rows: exponent bytes per (key, head)
  constexpr int XS = 4;                         // LDS bytes per key of a direct exponent load
  // 4-bit K and V: codes, then exponents, of K and then of V, all inside the
  // bf16 V tile's bytes (read out before the tile is written)
  constexpr int EXP_OFF = kBlock * RBS;
  constexpr int VC_OFF = (EXP_OFF + kBlock * XS + 1023) / 1024 * 1024;
  constexpr int VX_OFF = VC_OFF + kBlock * RBS;
  static_assert(!KV4 || VX_OFF + kBlock * XS <= kBlock * RB, "4-bit K and V fit the V tile");
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int PC = HPG;                       // P columns kept: the group's heads
  // K as stored (and 4-bit V as stored), then the bf16 V tile over it
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kBlock * RB];
  uint8_t* const Vs = Ks;
  __shared__ __attribute__((aligned(16))) uint4 Pl[4][2][2][PC];
  __shared__ float red_m[4][32], red_l[4][32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, half = lane >> 5;
  // r0: the pass's first row (partials are indexed from it); rz: this launch's
  const int r = rz + (int)blockIdx.z, slot = (int)blockIdx.y, g = (int)blockIdx.x;
  const RowPos rp = locate_row(r, cu_q, cu_k, batch);
  const int beta = sel[((size_t)r * G + g) * top_k + slot];
  if (beta < 0 || beta * kBlock >= rp.lk) return;   // the same for the whole workgroup
  const int kb = beta * kBlock;
  const int nvalid = min(kBlock, rp.lk - kb);       // rows of the block in the sequence
  const size_t row0 = kv.block_row(rp.b, rp.koff, beta);
  const uint8_t* const kbytes = static_cast<const uint8_t*>(k);
  const uint8_t* const vbytes = static_cast<const uint8_t*>(v);

  // Q^T: MFMA column n = head n of the query's group (columns >= HPG repeat
  // head 0 and are never stored).  bf16: k-step ks of lane half h covers
  // elements 16ks + 8h .. +7.  8-bit K: k-step 2j + e covers 32j + 16h + 8e ..
  // +7, so that a lane's two k-steps read one 16-byte chunk of K codes; 4-bit
  // K: k-step 4j + e covers 64j + 32h + 8e .. +7 (one 16-byte chunk of codes
  // = one 32-element scale group per four k-steps).  Raw query codes are
  // loaded before the block and dequantised once K has landed.
  const int hl = col < HPG ? col : 0;
  const size_t qrow = (size_t)r * Hq + g * HPG + hl;
  bf16x8 qf[KS];
  uint2 qraw[Q8 ? KS : 1];
  // exponent bytes are loaded before the block and used raw (subtracting the
  // bias at once would make the first block load wait for them)
  uint32_t qexp_b = Q8 ? (uint32_t)qe[qrow] : 127u;
  uint32_t kexp_b = 127u, vexp_b = 127u;
  if constexpr (Q8 && !KV4) {
    const size_t xi = kv.block_index(rp.b, beta, nb_max) * G + g;
    kexp_b = ke[xi];
    vexp_b = ve[xi];
  }
  if constexpr (KV4) {
    const uint8_t* qs = static_cast<const uint8_t*>(q) + qrow * D + half * 32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ks] = *reinterpret_cast<const uint2*>(qs + (ks >> 2) * 64 + (ks & 3) * 8);
  } else if constexpr (Q8) {
    const uint8_t* qs = static_cast<const uint8_t*>(q) + qrow * D + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[ks] = *reinterpret_cast<const uint2*>(qs + (ks >> 1) * 32 + (ks & 1) * 8);
  } else {
    const uint16_t* qs = static_cast<const uint16_t*>(q) + qrow * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qs + ks * 16));
  }

  auto swz_k = [](int m) { return (m / RS) % CPRS; };
  auto swz_v = [](int m) { return 4 * ((m / R) % (CPR / 4)); };
  // this wave's pieces of K (straight to LDS) and of V (to registers); rows
  // past the sequence read its last row (masked below: they only need to be
  // finite)
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int piece = wave * PER_WAVE + i;
    const int m = piece * ROWS_PER_PIECE + lane / CPRS;
    const size_t src = ((row0 + min(m, nvalid - 1)) * G + g) * RBS;
    lds_load16(kbytes + src + ((lane % CPRS) ^ swz_k(m)) * 16, Ks + piece * 1024);
  }
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u vreg[KV4 ? 1 : PER_WAVE];
  if constexpr (KV4) {
    // 4-bit rows are small: K's and V's codes and exponents all go straight to
    // LDS, waited for at once; V is dequantised from its LDS copy into the
    // bf16 tile after the scores.  Exponents: XB bytes per key, one key per
    // lane; loads of up to 4 bytes put lane L's bytes at 4 L (XS).
    const int key = (wave & 1) * 64 + lane;
    const size_t rk = ((row0 + min(key, nvalid - 1)) * G + g) * XB;
    if (wave < 2) lds_load_n<XB>(ke + rk, Ks + EXP_OFF + wave * 64 * XS);
    else lds_load_n<XB>(ve + rk, Ks + VX_OFF + (wave - 2) * 64 * XS);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      const int m = piece * ROWS_PER_PIECE + lane / CPRS;
      const size_t src = ((row0 + min(m, nvalid - 1)) * G + g) * RBS;
      lds_load16(vbytes + src + (lane % CPRS) * 16, Ks + VC_OFF + piece * 1024);
    }
  } else {
    // V into registers (the same coalesced pieces), written to LDS over K once
    // the scores are done
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      const int m = piece * ROWS_PER_PIECE + lane / CPRS;
      const size_t src = ((row0 + min(m, nvalid - 1)) * G + g) * RBS;
      vreg[i] = *reinterpret_cast<const v4u*>(vbytes + src + (lane % CPRS) * 16);
    }
  }

  auto barrier = []() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (KV4) wait_vmcnt<0>();
  else wait_vmcnt<PER_WAVE>();   // the query and this wave's K pieces (V may still be in flight)
  barrier();
  if constexpr (Q8) {
    // opaque after the barrier: the compiler would otherwise dequantise the
    // query before it and wait for every load, V's included, to do so
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qraw[ks].x), "+v"(qraw[ks].y));
    asm volatile("" : "+v"(qexp_b), "+v"(kexp_b), "+v"(vexp_b));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(dequant8_bf16(qraw[ks], (int)qexp_b - 127));
  }
  const int kexp = (int)kexp_b - 127, vexp = (int)vexp_b - 127;

  // S^T = K * Q^T for keys 32 wave .. 32 wave + 31
  f32x16 sacc = f32x16{};
  {
    const int m = wave * 32 + col;
    if constexpr (KV4) {
#pragma unroll
      for (int j = 0; j < KS / 4; ++j) {
        const int ch = 2 * j + half;   // elements 64j + 32 half .. +31: one scale group
        const uint4 c = *reinterpret_cast<const uint4*>(Ks + m * RBS + ((ch ^ swz_k(m)) * 16));
        const int e = (int)Ks[EXP_OFF + m * XS + ch] - 127;
        sacc = mfma32(as_bf16x8(dequant4_bf16(c.x, e)), qf[4 * j], sacc);
        sacc = mfma32(as_bf16x8(dequant4_bf16(c.y, e)), qf[4 * j + 1], sacc);
        sacc = mfma32(as_bf16x8(dequant4_bf16(c.z, e)), qf[4 * j + 2], sacc);
        sacc = mfma32(as_bf16x8(dequant4_bf16(c.w, e)), qf[4 * j + 3], sacc);
      }
    } else if constexpr (Q8) {
#pragma unroll
      for (int j = 0; j < KS / 2; ++j) {
        const uint4 c = *reinterpret_cast<const uint4*>(Ks + m * RBS + (((2 * j + half) ^ swz_k(m)) * 16));
        sacc = mfma32(as_bf16x8(dequant8_bf16(make_uint2(c.x, c.y), kexp)), qf[2 * j], sacc);
        sacc = mfma32(as_bf16x8(dequant8_bf16(make_uint2(c.z, c.w), kexp)), qf[2 * j + 1], sacc);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(Ks + m * RBS + (((2 * ks + half) ^ swz_k(m)) * 16));
        sacc = mfma32(as_bf16x8(a), qf[ks], sacc);
      }
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
  // 4-bit V: this lane's codes (32 codes, one scale group, per piece) and
  // their exponents leave LDS before the barrier, after which the tile is
  // overwritten
  uint4 vcode[KV4 ? PER_WAVE : 1];
  int vex[KV4 ? PER_WAVE : 1];
  if constexpr (KV4) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int piece = wave * PER_WAVE + i;
      const int mv = piece * ROWS_PER_PIECE + lane / CPRS;
      vcode[i] = *reinterpret_cast<const uint4*>(Ks + VC_OFF + piece * 1024 + lane * 16);
      vex[i] = (int)Ks[VX_OFF + mv * XS + lane % CPRS] - 127;
    }
  }
  barrier();
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
    if (col < PC)
      Pl[wave][s2][half][col] = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]),
                                           pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7]));
  }
  l += shfl_xor_f(l, 32);
  if (half == 0) red_l[wave][col] = l;
  // every wave's K (and 4-bit V) reads ended at the barrier above: V (bf16)
  // replaces them
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int piece = wave * PER_WAVE + i;
    const int mv = piece * ROWS_PER_PIECE + lane / CPRS;
    const int c = lane % CPRS;   // chunk of the stored row
    if constexpr (KV4) {
      // this lane's own piece of V codes (32 codes: one scale group) -> bf16
      // chunks 4c .. 4c + 3 of the row
      const uint4 cv = vcode[i];
      const int e = vex[i];
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((4 * c) ^ swz_v(mv)) * 16)) = dequant4_bf16(cv.x, e);
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((4 * c + 1) ^ swz_v(mv)) * 16)) = dequant4_bf16(cv.y, e);
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((4 * c + 2) ^ swz_v(mv)) * 16)) = dequant4_bf16(cv.z, e);
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((4 * c + 3) ^ swz_v(mv)) * 16)) = dequant4_bf16(cv.w, e);
    } else if constexpr (Q8) {
      // 16 codes -> bf16 chunks 2c and 2c + 1 of the row
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((2 * c) ^ swz_v(mv)) * 16)) =
          dequant8_bf16(make_uint2(vreg[i].x, vreg[i].y), vexp);
      *reinterpret_cast<uint4*>(Vs + mv * RB + (((2 * c + 1) ^ swz_v(mv)) * 16)) =
          dequant8_bf16(make_uint2(vreg[i].z, vreg[i].w), vexp);
    } else {
      *reinterpret_cast<v4u*>(Vs + mv * RB + ((c ^ swz_v(mv)) * 16)) = vreg[i];
    }
  }
  barrier();
  if (wave >= DT) return;

  // O^T = V^T * P^T for output columns 32 wave .. 32 wave + 31: lane <-> head,
  // register i <-> column 32 wave + 8(i/4) + 4 half + i%4
  f32x16 oacc = f32x16{};
  {
    const int grp = lane >> 4, mm = lane & 15;
    const int d0 = wave * 32 + 16 * (grp & 1);              // this 16-lane group's columns
    const int cb = (2 * d0 + 8 * (mm & 3)) >> 4;             // chunk of lane mm's 8-byte piece
    const int cofs = 8 * (mm & 1);                           // byte offset inside the chunk
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int kb1 = kt * 32 + 16 * s2 + 4 * (grp >> 1) + (mm >> 2);   // row this lane addresses
        const int kb2 = kb1 + 8;
        const uint2 lw = lds_read_tr16(Vs + kb1 * RB + ((cb ^ swz_v(kb1)) * 16) + cofs);
        const uint2 hw = lds_read_tr16(Vs + kb2 * RB + ((cb ^ swz_v(kb2)) * 16) + cofs);
        // P columns past the group's heads are zero (their outputs are never stored)
        const uint4 pb = col < PC ? Pl[kt][s2][half][col] : make_uint4(0, 0, 0, 0);
        oacc = mfma32(as_bf16x8(make_uint4(lw.x, lw.y, hw.x, hw.y)), as_bf16x8(pb), oacc);
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
  // rows go in grid z, whose limit is 65535: larger passes take several launches
  constexpr int kMaxRowsPerLaunch = 65535;
  for (int rz = r0; rz < r1; rz += kMaxRowsPerLaunch) {
    const dim3 grid(G, top_k, std::min(r1 - rz, kMaxRowsPerLaunch));
    if (f8.qe && f8.kv4)
      hipLaunchKernelGGL((attend_decode_lds_kernel<D, HPG, true, true>), grid, dim3(256), 0, st, q, k, v,
                         f8.qe, f8.ke, f8.ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel, r0, rz,
                         scale_log2, part_acc, part_ml);
    else if (f8.qe)
      hipLaunchKernelGGL((attend_decode_lds_kernel<D, HPG, true, false>), grid, dim3(256), 0, st, q, k, v,
                         f8.qe, f8.ke, f8.ve, cu_q, cu_k, kv, batch, G, Hq, top_k, nb_max, sel, r0, rz,
                         scale_log2, part_acc, part_ml);
    else
      hipLaunchKernelGGL((attend_decode_lds_kernel<D, HPG, false, false>), grid, dim3(256), 0, st, q, k, v,
                         (const uint8_t*)nullptr, (const uint8_t*)nullptr, (const uint8_t*)nullptr, cu_q,
                         cu_k, kv, batch, G, Hq, top_k, nb_max, sel, r0, rz, scale_log2, part_acc,
                         part_ml);
  }
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
