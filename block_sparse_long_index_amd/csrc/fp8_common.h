// OCP FP8 E4M3 codes with power-of-two (E8M0) scales: the shared pieces of
// the quantised Index Branch and the quantised Main Branch.  A row or block's
// exponent e is the smallest integer with amax * 2^-e <= 448 (the largest
// E4M3 value), clamped to [-127, 127]; codes are one round-to-nearest-even
// conversion of x * 2^-e; a code's value is decode(code) * 2^e.
#pragma once

#include "msa_common.h"

namespace msa {

// Smallest e with amax * 2^-e <= 448 (the largest E4M3 value), clamped to
// [-127, 127]; 0 for amax == 0.  amax = f * 2^E with f in [0.5, 1):
// f * 2^9 <= 448 exactly when f <= 0.875.
__device__ inline int fp8_scale_exponent(float amax) {
  if (amax == 0.f) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = f <= 0.875f ? E - 9 : E - 8;
  return min(127, max(-127, e));
}

// Eight bf16 values -> eight E4M3 codes of x * 2^-e (exact scaling, then one
// round-to-nearest-even conversion), little-endian in two dwords.
__device__ inline uint2 quantize8(const float (&x)[8], int e) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(448.f, fmaxf(-448.f, ldexpf(x[i], -e)));
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  return make_uint2((uint32_t)w0, (uint32_t)w1);
}

__device__ inline void unpack8_bf16(uint4 v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---------------------------------------------------------------------------
// Quantisation.  q rows: DI / 8 lanes per (query, group) row, each converting
// 8 elements; the row maximum is a shuffle reduction inside the row's lanes.
// ---------------------------------------------------------------------------
template <int DI>
__global__ __launch_bounds__(256) void quantize_q_kernel(const uint16_t* __restrict__ q,
                                                         long long rows,
                                                         uint8_t* __restrict__ q8,
                                                         uint8_t* __restrict__ qe) {
  constexpr int LPR = DI / 8;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int c = (int)(t % LPR);
  const bool ok = row < rows;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (ok) v = *reinterpret_cast<const uint4*>(q + row * DI + c * 8);
  float x[8];
  unpack8_bf16(v, x);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) a = fmaxf(a, shfl_xor_f(a, off));
  const int e = fp8_scale_exponent(a);
  const uint2 w = quantize8(x, e);
  if (ok) {
    *reinterpret_cast<uint2*>(q8 + row * DI + c * 8) = w;
    if (c == 0) qe[row] = (uint8_t)(e + 127);
  }
}

// Eight E4M3 codes (little-endian in two dwords) at exponent e -> their
// eight values as bf16.  decode(code) * 2^e has at most 4 significant bits
// and its lowest set bit is at least 2^(e-9), so it is a bf16 number -- and
// the conversion exact -- whenever e >= -124 (bf16's finest subnormal step is
// 2^-133); for e in -127 .. -125 the smallest codes' values lie below that
// step and are rounded to nearest even, like any value rounded to bf16 (an
// absolute change below 2^-133).  One scaled conversion
// (v_cvt_scalef32_pk_bf16_fp8) turns the two codes of one 16-bit half and the
// scale 2^e into two bf16 values, low byte first; over every code that is not
// NaN (the quantisers never produce one), both byte positions and exponents
// -127 .. 127 it gives the round-to-nearest-even bf16 of the exact product.
__device__ inline uint4 dequant8_bf16(uint2 w, int e) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const float s = ldexpf(1.f, e);
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, s, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, s, true)));
}

// ---------------------------------------------------------------------------
// 4-bit codes (index keys; Main-Branch keys and values).  A 32-element
// group's exponent e is the smallest integer with amax * 2^-e <= 6 (the
// largest E2M1 value), clamped to [-127, 127], 0 for an all-zero group; codes
// are the nearest E2M1 value of x * 2^-e, ties to the even code, with x's
// sign bit.
// ---------------------------------------------------------------------------
__device__ inline int fp4_scale_exponent(float amax) {
  if (amax == 0.f) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = f <= 0.75f ? E - 3 : E - 2;   // f * 2^3 <= 6 exactly when f <= 0.75
  return min(127, max(-127, e));
}

// E2M1 code of one value already scaled into [-6, 6].  The thresholds are the
// midpoints of the grid 0, .5, 1, 1.5, 2, 3, 4, 6; at a midpoint the even code
// (mantissa bit 0: 0, 1, 2, 4) wins, hence > below even codes and >= below odd.
__device__ inline uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.f);
  return c | ((__float_as_uint(y) >> 31) << 3);
}

// Eight E2M1 codes (element i in nibble i of w, low nibble first) times the
// group scale s = 2^e -> eight bf16 values.  A code's value has at most 2
// significant bits and its lowest set bit is at least 2^(e-1), so the product
// is a bf16 number for every e in -127 .. 127 and the conversion is exact.
// One scaled conversion (v_cvt_scalef32_pk_bf16_fp4) turns the two codes of
// one byte into two bf16 values, low nibble first.
__device__ inline uint4 dequant4_bf16_scaled(uint32_t w, float s) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3)));
}

__device__ inline uint4 dequant4_bf16(uint32_t w, int e) { return dequant4_bf16_scaled(w, ldexpf(1.f, e)); }

}  // namespace msa
