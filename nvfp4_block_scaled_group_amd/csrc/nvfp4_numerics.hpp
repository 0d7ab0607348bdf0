// nvfp4_numerics.hpp -- device-side bit helpers and the NVFP4 scale /
// encode steps shared by the kernels of libnvfp4g.so (and exercised
// exhaustively by the GPU self-test library of the test suite).
//
// The numerics follow the per-token NVFP4 recipe ("Implement per-token NVFP4
// fprop recipe", TransformerEngine PR 2931, Description): one fp32 amax per
// line, E2M1 values, one E4M3 scale per 16 elements, with the fixed fp32
// reading  s = A/2688,  S = E4M3((b/6)/s),  m = 1/(value(S)*s),
// code = E2M1(x*m).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>

namespace nvfp4g {

// ------------------------------------------------------------ bit helpers

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
      __builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}

__device__ __forceinline__ uint32_t hmax(uint32_t a) {  // max of the two halves
  return max(a & 0xFFFFu, a >> 16);
}

// DPP row_ror:8 inside a 16-lane row == lane ^ 8.
__device__ __forceinline__ uint32_t swap8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}
// quad_perm [1,0,3,2] == lane ^ 1; quad_perm [2,3,0,1] == lane ^ 2;
// row_half_mirror maps lane i of an 8-lane half row to 7 - i.
__device__ __forceinline__ uint32_t dpp_x1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_x2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_hmirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
}

// gfx950 cross-row swaps: permlane32_swap(a, b) exchanges lanes 32..63 of a
// with lanes 0..31 of b; permlane16_swap(a, b) exchanges the odd 16-lane rows
// of a with the even rows of b.  The max of the two results is the max over
// lane pairs l, l^32 (resp. l, l^16) of a in the lower half (even rows) and of
// b in the upper half (odd rows).
__device__ __forceinline__ uint32_t swap32_max(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return pkmax(r[0], r[1]);
}
__device__ __forceinline__ uint32_t swap16_max(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return pkmax(r[0], r[1]);
}

// Reduce-scatter of 8 packed values over the 64 lanes of a wave: returns, in
// every lane, the max over all lanes of value[lane >> 3].
__device__ __forceinline__ uint32_t wave_reduce_scatter8(const uint32_t (&v)[8], int lane) {
  uint32_t n[4], m[2];
#pragma unroll
  for (int p = 0; p < 4; ++p) n[p] = swap32_max(v[p], v[p + 4]);  // value p + 4*bit5
#pragma unroll
  for (int q = 0; q < 2; ++q) m[q] = swap16_max(n[q], n[q + 2]);  // + 2*bit4
  const bool b3 = (lane >> 3) & 1;                                  // + bit3
  uint32_t r = pkmax(b3 ? m[1] : m[0], swap8(b3 ? m[0] : m[1]));
  r = pkmax(r, dpp_x1(r));
  r = pkmax(r, dpp_x2(r));
  return pkmax(r, dpp_hmirror(r));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- numerics

// E4M3FN code of t >= 0 (finite or +inf): nearest, ties to even, saturating
// at 448 (0x7E).  gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN) rounds to nearest
// with ties to even; it does not saturate (t >= 464 gives NaN), so t is
// clamped at 448 first.  With the clamp it equals the plain rule (round the
// fp32 mantissa to 3 bits and re-bias the exponent by 7 - 127; below 2^-6
// the nearest multiple of 2^-9; 0x7E from 448 up) on every fp32 t in
// [0, +inf], as checked on the hardware by the GPU self-test.
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// value(c) of an E4M3FN code (0 .. 0x7E), exact: v_cvt_f32_fp8, checked on
// the hardware against  e ? 2^(e-7) * (1 + f/8) : f * 2^-9  for every code.
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// Block step: E4M3 scale code of a block with amax b on a line with scale s,
// and the element multiplier m = 1 / (value(S) * s).
__device__ __forceinline__ uint32_t block_scale(float b, float s, float* m) {
  const float t = (s == 0.0f) ? 0.0f : (b / 6.0f) / s;
  const uint32_t S = e4m3_code(t);
  const float d = e4m3_value(S) * s;
  *m = (d == 0.0f) ? 0.0f : fminf(1.0f / d, FLT_MAX);
  return S;
}

// Same step with fewer operations, for line scales s >= 2^-112 (line amax of
// about 2^-100.6 or more), given ys = 1/s (correctly rounded, once per line):
//   u = b/6 as q0 = b*RN(1/6) plus one fused residual correction,
//   t = u/s as t0 = u*ys plus one fused residual correction,
//   m = 1/d as the hardware reciprocal plus one Newton step.
// Over every pair of bf16 values b <= A with A >= 2^-102 this gives the same
// E4M3 code, and (for A >= 2^-105) the same m bits, as the correctly rounded
// divisions above; smaller lines take the exact path.
constexpr float kFastMinLineScale = 0x1p-112f;

__device__ __forceinline__ uint32_t block_scale_fast(float b, float s, float ys, float* m) {
  const float r6 = 0x1.555556p-3f;  // RN(1/6)
  const float q0 = b * r6;
  const float u = __builtin_fmaf(__builtin_fmaf(-6.0f, q0, b), r6, q0);
  const float t0 = u * ys;
  const float t = __builtin_fmaf(__builtin_fmaf(-s, t0, u), ys, t0);
  const uint32_t S = e4m3_code(t);
  const float d = e4m3_value(S) * s;
  const float y0 = __builtin_amdgcn_rcpf(d);
  const float y1 = __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
  *m = (d == 0.0f) ? 0.0f : fminf(y1, FLT_MAX);
  return S;
}

__device__ __forceinline__ uint32_t block_step(float b, float s, float ys, float* m) {
  if (s >= kFastMinLineScale) return block_scale_fast(b, s, ys, m);
  return block_scale(b, s, m);
}

// RN(1/d) for 2^-126 <= d < 2^126 (d and 1/d normal): the hardware
// reciprocal plus one Newton step.  On the hardware it equals the IEEE
// division 1/d on every fp32 d in that range (GPU self-test).
__device__ __forceinline__ float rcp_rn(float d) {
  const float y0 = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, y0, 1.0f), y0, y0);
}

// RN(b/6) for a bf16 value b >= 0 (given as fp32): b * RN(1/6) plus one
// residual correction.  Equals the IEEE division b/6 on every finite
// non-negative bf16 value (GPU self-test).
__device__ __forceinline__ float div6_bf16(float b) {
  const float r6 = 0x1.555556p-3f;  // RN(1/6)
  const float q0 = b * r6;
  return __builtin_fmaf(__builtin_fmaf(-6.0f, q0, b), r6, q0);
}

// u / s as u * ys plus one fused residual correction, given ys = RN(1/s)
// (once per line).  For the four-over-six block steps -- s = A / (6 * Bnd)
// with A a bf16 line amax, s >= 2^-112, Bnd in 1 .. 448, u = RN(b / 6) or
// b / 4 for every bf16 block amax b <= A -- it gives the IEEE quotient's
// E4M3 code on every input (exhaustive GPU self-test).
__device__ __forceinline__ float quot_fast(float u, float s, float ys) {
  const float t0 = u * ys;
  return __builtin_fmaf(__builtin_fmaf(-s, t0, u), ys, t0);
}

// Hardware FP4 conversion (gfx950): two fp32 values -> one E2M1x2 byte
// (first value in the low nibble) placed at byte SEL of `old`.  With scale
// 1.0 it rounds to nearest (ties to the even code), saturates at +-6 and
// keeps the sign of zero: it equals e2m1_code below on every non-NaN fp32
// input.
#define FP4X2(old, a, b, SEL) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (SEL))

// 4-bit E2M1 code of v: sign bit of v, magnitude nearest on
// {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even code, saturating.
// |v| >= 1: round the fp32 mantissa to 1 bit; the code is then the fp32
// exponent/mantissa re-biased (code 2 = 1.0).  |v| < 1: the code is the
// nearest integer (ties even) to 2|v|.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t vb = __float_as_uint(v);
  const uint32_t sign = (vb >> 28) & 8u;
  const uint32_t a = vb & 0x7FFFFFFFu;
  uint32_t hi = (a + 0x1FFFFFu + ((a >> 22) & 1u) - 0x3F000000u) >> 22;
  hi = min(hi, 7u);
  const uint32_t lo = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  return sign | (a >= 0x3F800000u ? hi : lo);
}

}  // namespace nvfp4g
