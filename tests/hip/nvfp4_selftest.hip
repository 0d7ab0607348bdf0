// nvfp4_selftest.hip -- test-only GPU library that runs the device numerics
// of libnvfp4g.so (csrc/nvfp4_numerics.hpp) exhaustively or on given samples,
// for tests/test_gpu_numerics.py.  Not part of the product library.
//
//  * the hardware FP4 convert (FP4X2, scale 1.0) against the software E2M1
//    rule (e2m1_code) on every non-NaN fp32 pattern, both nibble positions;
//  * the hardware E4M3 encode / decode (e4m3_code, e4m3_value) against the
//    plain E4M3FN rule on every fp32 t in [0, +inf] and every finite code;
//  * the kernels' block step (fast path for line scales >= 2^-112, IEEE
//    divisions below) against the IEEE-division block step on every pair of
//    bf16 values b <= A (b = block amax, A = line amax);
//  * the hardware FP4 -> fp32 convert with unit scale (the four-over-six
//    cast's dequantised values) on every byte at every byte position;
//  * the fast reciprocal (rcp_rn) against the IEEE division on every normal
//    fp32 d with a normal reciprocal, and the fast b/6 (div6_bf16) on every
//    finite non-negative bf16 b;
//  * the fast quotient of the four-over-six block step (quot_fast) against
//    the IEEE division on every (A, bound, b, candidate) it is used for;
//  * sample outputs (block step, FP4 codes) that the tests compare with the
//    CPU oracle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../nvfp4_block_scaled_group_amd/csrc/nvfp4_numerics.hpp"

using namespace nvfp4g;

namespace {

__global__ void fp4_exhaustive_kernel(unsigned long long* counts, uint32_t base) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long n = 0, bad_lo = 0, bad_hi = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 31); i += stride) {
    const float v = __uint_as_float(base + (uint32_t)i);
    if (v != v) continue;
    const uint32_t sw = e2m1_code(v);
    const uint32_t lo = FP4X2(0u, v, 0.0f, 0) & 0xFFu;
    const uint32_t hi = FP4X2(0u, 0.0f, v, 0) & 0xFFu;
    n++;
    bad_lo += lo != sw;            // v in the low nibble, +0 (code 0) in the high one
    bad_hi += hi != (sw << 4);     // v in the high nibble
  }
  atomicAdd(&counts[0], n);
  atomicAdd(&counts[1], bad_lo);
  atomicAdd(&counts[2], bad_hi);
}

// The plain E4M3FN rule for t >= 0: saturate at 448 (0x7E); t >= 2^-6:
// round the fp32 mantissa to 3 bits (nearest, ties to even) and re-bias the
// exponent from 127 to 7; below: the nearest multiple of 2^-9 (ties even),
// found by adding 2^14, whose fp32 spacing is 2^-9.
__device__ uint32_t e4m3_code_rule(float t) {
  if (t >= 448.0f) return 0x7Eu;
  const uint32_t tb = __float_as_uint(t);
  if (tb >= 0x3C800000u) return ((tb + 0x7FFFFu + ((tb >> 20) & 1u)) >> 20) - (120u << 3);
  return __float_as_uint(t + 16384.0f) - 0x46800000u;
}
// value of an E4M3FN code: e ? 2^(e-7) * (1 + f/8) : f * 2^-9
__device__ float e4m3_value_rule(uint32_t c) {
  const uint32_t e = c >> 3, f = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (f << 20)) : (float)f * 0.001953125f;
}

__global__ void e4m3_exhaustive_kernel(unsigned long long* counts) {
  const uint32_t stride = gridDim.x * blockDim.x;
  unsigned long long n = 0, bad = 0;
  for (uint32_t p = blockIdx.x * blockDim.x + threadIdx.x; p <= 0x7F800000u; p += stride) {
    const float t = __uint_as_float(p);
    n++;
    bad += e4m3_code(t) != e4m3_code_rule(t);
  }
  atomicAdd(&counts[0], n);
  atomicAdd(&counts[1], bad);
  if (blockIdx.x == 0 && threadIdx.x <= 0x7Eu)
    atomicAdd(&counts[2], (unsigned long long)(__float_as_uint(e4m3_value(threadIdx.x)) !=
                                               __float_as_uint(e4m3_value_rule(threadIdx.x))));
}

// one workgroup per line amax A (bf16 pattern 1..0x7F7F), b over 0..A
__global__ void block_step_exhaustive_kernel(unsigned long long* counts) {
  const uint32_t A16 = 1u + blockIdx.x;
  const float A = __uint_as_float(A16 << 16);
  const float s = A / 2688.0f, ys = 1.0f / s;
  unsigned long long n = 0, badS = 0, badm = 0;
  for (uint32_t b16 = threadIdx.x; b16 <= A16; b16 += blockDim.x) {
    const float b = __uint_as_float(b16 << 16);
    float m1, m2;
    const uint32_t S1 = block_scale(b, s, &m1);
    const uint32_t S2 = block_step(b, s, ys, &m2);
    n++;
    badS += S1 != S2;
    badm += __float_as_uint(m1) != __float_as_uint(m2);
  }
  atomicAdd(&counts[0], n);
  atomicAdd(&counts[1], badS);
  atomicAdd(&counts[2], badm);
}

__global__ void block_step_sample_kernel(const uint16_t* b16, const uint16_t* A16, int64_t n, uint8_t* S,
                                         float* m) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float A = __uint_as_float((uint32_t)A16[i] << 16);
  const float s = A / 2688.0f, ys = 1.0f / s;
  float mm;
  S[i] = (uint8_t)block_step(__uint_as_float((uint32_t)b16[i] << 16), s, ys, &mm);
  m[i] = mm;
}

__global__ void fp4_codes_kernel(const float* v, int64_t n, uint8_t* codes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  codes[i] = (uint8_t)(FP4X2(0u, v[i], 0.0f, 0) & 0xFu);
}

// out[2 * (4 * byte + sel) + h]: nibble h of `byte` placed at byte position
// sel of a word whose other bytes are 0x5A, decoded with unit scale.
__global__ void fp4_decode_kernel(float* out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. 1023
  if (t >= 1024) return;
  const uint32_t byte = t >> 2, sel = t & 3;
  const uint32_t w = (0x5A5A5A5Au & ~(0xFFu << (8 * sel))) | (byte << (8 * sel));
  float lo, hi;
  switch (sel) {
    case 0: { const auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); lo = q[0]; hi = q[1]; break; }
    case 1: { const auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); lo = q[0]; hi = q[1]; break; }
    case 2: { const auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); lo = q[0]; hi = q[1]; break; }
    default: { const auto q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); lo = q[0]; hi = q[1]; break; }
  }
  out[2 * t] = lo;
  out[2 * t + 1] = hi;
}

// d over every fp32 pattern in [2^-126, 2^126)
__global__ void rcp_exhaustive_kernel(unsigned long long* counts) {
  const uint32_t stride = gridDim.x * blockDim.x;
  unsigned long long n = 0, bad = 0;
  for (uint32_t p = 0x00800000u + blockIdx.x * blockDim.x + threadIdx.x; p < 0x7E800000u; p += stride) {
    const float d = __uint_as_float(p);
    n++;
    bad += __float_as_uint(rcp_rn(d)) != __float_as_uint(1.0f / d);
  }
  atomicAdd(&counts[0], n);
  atomicAdd(&counts[1], bad);
}

// b over every finite non-negative bf16 pattern (0 .. 0x7F7F)
__global__ void div6_exhaustive_kernel(unsigned long long* counts) {
  const uint32_t b16 = blockIdx.x * blockDim.x + threadIdx.x;
  if (b16 > 0x7F7Fu) return;
  const float b = __uint_as_float(b16 << 16);
  atomicAdd(&counts[0], 1ull);
  if (__float_as_uint(div6_bf16(b)) != __float_as_uint(b / 6.0f)) atomicAdd(&counts[1], 1ull);
}

// one work-group per (line amax A = bf16 pattern 1..0x7F7F, bound 1..448);
// b over every bf16 pattern 0..A, both candidates (u = b/6 and b/4):
// quot_fast against the IEEE quotient u/s, by bits and by E4M3 code.  Lines
// with s < 2^-112 are skipped (they keep the IEEE division) and counted.
__global__ void quot_4o6_exhaustive_kernel(unsigned long long* counts) {
  const uint32_t A16 = 1u + blockIdx.x;
  const float A = __uint_as_float(A16 << 16);
  const float s = A / (6.0f * (float)(1u + blockIdx.y));
  if (!(s >= 0x1p-112f)) {
    if (threadIdx.x == 0) atomicAdd(&counts[3], 1ull);
    return;
  }
  const float ys = 1.0f / s;
  unsigned long long n = 0, badt = 0, badS = 0;
  for (uint32_t b16 = threadIdx.x; b16 <= A16; b16 += blockDim.x) {
    const float b = __uint_as_float(b16 << 16);
    const float u6 = b / 6.0f, u4 = b * 0.25f;
    const float e6 = u6 / s, f6 = quot_fast(u6, s, ys);
    const float e4 = u4 / s, f4 = quot_fast(u4, s, ys);
    n += 2;
    badt += (__float_as_uint(e6) != __float_as_uint(f6)) + (__float_as_uint(e4) != __float_as_uint(f4));
    badS += (e4m3_code(e6) != e4m3_code(f6)) + (e4m3_code(e4) != e4m3_code(f4));
  }
  atomicAdd(&counts[0], n);
  atomicAdd(&counts[1], badt);
  atomicAdd(&counts[2], badS);
}

int status() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

// counts (device, 3 x u64, zeroed by the caller): patterns, low-nibble and
// high-nibble mismatches.
int selftest_fp4_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(fp4_exhaustive_kernel, dim3(4096), dim3(256), 0, 0, counts, 0u);
  hipLaunchKernelGGL(fp4_exhaustive_kernel, dim3(4096), dim3(256), 0, 0, counts, 0x80000000u);
  return status();
}

// counts (device, 3 x u64, zeroed by the caller): encoded patterns, encode
// mismatches, decode mismatches.
int selftest_e4m3_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(e4m3_exhaustive_kernel, dim3(4096), dim3(256), 0, 0, counts);
  return status();
}

// counts (device, 3 x u64, zeroed by the caller): pairs, scale-code and
// multiplier-bit mismatches.
int selftest_block_step_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(block_step_exhaustive_kernel, dim3(0x7F7F), dim3(256), 0, 0, counts);
  return status();
}

int selftest_block_step_sample(const uint16_t* b16, const uint16_t* A16, int64_t n, uint8_t* S, float* m) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(block_step_sample_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, b16, A16, n,
                     S, m);
  return status();
}

int selftest_fp4_codes(const float* v, int64_t n, uint8_t* codes) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(fp4_codes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, 0, v, n, codes);
  return status();
}

// counts (device, 2 x u64, zeroed by the caller): values, mismatches.
int selftest_rcp_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(rcp_exhaustive_kernel, dim3(4096), dim3(256), 0, 0, counts);
  return status();
}
int selftest_div6_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(div6_exhaustive_kernel, dim3(128), dim3(256), 0, 0, counts);
  return status();
}

// counts (device, 4 x u64, zeroed by the caller): quotients checked, bit
// mismatches, E4M3-code mismatches, (A, bound) lines skipped.
int selftest_quot_4o6_exhaustive(unsigned long long* counts) {
  hipLaunchKernelGGL(quot_4o6_exhaustive_kernel, dim3(0x7F7F, 448), dim3(256), 0, 0, counts);
  return status();
}

// out: device fp32[2048] (see fp4_decode_kernel).
int selftest_fp4_decode(float* out) {
  hipLaunchKernelGGL(fp4_decode_kernel, dim3(4), dim3(256), 0, 0, out);
  return status();
}

}  // extern "C"
