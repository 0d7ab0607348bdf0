// nvfp4_dequant.hip -- GPU dequantisation of row-scaled NVFP4 (the inverse of
// the grouped cast), behind the C ABI of include/nvfp4_group.h.
//
// "Implement per-token NVFP4 fprop recipe" (TransformerEngine PR 2931),
// Important Files Changed: the dequant kernel takes the amax per row and
// looks it up by the element's row.  Here every line -- a row of the rowwise
// output, or one column line of an expert in the columnwise (transposed)
// output -- is dequantised with its own amax A and the E4M3 scale S of each
// 16-element block:  x^ = (value(code) * value(S)) * (A / 2688),  the first
// product exact, one rounding in the second, the same order as the oracle's
// decode.
//
// Both outputs are laid out like the data they decode: element i of the
// rowwise output (row i / K) or of the columnwise output (expert blocks of
// [K, M_e] lines, concatenated in expert order) has its data nibble in byte
// i/2 and its scale in byte i/16, and is written to out[i] (fp32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_common.hpp"
#include "nvfp4_numerics.hpp"

namespace {

using namespace nvfp4g;

// Work unit: a chunk of 2048 consecutive output elements per wave.  Lane l
// decodes the four elements 256g + 4l .. +3 of the chunk for g = 0..7, so
// each of the wave's eight 16-byte stores covers 1 KB of contiguous output.
// A 16-element block (and so a line) never splits across a lane's group of
// four.  In the columnwise layout expert e's span [K*r_e, K*r_{e+1}) is a
// multiple of 2048 elements (r_e a multiple of 128, K of 16), so a chunk
// lies in one expert: the expert search and the 64-bit division that places
// the chunk on its first line are per chunk and wave-uniform.  All loads of
// a chunk (codes, scale bytes, line amax) are issued before any is used, so
// a chunk costs one memory round trip.
constexpr int kChunk = 2048;
constexpr int kGroups = kChunk / 256;

// Magnitudes of the E2M1 codes 0..7 in units of 0.5 (0 1 2 3 4 6 8 12),
// one nibble each.
constexpr uint32_t kE2m1Halves = 0xC8643210u;

// value(code) * value(S) * s for the four codes of a 16-bit group, with
// hS = value(S) / 2: n * hS is the exact product value(code) * value(S) (a
// 4-bit integer times an E4M3 value), so the one rounding is the product
// with s, as in (value(code) * value(S)) * s; the sign is applied last
// (rounding to nearest is symmetric).
// value(S) of an E4M3FN scale code by bit arithmetic: e ? 2^(e-7)*(1 + f/8)
// : f * 2^-9.  (The hardware fp8 convert gives the same values; in this
// kernel the integer form measured ~2% faster.)
__device__ __forceinline__ float scale_value(uint32_t c) {
  const uint32_t e = c >> 3, f = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (f << 20)) : (float)f * 0.001953125f;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 decode4(uint32_t q, float hS, float s) {
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t c = (q >> (4 * j)) & 15u;
    const float mag = (float)((kE2m1Halves >> ((c & 7u) * 4u)) & 15u) * hS;
    r[j] = __uint_as_float(__float_as_uint(mag * s) | ((c & 8u) << 28));
  }
  return f32x4{r[0], r[1], r[2], r[3]};
}

__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ data, const uint8_t* __restrict__ scale, const float* __restrict__ amax,
    int64_t k, int64_t n_elems, bool columnwise, Routing R, float* __restrict__ out) {
  if (columnwise && !routing_ok(R)) return;
  if (columnwise) n_elems = k * route_end(R, R.num_experts - 1);
  const int64_t nchunks = (n_elems + kChunk - 1) / kChunk;
  const uint32_t lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t c = uni((uint32_t)(blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6))); c < nchunks;
       c += nwaves) {
    const int64_t c0 = c * kChunk;
    // the chunk's lines: element c0 + o lies on line  lbase + (rem0 + o) / len
    int64_t lbase, rem0, len;
    if (columnwise) {
      int32_t rbeg, rend;
      const int e = find_expert(R, (int32_t)(c0 / k), &rbeg, &rend);
      len = rend - rbeg;
      const int64_t t = c0 - k * rbeg;
      lbase = (int64_t)e * k + t / len;
      rem0 = t % len;
    } else {
      len = k;
      lbase = c0 / k;
      rem0 = c0 % k;
    }
    const uint32_t ulen = uni((uint32_t)len), urem = uni((uint32_t)rem0);
    const float inv_len = 1.0f / (float)ulen;
    const uint32_t left = (uint32_t)min<int64_t>(n_elems - c0, kChunk);  // elements of this chunk
    const uint8_t* dch = data + c0 / 2;
    const uint8_t* sch = scale + c0 / 16;
    const float* ach = amax + uni(lbase);
    float* och = out + c0;
    uint32_t q[kGroups], sb[kGroups];
    float A[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t o = 256u * g + 4u * lane;
      const bool live = o < left;
      // line offset (urem + o) / ulen: float estimate, then one correction
      // step (the estimate is within 1 for quotients below 2^22)
      const uint32_t v = urem + o;
      uint32_t d = (uint32_t)((float)v * inv_len);
      const int32_t rem = (int32_t)(v - d * ulen);
      d = rem < 0 ? d - 1 : (rem >= (int32_t)ulen ? d + 1 : d);
      q[g] = live ? *reinterpret_cast<const uint16_t*>(dch + o / 2) : 0u;
      sb[g] = live ? sch[o / 16] : 0u;
      A[g] = live ? ach[d] : 0.0f;
    }
    // streaming (non-temporal) stores: the fp32 output is written once and
    // is far larger than the caches
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t o = 256u * g + 4u * lane;
      if (o < left) __builtin_nontemporal_store(decode4(q[g], scale_value(sb[g]) * 0.5f, A[g] / 2688.0f),
                                                reinterpret_cast<f32x4*>(och + o));
    }
  }
}

int launch_dequant(const uint8_t* data, const uint8_t* scale, const float* amax, int64_t k, int64_t n_elems,
                   bool columnwise, const Routing& R, float* out, hipStream_t st) {
  if (n_elems == 0) return NVFP4G_OK;
  const int64_t waves = (n_elems + kChunk - 1) / kChunk;
  const unsigned grid = (unsigned)std::min<int64_t>((waves + 3) / 4, 8192);
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(kThreads), 0, st, data, scale, amax, k, n_elems, columnwise,
                     R, out);
  return hip_status();
}

int check_dequant(const uint8_t* data, const uint8_t* scale, const float* amax, int64_t rows, int64_t k,
                  const float* out) {
  if (k <= 0 || k % 16 != 0 || k > kMaxK || rows < 0 || rows > kMaxRows) return NVFP4G_EINVAL;
  if (rows > 0 && (!data || !scale || !amax || !out)) return NVFP4G_EINVAL;
  if (!aligned(data, 16) || !aligned(scale, 16) || !aligned(amax, 4) || !aligned(out, 16)) return NVFP4G_EALIGN;
  return NVFP4G_OK;
}

}  // namespace

extern "C" {

int nvfp4_group_dequant_rowwise(const uint8_t* row_data, const uint8_t* row_scale, const float* row_amax,
                                int64_t rows, int64_t k, float* out, void* stream) {
  int rc = check_dequant(row_data, row_scale, row_amax, rows, k, out);
  if (rc) return rc;
  Routing R;
  R.d_offs = nullptr;
  R.d_status = nullptr;
  R.num_experts = 1;
  R.m_capacity = (int32_t)rows;
  return launch_dequant(row_data, row_scale, row_amax, k, rows * k, false, R, out, (hipStream_t)stream);
}

int nvfp4_group_dequant_columnwise(const uint8_t* col_data, const uint8_t* col_scale, const float* col_amax,
                                   int64_t sum_m, int64_t k, int32_t num_experts, const int64_t* h_splits,
                                   float* out, void* stream) {
  int rc = check_dequant(col_data, col_scale, col_amax, sum_m, k, out);
  if (rc) return rc;
  Routing R;
  if ((rc = check_common(col_data, sum_m, k, num_experts, &R))) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  return launch_dequant(col_data, col_scale, col_amax, k, sum_m * k, true, R, out, (hipStream_t)stream);
}

int nvfp4_group_dequant_columnwise_graphsafe(const uint8_t* col_data, const uint8_t* col_scale,
                                             const float* col_amax, int64_t m_capacity, int64_t k,
                                             int32_t num_experts, const int32_t* d_offs, float* out,
                                             int32_t* d_status, void* stream) {
  int rc = check_dequant(col_data, col_scale, col_amax, m_capacity, k, out);
  if (rc) return rc;
  Routing R;
  if ((rc = check_common(col_data, m_capacity, k, num_experts, &R))) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  return launch_dequant(col_data, col_scale, col_amax, k, m_capacity * k, true, R, out, (hipStream_t)stream);
}

}  // extern "C"
