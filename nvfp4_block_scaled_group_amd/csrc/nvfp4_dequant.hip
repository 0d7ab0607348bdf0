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
// i/2 and its scale in byte i/16, and is written to out[i] (fp32).  One
// thread decodes one 16-element block: an 8-byte data load, one scale byte,
// one line amax, four 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_common.hpp"
#include "nvfp4_numerics.hpp"

namespace {

using namespace nvfp4g;

// Value of a 4-bit E2M1 code: magnitudes 0, 0.5 for codes 0, 1; for codes
// 2..7 the fp32 pattern with exponent (code >> 1) - 1 and mantissa bit code & 1.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t mag = code & 7u;
  const float v = mag >= 2u ? __uint_as_float((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22))
                            : (float)mag * 0.5f;
  return __uint_as_float(__float_as_uint(v) | ((code & 8u) << 28));
}

// Line-amax index of element i in the columnwise layout: expert e owns the
// elements [K*r_e, K*r_{e+1}), line c = (i - K*r_e) / M_e.
__device__ __forceinline__ int64_t col_line(const Routing& R, int64_t k, int64_t i) {
  int lo = 0, hi = R.num_experts - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)route_end_lane(R, mid) * k > i) hi = mid; else lo = mid + 1;
  }
  const int64_t rb = lo ? route_end_lane(R, lo - 1) : 0;
  const int64_t me = route_end_lane(R, lo) - rb;
  return (int64_t)lo * k + (i - k * rb) / me;
}

// columnwise = false: line = i / k (rowwise); true: col_line (needs R).
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ data, const uint8_t* __restrict__ scale, const float* __restrict__ amax,
    int64_t k, int64_t n_elems, bool columnwise, Routing R, float* __restrict__ out) {
  if (columnwise && !routing_ok(R)) return;
  if (columnwise) n_elems = k * route_end(R, R.num_experts - 1);
  const int64_t nblocks = n_elems / 16;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t i = 16 * b;
    const int64_t line = columnwise ? col_line(R, k, i) : i / k;
    const float s = amax[line] / 2688.0f;
    const float S = e4m3_value(scale[b]);
    const uint2 q = *reinterpret_cast<const uint2*>(data + 8 * b);
    float4 o[4];
    float* f = reinterpret_cast<float*>(o);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t word = j < 8 ? q.x : q.y;
      const uint32_t code = (word >> (4 * (j & 7))) & 15u;
      f[j] = (e2m1_value(code) * S) * s;
    }
    float4* dst = reinterpret_cast<float4*>(out + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = o[j];
  }
}

int launch_dequant(const uint8_t* data, const uint8_t* scale, const float* amax, int64_t k, int64_t n_elems,
                   bool columnwise, const Routing& R, float* out, hipStream_t st) {
  const int64_t nblocks = n_elems / 16;
  if (nblocks == 0 && !columnwise) return NVFP4G_OK;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((nblocks + kThreads - 1) / kThreads, 8192));
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
