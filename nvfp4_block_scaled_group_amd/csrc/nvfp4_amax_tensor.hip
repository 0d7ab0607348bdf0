// nvfp4_amax_tensor.hip -- per-tensor amax for casts with row scaling off,
// behind the C ABI of include/nvfp4_group.h.
//
// The row_scaled knob of the four-over-six converter page ("[NVFP4 4over6]
// Add the grouped-experts four-over-six converter", Summary and Review pass)
// switches the per-row amax off; the per-token page ("Implement per-token
// NVFP4 fprop recipe", Description) describes the per-row amax as replacing a
// per-tensor one.  With it off, every line of expert e takes the expert's
// tensor amax A_e = max |x| over all of its rows and columns, delivered as the
// amax vectors the casts consume (row_amax[r] = A_e, col_amax[e*k + c] = A_e),
// so the casts run unchanged.
//
// The grouped amax computes the line maxima; one more launch, one
// work-group per expert, takes their maximum and writes it to every line.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4_group.h"
#include "nvfp4_common.hpp"

namespace {

using namespace nvfp4g;

// One work-group per expert: the maximum of the expert's row amax (or,
// without a rowwise output, of its column amax -- both are the maximum of |x|
// over the expert), then written to all of its lines in both vectors.  An
// expert without rows keeps 0 (its column amax is 0).  The values are
// non-negative floats, so the integer maximum of their bit patterns is their
// maximum.
__global__ __launch_bounds__(kThreads) void amax_tensor_kernel(Routing R, int64_t k, float* __restrict__ row_amax,
                                                                float* __restrict__ col_amax) {
  __shared__ uint32_t l_max[kThreads];
  if (!routing_ok(R)) return;
  const int e = blockIdx.x;
  const int32_t rend = route_end(R, e), rbeg = e ? route_end(R, e - 1) : 0;
  const int tid = threadIdx.x;
  uint32_t m = 0;
  if (row_amax) {
    for (int32_t r = rbeg + tid; r < rend; r += kThreads) m = max(m, __float_as_uint(row_amax[r]));
  } else {
    for (int64_t c = tid; c < k; c += kThreads) m = max(m, __float_as_uint(col_amax[(int64_t)e * k + c]));
  }
  l_max[tid] = m;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) l_max[tid] = max(l_max[tid], l_max[tid + w]);
    __syncthreads();
  }
  const float A = __uint_as_float(l_max[0]);
  if (row_amax)
    for (int32_t r = rbeg + tid; r < rend; r += kThreads) row_amax[r] = A;
  if (col_amax)
    for (int64_t c = tid; c < k; c += kThreads) col_amax[(int64_t)e * k + c] = A;
}

int launch_broadcast(const Routing& R, int64_t k, float* row_amax, float* col_amax, void* stream) {
  if (!row_amax && !col_amax) return NVFP4G_OK;
  hipLaunchKernelGGL(amax_tensor_kernel, dim3((unsigned)R.num_experts), dim3(kThreads), 0, (hipStream_t)stream, R, k,
                     row_amax, col_amax);
  return hip_status();
}

}  // namespace

extern "C" {

int nvfp4_group_amax_tensor(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts,
                            const int64_t* h_splits, float* row_amax, float* col_amax, void* stream) {
  int rc = nvfp4_group_amax(x, sum_m, k, num_experts, h_splits, row_amax, col_amax, stream);
  if (rc) return rc;
  Routing R;
  if ((rc = check_common(x, sum_m, k, num_experts, &R))) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  return launch_broadcast(R, k, row_amax, col_amax, stream);
}

int nvfp4_group_amax_tensor_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                                      const int32_t* d_offs, float* row_amax, float* col_amax, int32_t* d_status,
                                      void* stream) {
  int rc = nvfp4_group_amax_graphsafe(x, m_capacity, k, num_experts, d_offs, row_amax, col_amax, d_status, stream);
  if (rc) return rc;
  Routing R;
  if ((rc = check_common(x, m_capacity, k, num_experts, &R))) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  return launch_broadcast(R, k, row_amax, col_amax, stream);
}

}  // extern "C"
