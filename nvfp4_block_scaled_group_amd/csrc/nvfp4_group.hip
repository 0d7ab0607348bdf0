// nvfp4_group.hip -- grouped, row-scaled (per-token) NVFP4 amax + cast for
// packed MoE activations on MI355X (gfx950), behind the C ABI declared in
// include/nvfp4_group.h.
//
// Operation (cited by page title and section):
//  * "[Common] Single-launch grouped row-scaled NVFP4 cast" (TransformerEngine
//    issue 3649), Description: a grouped amax over the packed (sum_M, K)
//    buffer gives rowwise [sum_M] and columnwise [num_experts*K] amax in one
//    pass; a grouped cast consumes them; graph-safe twins read the routing
//    from device offsets and share the device body (byte-identical output).
//  * "Implement per-token NVFP4 fprop recipe" (TransformerEngine PR 2931):
//    one amax per row, E2M1 data, one E4M3 scale per 16 elements.
//  * "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
//    GroupedLinear" (TransformerEngine PR 3324): per-column amax for the
//    transposed (columnwise) operand.
//
// Design (bandwidth-bound, no MFMA):
//  * Work unit = a tile of 128 rows x 256 columns.  Expert groups are
//    multiples of 128 rows, so each tile lies in one expert; the tile's
//    expert comes from a binary search over the inclusive row ends (kernel
//    arguments for host splits, device memory for the graph-safe calls: the
//    only difference between the two paths).
//  * A workgroup is 4 wave64s; a wave covers 128 rows x 64 columns and lane
//    L holds rows 16*(L%8)..+15 and columns 8*(L/8)..+7 of it: 16 coalesced
//    16-byte loads (8 lanes read 128 contiguous bytes of a row).  A rowwise
//    block (16 columns) is the lane's 8 values plus those of lane L^8 (one
//    DPP swap); a columnwise block (16 rows) is entirely inside one lane, so
//    the transposed cast needs no LDS round trip, and 8 neighbouring lanes
//    write 64 contiguous bytes of a transposed line.
//  * amax: abs-max on bf16 bit patterns (integer max orders non-negative
//    floats), reduced across lanes, then one atomic max per row and per
//    column per tile into zero-initialised outputs (atomic max of the fp32
//    bit patterns of non-negative values is order independent, so results
//    are deterministic).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>

#include "../../include/nvfp4_group.h"

namespace {

constexpr int kThreads = 256;    // 4 wave64
constexpr int kTileRows = 128;   // expert groups are multiples of 128 rows
constexpr int kTileCols = 256;   // 4 waves x 64 columns

// ------------------------------------------------------------------ routing

struct Routing {
  const int32_t* d_offs;  // device inclusive row ends (graph-safe) or null
  int32_t* d_status;      // graph-safe status word
  int32_t num_experts;
  int32_t m_capacity;     // rows in the buffers
  int32_t h_offs[NVFP4G_MAX_EXPERTS_HOST];  // host-split inclusive row ends
};

__device__ __forceinline__ int32_t route_end(const Routing& R, int e) {
  return R.d_offs ? R.d_offs[e] : R.h_offs[e];
}

// Device routing check (graph-safe calls only): every wave checks all
// offsets; on failure the status bits are ORed in and the caller returns.
__device__ bool routing_ok(const Routing& R) {
  if (!R.d_offs) return true;
  const int lane = threadIdx.x & 63;
  uint32_t bad = 0;
  for (int e = lane; e < R.num_experts; e += 64) {
    const int32_t hi = R.d_offs[e];
    const int32_t lo = e ? R.d_offs[e - 1] : 0;
    if (hi < lo) bad |= NVFP4G_DEV_NONMONO;
    if (hi & (kTileRows - 1)) bad |= NVFP4G_DEV_UNALIGNED;
    if (hi > R.m_capacity) bad |= NVFP4G_DEV_OVERFLOW;
  }
  uint32_t all = 0;
  if (__ballot(bad & NVFP4G_DEV_UNALIGNED)) all |= NVFP4G_DEV_UNALIGNED;
  if (__ballot(bad & NVFP4G_DEV_NONMONO)) all |= NVFP4G_DEV_NONMONO;
  if (__ballot(bad & NVFP4G_DEV_OVERFLOW)) all |= NVFP4G_DEV_OVERFLOW;
  if (all && lane == 0 && R.d_status) atomicOr(R.d_status, (int32_t)all);
  return all == 0;
}

// Expert owning row `row` (< total): first e with end(e) > row.
__device__ __forceinline__ int find_expert(const Routing& R, int32_t row,
                                           int32_t* begin, int32_t* end) {
  int lo = 0, hi = R.num_experts - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (route_end(R, mid) > row) hi = mid; else lo = mid + 1;
  }
  *end = route_end(R, lo);
  *begin = lo ? route_end(R, lo - 1) : 0;
  return lo;
}

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

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- numerics

// E4M3FN code of t >= 0 (finite or +inf): nearest, ties to even, saturating
// at 448 (0x7E).  Normal range: round the fp32 mantissa to 3 bits and
// re-bias the exponent (7 - 127); subnormal range (t < 2^-6): the nearest
// multiple of 2^-9, found by adding 2^14 (whose fp32 spacing is 2^-9).
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  if (t >= 448.0f) return 0x7Eu;
  const uint32_t tb = __float_as_uint(t);
  if (tb >= 0x3C800000u) {  // t >= 2^-6
    const uint32_t r = (tb + 0x7FFFFu + ((tb >> 20) & 1u)) >> 20;
    return r - (120u << 3);
  }
  return __float_as_uint(t + 16384.0f) - 0x46800000u;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, f = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (f << 20))
           : (float)f * 0.001953125f;  // f * 2^-9, exact
}

// Block step: E4M3 scale code of a block with amax b on a line with scale s,
// and the element multiplier m = 1 / (value(S) * s).
__device__ __forceinline__ uint32_t block_scale(float b, float s, float* m) {
  const float t = (s == 0.0f) ? 0.0f : (b / 6.0f) / s;
  const uint32_t S = e4m3_code(t);
  const float d = e4m3_value(S) * s;
  *m = (d == 0.0f) ? 0.0f : fminf(1.0f / d, FLT_MAX);
  return S;
}

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

// Two packed bf16 (element 2j low, 2j+1 high) -> one FP4x2 byte.
__device__ __forceinline__ uint32_t enc_pair(uint32_t w, float m) {
  return e2m1_code(bf16lo(w) * m) | (e2m1_code(bf16hi(w) * m) << 4);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ------------------------------------------------------------------ kernels

// Zero the amax outputs (atomics accumulate into them).  Rows at or beyond
// the routed total are left untouched.
__global__ __launch_bounds__(kThreads) void amax_init_kernel(
    Routing R, int64_t k, float* __restrict__ row_amax, float* __restrict__ col_amax) {
  if (!routing_ok(R)) return;
  const int64_t nrow = row_amax ? (int64_t)route_end(R, R.num_experts - 1) : 0;
  const int64_t ncol = col_amax ? (int64_t)R.num_experts * k : 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nrow + ncol; i += stride) {
    if (i < nrow) row_amax[i] = 0.0f; else col_amax[i - nrow] = 0.0f;
  }
}

// Grouped amax: grid (row tiles, column chunks).
__global__ __launch_bounds__(kThreads) void group_amax_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R,
    uint32_t* __restrict__ row_amax, uint32_t* __restrict__ col_amax) {
  __shared__ uint32_t red[4][64];
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const int32_t row0 = (int32_t)blockIdx.x * kTileRows;
  if (row0 >= total) return;
  int32_t rbeg, rend;
  const int e = find_expert(R, row0, &rbeg, &rend);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rb = lane & 7, cg = lane >> 3;
  const int64_t col = (int64_t)blockIdx.y * kTileCols + wave * 64 + cg * 8;
  const bool active = col < k;

  uint32_t v[16][4];
  const uint16_t* p = x + ((int64_t)row0 + 16 * rb) * k + col;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint4 q = active ? ldg16(p + i * k) : make_uint4(0, 0, 0, 0);
    v[i][0] = q.x & 0x7FFF7FFFu; v[i][1] = q.y & 0x7FFF7FFFu;
    v[i][2] = q.z & 0x7FFF7FFFu; v[i][3] = q.w & 0x7FFF7FFFu;
  }

  if (row_amax) {
    // per row pair (2p, 2p+1): low half = row 2p, high half = row 2p+1
    uint32_t rp[8];
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      const uint32_t a = pkmax(pkmax(v[2 * pr][0], v[2 * pr][1]), pkmax(v[2 * pr][2], v[2 * pr][3]));
      const uint32_t b = pkmax(pkmax(v[2 * pr + 1][0], v[2 * pr + 1][1]),
                               pkmax(v[2 * pr + 1][2], v[2 * pr + 1][3]));
      const uint32_t lo = (a & 0xFFFFu) | (b << 16);
      const uint32_t hi = (a >> 16) | (b & 0xFFFF0000u);
      uint32_t r = pkmax(lo, hi);
      r = pkmax(r, swap8(r));
      r = pkmax(r, (uint32_t)__shfl_xor((int)r, 16));
      r = pkmax(r, (uint32_t)__shfl_xor((int)r, 32));
      rp[pr] = r;
    }
    if (cg == 0) {
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) red[wave][rb * 8 + pr] = rp[pr];
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int t = threadIdx.x;
      const uint32_t r = pkmax(pkmax(red[0][t], red[1][t]), pkmax(red[2][t], red[3][t]));
      const int64_t row = (int64_t)row0 + 16 * (t >> 3) + 2 * (t & 7);
      atomicMax(row_amax + row, r << 16);
      atomicMax(row_amax + row + 1, r & 0xFFFF0000u);
    }
  }

  if (col_amax) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t m = v[0][j];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = pkmax(m, v[i][j]);
      m = pkmax(m, dpp_x1(m));
      m = pkmax(m, dpp_x2(m));
      m = pkmax(m, dpp_hmirror(m));
      c[j] = m;
    }
    // lanes rb = 0..3 each publish one column pair
    if (active && rb < 4) {
      const uint32_t m = rb == 0 ? c[0] : rb == 1 ? c[1] : rb == 2 ? c[2] : c[3];
      uint32_t* dst = col_amax + (int64_t)e * k + col + 2 * rb;
      atomicMax(dst, m << 16);
      atomicMax(dst + 1, m & 0xFFFF0000u);
    }
  }
}

// Grouped cast: grid (row tiles, column chunks); rowwise and/or columnwise.
__global__ __launch_bounds__(kThreads) void group_cast_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R,
    const float* __restrict__ row_amax, const float* __restrict__ col_amax,
    uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scale) {
  __shared__ float s_row[kTileRows];
  __shared__ float s_col[kTileCols];
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const int32_t row0 = (int32_t)blockIdx.x * kTileRows;
  if (row0 >= total) return;
  int32_t rbeg, rend;
  const int e = find_expert(R, row0, &rbeg, &rend);
  const int64_t me = rend - rbeg;

  const int tid = threadIdx.x;
  const int64_t col_base = (int64_t)blockIdx.y * kTileCols;
  // line scales s = A / (6 * 448), once per line per tile
  if (row_data && tid < kTileRows) s_row[tid] = row_amax[row0 + tid] / 2688.0f;
  if (col_data) {
    const int64_t c = col_base + tid;
    s_col[tid] = c < k ? col_amax[(int64_t)e * k + c] / 2688.0f : 0.0f;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int rb = lane & 7, cg = lane >> 3;
  const int64_t col = col_base + wave * 64 + cg * 8;
  const bool active = col < k;

  uint32_t v[16][4];
  const uint16_t* p = x + ((int64_t)row0 + 16 * rb) * k + col;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint4 q = active ? ldg16(p + i * k) : make_uint4(0, 0, 0, 0);
    v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
  }

  if (row_data) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t a = pkmax(pkmax(v[i][0] & 0x7FFF7FFFu, v[i][1] & 0x7FFF7FFFu),
                               pkmax(v[i][2] & 0x7FFF7FFFu, v[i][3] & 0x7FFF7FFFu));
      uint32_t b16 = hmax(a);
      b16 = max(b16, swap8(b16));
      float m;
      const uint32_t S = block_scale(__uint_as_float(b16 << 16), s_row[16 * rb + i], &m);
      const uint32_t packed = enc_pair(v[i][0], m) | (enc_pair(v[i][1], m) << 8) |
                              (enc_pair(v[i][2], m) << 16) | (enc_pair(v[i][3], m) << 24);
      const int64_t r = (int64_t)row0 + 16 * rb + i;
      if (active) {
        *reinterpret_cast<uint32_t*>(row_data + r * (k / 2) + col / 2) = packed;
        if (!(cg & 1)) row_scale[r * (k / 16) + col / 16] = (uint8_t)S;
      }
    }
  }

  if (col_data) {
    uint8_t* cd = col_data + k * (int64_t)rbeg / 2;
    uint8_t* cs = col_scale + k * (int64_t)rbeg / 16;
    const int64_t rofs = (int64_t)row0 - rbeg + 16 * rb;  // row within expert
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = pkmax(mx, v[i][j >> 1] & 0x7FFF7FFFu);
      const uint32_t b16 = (j & 1) ? (mx >> 16) : (mx & 0xFFFFu);
      float m;
      const uint32_t S = block_scale(__uint_as_float(b16 << 16), s_col[wave * 64 + cg * 8 + j], &m);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = v[i][j >> 1];
        lo |= e2m1_code(((j & 1) ? bf16hi(w) : bf16lo(w)) * m) << (4 * i);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = v[8 + i][j >> 1];
        hi |= e2m1_code(((j & 1) ? bf16hi(w) : bf16lo(w)) * m) << (4 * i);
      }
      if (active) {
        const int64_t c = col + j;
        *reinterpret_cast<uint2*>(cd + c * (me / 2) + rofs / 2) = make_uint2(lo, hi);
        cs[c * (me / 16) + rofs / 16] = (uint8_t)S;
      }
    }
  }
}

// ------------------------------------------------------------- host side

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int hip_status() {
  return hipGetLastError() == hipSuccess ? NVFP4G_OK : NVFP4G_EHIP;
}

// Common static checks; fills R (all but the offsets).
int check_common(const uint16_t* x, int64_t rows, int64_t k, int32_t E, Routing* R) {
  if (k <= 0 || k % 16 != 0 || k > (int64_t)1 << 30) return NVFP4G_EINVAL;
  if (rows < 0 || rows > INT32_MAX - kTileRows) return NVFP4G_EINVAL;
  if (rows > 0 && x == nullptr) return NVFP4G_EINVAL;
  if (!aligned(x, 16)) return NVFP4G_EALIGN;
  R->num_experts = E;
  R->m_capacity = (int32_t)rows;
  R->d_offs = nullptr;
  R->d_status = nullptr;
  return NVFP4G_OK;
}

int host_routing(const int64_t* h_splits, int64_t sum_m, int32_t E, Routing* R) {
  if (E < 1 || E > NVFP4G_MAX_EXPERTS_HOST) return NVFP4G_EINVAL;
  if (!h_splits) return NVFP4G_EINVAL;
  int64_t acc = 0;
  for (int32_t e = 0; e < E; ++e) {
    const int64_t m = h_splits[e];
    if (m < 0 || m % kTileRows != 0) return NVFP4G_ESPLITS;
    acc += m;
    if (acc > sum_m) return NVFP4G_ESPLITS;
    R->h_offs[e] = (int32_t)acc;
  }
  return acc == sum_m ? NVFP4G_OK : NVFP4G_ESPLITS;
}

int check_cast_outputs(const float* row_amax, const float* col_amax, const uint8_t* row_data,
                       const uint8_t* row_scale, const uint8_t* col_data, const uint8_t* col_scale) {
  if (row_data && (!row_scale || !row_amax)) return NVFP4G_EINVAL;
  if (col_data && (!col_scale || !col_amax)) return NVFP4G_EINVAL;
  if (!aligned(row_data, 16) || !aligned(row_scale, 16) || !aligned(col_data, 16) ||
      !aligned(col_scale, 16) || !aligned(row_amax, 4) || !aligned(col_amax, 4))
    return NVFP4G_EALIGN;
  return NVFP4G_OK;
}

dim3 tile_grid(int64_t rows, int64_t k) {
  return dim3((unsigned)((rows + kTileRows - 1) / kTileRows), (unsigned)((k + kTileCols - 1) / kTileCols));
}

int launch_amax(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, float* row_amax,
                float* col_amax, hipStream_t st) {
  if (!row_amax && !col_amax) return NVFP4G_OK;
  const int64_t n = (row_amax ? rows : 0) + (col_amax ? (int64_t)R.num_experts * k : 0);
  const unsigned init_blocks = (unsigned)std::min<int64_t>(std::max<int64_t>((n + kThreads - 1) / kThreads, 1), 4096);
  hipLaunchKernelGGL(amax_init_kernel, dim3(init_blocks), dim3(kThreads), 0, st, R, k, row_amax, col_amax);
  if (rows > 0)
    hipLaunchKernelGGL(group_amax_kernel, tile_grid(rows, k), dim3(kThreads), 0, st, x, k, R,
                       reinterpret_cast<uint32_t*>(row_amax), reinterpret_cast<uint32_t*>(col_amax));
  return hip_status();
}

int launch_cast(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, const float* row_amax,
                const float* col_amax, uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                uint8_t* col_scale, hipStream_t st) {
  if ((!row_data && !col_data) || rows == 0) return NVFP4G_OK;
  hipLaunchKernelGGL(group_cast_kernel, tile_grid(rows, k), dim3(kThreads), 0, st, x, k, R, row_amax,
                     col_amax, row_data, row_scale, col_data, col_scale);
  return hip_status();
}

int graph_routing(const int32_t* d_offs, int32_t* d_status, int32_t E, int64_t m_capacity, Routing* R) {
  if (E < 1 || E > NVFP4G_MAX_EXPERTS_DEVICE) return NVFP4G_EINVAL;
  if (!d_offs || !d_status || m_capacity % kTileRows != 0) return NVFP4G_EINVAL;
  if (!aligned(d_offs, 4) || !aligned(d_status, 4)) return NVFP4G_EALIGN;
  R->d_offs = d_offs;
  R->d_status = d_status;
  return NVFP4G_OK;
}

}  // namespace

// ------------------------------------------------------------------- C ABI

extern "C" {

int nvfp4_group_amax(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts,
                     const int64_t* h_splits, float* row_amax, float* col_amax, void* stream) {
  Routing R;
  int rc = check_common(x, sum_m, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  if (!aligned(row_amax, 4) || !aligned(col_amax, 4)) return NVFP4G_EALIGN;
  return launch_amax(x, sum_m, k, R, row_amax, col_amax, (hipStream_t)stream);
}

int nvfp4_group_cast(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts,
                     const int64_t* h_splits, const float* row_amax, const float* col_amax,
                     uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale,
                     void* stream) {
  Routing R;
  int rc = check_common(x, sum_m, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  return launch_cast(x, sum_m, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale,
                     (hipStream_t)stream);
}

int nvfp4_group_amax_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                               const int32_t* d_offs, float* row_amax, float* col_amax,
                               int32_t* d_status, void* stream) {
  Routing R;
  int rc = check_common(x, m_capacity, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  if (!aligned(row_amax, 4) || !aligned(col_amax, 4)) return NVFP4G_EALIGN;
  return launch_amax(x, m_capacity, k, R, row_amax, col_amax, (hipStream_t)stream);
}

int nvfp4_group_cast_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                               const int32_t* d_offs, const float* row_amax, const float* col_amax,
                               uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                               uint8_t* col_scale, int32_t* d_status, void* stream) {
  Routing R;
  int rc = check_common(x, m_capacity, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  return launch_cast(x, m_capacity, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale,
                     (hipStream_t)stream);
}

int nvfp4_group_quantize(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts,
                         const int64_t* h_splits, float* row_amax, float* col_amax, uint8_t* row_data,
                         uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale, void* stream) {
  Routing R;
  int rc = check_common(x, sum_m, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = launch_amax(x, sum_m, k, R, row_data ? row_amax : nullptr, col_data ? col_amax : nullptr, st)))
    return rc;
  return launch_cast(x, sum_m, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale, st);
}

int nvfp4_group_quantize_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                                   const int32_t* d_offs, float* row_amax, float* col_amax,
                                   uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                                   uint8_t* col_scale, int32_t* d_status, void* stream) {
  Routing R;
  int rc = check_common(x, m_capacity, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  hipStream_t st = (hipStream_t)stream;
  if ((rc = launch_amax(x, m_capacity, k, R, row_data ? row_amax : nullptr, col_data ? col_amax : nullptr,
                        st)))
    return rc;
  return launch_cast(x, m_capacity, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale, st);
}

const char* nvfp4_group_strerror(int status) {
  switch (status) {
    case NVFP4G_OK: return "ok";
    case NVFP4G_EINVAL: return "invalid argument (size, expert count, NULL pointer or direction)";
    case NVFP4G_ESPLITS: return "invalid host splits (negative, not a multiple of 128, or sum != sum_m)";
    case NVFP4G_EALIGN: return "misaligned pointer (x/data/scales need 16 bytes, amax 4)";
    case NVFP4G_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
