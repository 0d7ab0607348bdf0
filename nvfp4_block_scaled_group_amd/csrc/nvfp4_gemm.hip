// nvfp4_gemm.hip -- row-scaled NVFP4 grouped GEMM on the MFMA units of gfx950:
// the consumer of the grouped cast, behind the C ABI of include/nvfp4_group.h.
//
// What is computed (cited by page title and section):
//  * "Implement per-token NVFP4 fprop recipe" (TransformerEngine PR 2931),
//    Greptile Summary and its sequence diagram: the forward GEMM runs on the
//    block-scaled FP4 operands with the per-row amax set aside, produces fp32,
//    and its rows are then multiplied by the row amax; the grouped form runs
//    one such GEMM per expert.
//  * "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
//    GroupedLinear" (TransformerEngine PR 3324), Greptile Summary: the weight
//    gradient is an NT GEMM per expert on the columnwise (transposed)
//    operands, each with a per-column amax.
//
// Both forms are "NT" products C[i, j] = sum_t xa[i, t] * xb[j, t] of two
// row-scaled NVFP4 operands stored along the contraction index t, where an
// element decodes to  value(code) * value(S) * (A / 2688)  (A = its line's
// amax, S = its 16-block's E4M3 scale).  The line factor A / 2688 leaves the
// sum, so
//     C[i, j] = (acc[i, j] * (Aa_i / 2688)) * (Ab_j / 2688),
//     acc[i, j] = sum_t (value(qa) * value(Sa)) * (value(qb) * value(Sb)).
// value(code) * value(S) needs at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16; the MFMA multiplies fp16 pairs
// exactly and accumulates in fp32.  The sum is therefore the only rounding
// besides the three fp32 operations of the epilogue.
//
// Design:
//  * Work-group tile 128 (i) x 256 (j), 4 wave64s each computing 64 x 128 with
//    2 x 4 v_mfma_f32_32x32x16_f16; the contraction advances 64 at a time.
//  * Per step each thread loads raw FP4 bytes and E4M3 scale bytes (buffer
//    loads: rows beyond the operand read as zero), decodes them with
//    v_cvt_scalef32_pk_f16_fp4 (scale 1: the exact E2M1 values, two per
//    instruction) and one packed fp16 multiply by value(S) per pair, and
//    stores fp16 rows to LDS (row pitch 144 bytes: 16-byte fragment reads of
//    8 consecutive rows hit distinct banks).  The next step's raw bytes are
//    loaded while the MFMAs of the current step run.
//  * Tile order: work-group ids are remapped so each XCD (own L2) gets a
//    contiguous run of tiles, and inside it groups of 8 row tiles sweep the
//    column tiles together, so A and B slices are shared through L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4_group.h"
#include "nvfp4_common.hpp"
#include "nvfp4_numerics.hpp"

namespace {

using namespace nvfp4g;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;            // tile rows (i)
constexpr int kBN = 256;            // tile columns (j)
constexpr int kBK = 64;             // contraction step
constexpr int kPitch = kBK + 8;     // fp16 per LDS row (144 bytes)
constexpr int kGroupRows = 8;       // row tiles per column sweep

// One NT operand tile: `rows` lines of length L starting at the tile's first
// line; lines at or beyond `valid` read as zero.
struct OperandTile {
  const uint8_t* data;   // first line's codes; line pitch L/2 bytes
  const uint8_t* scale;  // first line's scales; line pitch L/16 bytes
  uint32_t valid;        // lines that exist
};

// Logical tile index: each XCD gets a contiguous run (work-groups are
// dispatched round-robin over the 8 XCDs).
__device__ __forceinline__ uint32_t xcd_logical_id() {
  const uint32_t nb = gridDim.x, L = blockIdx.x;
  const uint32_t xcd = L % kNumXcd, q = nb / kNumXcd, r = nb % kNumXcd;
  return uni(xcd * q + min(xcd, r) + L / kNumXcd);
}

// Grouped order inside `ntm` x `ntn` tiles: groups of kGroupRows row tiles
// walk the column tiles together.
__device__ __forceinline__ void grouped_tile(uint32_t t, uint32_t ntm, uint32_t ntn, uint32_t* tm, uint32_t* tn) {
  const uint32_t g = t / (kGroupRows * ntn), in = t % (kGroupRows * ntn);
  const uint32_t first = g * kGroupRows, gm = min((uint32_t)kGroupRows, ntm - first);
  *tm = uni(first + in % gm);
  *tn = uni(in / gm);
}

// fp16 value of an E4M3 code (exact).
__device__ __forceinline__ _Float16 scale_h(uint32_t code) { return (_Float16)e4m3_value(code & 0xFFu); }

// Decode 8 bytes (16 codes of one block) scaled by value(S) into 16 fp16.
__device__ __forceinline__ void decode_block(uint32_t w0, uint32_t w1, _Float16 s, h8_t* lo, h8_t* hi) {
  const h2_t ss = {s, s};
#define NVFP4G_CVT(w, b) (__builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), 1.0f, (b)) * ss)
  const h2_t p[8] = {NVFP4G_CVT(w0, 0), NVFP4G_CVT(w0, 1), NVFP4G_CVT(w0, 2), NVFP4G_CVT(w0, 3),
                     NVFP4G_CVT(w1, 0), NVFP4G_CVT(w1, 1), NVFP4G_CVT(w1, 2), NVFP4G_CVT(w1, 3)};
#undef NVFP4G_CVT
  *lo = h8_t{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  *hi = h8_t{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// acc[im][in] += A[64 rows of wave] x B[128 rows of wave]^T over the whole
// contraction length L (a multiple of kBK).
__device__ __forceinline__ void gemm_tile(const OperandTile& A, const OperandTile& B, uint32_t L,
                                          f32x16 (&acc)[2][4], _Float16* la, _Float16* lb) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t dpitch = L / 2, spitch = L / 16;
  // A: thread -> line tid/2, half (tid&1) of the 64-element step (16 bytes)
  const uint32_t a_line = tid >> 1, a_half = tid & 1;
  const rsrc_t ad = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A.data), 0, A.valid * dpitch, 0x00020000);
  const rsrc_t as = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(A.scale), 0, A.valid * spitch, 0x00020000);
  const uint32_t a_doff = a_line * dpitch + 16u * a_half, a_soff = a_line * spitch + 2u * a_half;
  // B: thread -> line tid (32 bytes)
  const rsrc_t bd = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(B.data), 0, B.valid * dpitch, 0x00020000);
  const rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(B.scale), 0, B.valid * spitch, 0x00020000);
  const uint32_t b_doff = (uint32_t)tid * dpitch, b_soff = (uint32_t)tid * spitch;

  u32x4 ra, rb0, rb1;
  uint32_t ras, rbs;
  auto load = [&](uint32_t ks) {
    ra = __builtin_amdgcn_raw_buffer_load_b128(ad, a_doff, ks * 32u, 0);
    ras = __builtin_amdgcn_raw_buffer_load_b16(as, a_soff, ks * 4u, 0);
    rb0 = __builtin_amdgcn_raw_buffer_load_b128(bd, b_doff, ks * 32u, 0);
    rb1 = __builtin_amdgcn_raw_buffer_load_b128(bd, b_doff + 16u, ks * 32u, 0);
    rbs = __builtin_amdgcn_raw_buffer_load_b32(bs, b_soff, ks * 4u, 0);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t nk = L / kBK;
  if (nk) load(0);
#pragma unroll 1
  for (uint32_t ks = 0; ks < nk; ++ks) {
    {
      h8_t q0, q1, q2, q3;
      decode_block(ra.x, ra.y, scale_h(ras), &q0, &q1);
      decode_block(ra.z, ra.w, scale_h(ras >> 8), &q2, &q3);
      h8_t* dst = reinterpret_cast<h8_t*>(la + a_line * kPitch + 32 * a_half);
      dst[0] = q0; dst[1] = q1; dst[2] = q2; dst[3] = q3;
      h8_t r0, r1, r2, r3, r4, r5, r6, r7;
      decode_block(rb0.x, rb0.y, scale_h(rbs), &r0, &r1);
      decode_block(rb0.z, rb0.w, scale_h(rbs >> 8), &r2, &r3);
      decode_block(rb1.x, rb1.y, scale_h(rbs >> 16), &r4, &r5);
      decode_block(rb1.z, rb1.w, scale_h(rbs >> 24), &r6, &r7);
      h8_t* dstb = reinterpret_cast<h8_t*>(lb + tid * kPitch);
      dstb[0] = r0; dstb[1] = r1; dstb[2] = r2; dstb[3] = r3;
      dstb[4] = r4; dstb[5] = r5; dstb[6] = r6; dstb[7] = r7;
    }
    __syncthreads();
    if (ks + 1 < nk) load(ks + 1);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      h8_t af[2], bf[4];
#pragma unroll
      for (int im = 0; im < 2; ++im)
        af[im] = *reinterpret_cast<const h8_t*>(la + (wm * 64 + im * 32 + (lane & 31)) * kPitch + 16 * s + 8 * (lane >> 5));
#pragma unroll
      for (int in = 0; in < 4; ++in)
        bf[in] = *reinterpret_cast<const h8_t*>(lb + (wn * 128 + in * 32 + (lane & 31)) * kPitch + 16 * s + 8 * (lane >> 5));
#pragma unroll
      for (int im = 0; im < 2; ++im)
#pragma unroll
        for (int in = 0; in < 4; ++in)
          acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[im], bf[in], acc[im][in], 0, 0, 0);
    }
    __syncthreads();
  }
}

// out[i, j] = (acc * sa[i]) * sb[j] for i < rows_i, j < rows_j; the line
// scales of the tile are staged in LDS first.
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[2][4], const float* a_amax, uint32_t rows_i,
                                         const float* b_amax, uint32_t rows_j, float* out, int64_t ldo,
                                         float* lsa, float* lsb) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < kBM) lsa[tid] = (uint32_t)tid < rows_i ? a_amax[tid] / 2688.0f : 0.0f;
  lsb[tid] = (uint32_t)tid < rows_j ? b_amax[tid] / 2688.0f : 0.0f;
  __syncthreads();
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int in = 0; in < 4; ++in) {
    const uint32_t j = wn * 128 + in * 32 + (lane & 31);
    const float sb = lsb[j];
#pragma unroll
    for (int im = 0; im < 2; ++im)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t i = wm * 64 + im * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (i < rows_i && j < rows_j) out[(int64_t)i * ldo + j] = (acc[im][in][v] * lsa[i]) * sb;
      }
  }
}

// Forward form: expert e's rows of a times b_e^T.  Tiles: 128-row tiles of
// the routed rows (each inside one expert) x 256-column tiles of n.
__global__ __launch_bounds__(kThreads, 2) void gemm_fwd_kernel(
    const uint8_t* __restrict__ a_data, const uint8_t* __restrict__ a_scale, const float* __restrict__ a_amax,
    const uint8_t* __restrict__ b_data, const uint8_t* __restrict__ b_scale, const float* __restrict__ b_amax,
    int64_t n, int64_t k, Routing R, uint32_t ntm, uint32_t ntn, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 la[kBM * kPitch];
  __shared__ __attribute__((aligned(16))) _Float16 lb[kBN * kPitch];
  __shared__ float lsa[kBM], lsb[kBN];
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  uint32_t tm, tn;
  grouped_tile(xcd_logical_id(), ntm, ntn, &tm, &tn);
  const int32_t row0 = (int32_t)(tm * kBM);
  if (row0 >= total) return;
  int32_t rbeg, rend;
  const int e = find_expert(R, row0, &rbeg, &rend);
  const int64_t col0 = (int64_t)tn * kBN;
  const uint32_t cols = (uint32_t)min<int64_t>(n - col0, kBN);
  const int64_t brow0 = (int64_t)e * n + col0;  // first line of b in this tile
  const OperandTile A{a_data + (int64_t)row0 * (k / 2), a_scale + (int64_t)row0 * (k / 16), (uint32_t)kBM};
  const OperandTile B{b_data + brow0 * (k / 2), b_scale + brow0 * (k / 16), cols};
  f32x16 acc[2][4];
#pragma unroll
  for (int im = 0; im < 2; ++im)
#pragma unroll
    for (int in = 0; in < 4; ++in) acc[im][in] = f32x16{};
  gemm_tile(A, B, (uint32_t)k, acc, la, lb);
  epilogue(acc, a_amax + row0, kBM, b_amax + brow0, cols, out + (int64_t)row0 * n + col0, n, lsa, lsb);
}

// Weight-gradient form: for expert e, out_e[i, j] = sum over its rows r of
// xa_e[i, r] * xb_e[j, r], with a and b columnwise cast outputs (expert e's
// lines at byte n*r_e/2 resp. k*r_e/2, line length M_e).  Tiles: per expert,
// 128-line tiles of a x 256-line tiles of b.
__global__ __launch_bounds__(kThreads, 2) void gemm_wgrad_kernel(
    const uint8_t* __restrict__ a_data, const uint8_t* __restrict__ a_scale, const float* __restrict__ a_amax,
    const uint8_t* __restrict__ b_data, const uint8_t* __restrict__ b_scale, const float* __restrict__ b_amax,
    int64_t n, int64_t k, Routing R, uint32_t ntm, uint32_t ntn, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 la[kBM * kPitch];
  __shared__ __attribute__((aligned(16))) _Float16 lb[kBN * kPitch];
  __shared__ float lsa[kBM], lsb[kBN];
  if (!routing_ok(R)) return;
  const uint32_t t = xcd_logical_id(), per = ntm * ntn;
  const int e = (int)uni(t / per);
  uint32_t tm, tn;
  grouped_tile(t % per, ntm, ntn, &tm, &tn);
  const int32_t rend = route_end(R, e), rbeg = e ? route_end(R, e - 1) : 0;
  const uint32_t me = (uint32_t)(rend - rbeg);
  const int64_t i0 = (int64_t)tm * kBM, j0 = (int64_t)tn * kBN;
  const uint32_t rows_i = (uint32_t)min<int64_t>(n - i0, kBM), rows_j = (uint32_t)min<int64_t>(k - j0, kBN);
  const OperandTile A{a_data + n * (int64_t)rbeg / 2 + i0 * (me / 2), a_scale + n * (int64_t)rbeg / 16 + i0 * (me / 16),
                      rows_i};
  const OperandTile B{b_data + k * (int64_t)rbeg / 2 + j0 * (me / 2), b_scale + k * (int64_t)rbeg / 16 + j0 * (me / 16),
                      rows_j};
  f32x16 acc[2][4];
#pragma unroll
  for (int im = 0; im < 2; ++im)
#pragma unroll
    for (int in = 0; in < 4; ++in) acc[im][in] = f32x16{};
  gemm_tile(A, B, me, acc, la, lb);
  epilogue(acc, a_amax + (int64_t)e * n + i0, rows_i, b_amax + (int64_t)e * k + j0, rows_j,
           out + (int64_t)e * n * k + i0 * k + j0, k, lsa, lsb);
}

// ------------------------------------------------------------- host side

constexpr int64_t kGemmMaxN = 1 << 20;

int check_gemm_ptrs(const uint8_t* ad, const uint8_t* as, const float* aa, const uint8_t* bd, const uint8_t* bs,
                    const float* ba, const float* out) {
  if (!ad || !as || !aa || !bd || !bs || !ba || !out) return NVFP4G_EINVAL;
  if (!aligned(ad, 16) || !aligned(bd, 16) || !aligned(as, 4) || !aligned(bs, 4) || !aligned(aa, 4) ||
      !aligned(ba, 4) || !aligned(out, 4))
    return NVFP4G_EALIGN;
  return NVFP4G_OK;
}

int launch_fwd(const uint8_t* ad, const uint8_t* as, const float* aa, const uint8_t* bd, const uint8_t* bs,
               const float* ba, int64_t rows, int64_t n, int64_t k, const Routing& R, float* out, hipStream_t st) {
  if (rows == 0) return NVFP4G_OK;
  const uint32_t ntm = (uint32_t)(rows / kBM), ntn = (uint32_t)((n + kBN - 1) / kBN);
  hipLaunchKernelGGL(gemm_fwd_kernel, dim3(ntm * ntn), dim3(kThreads), 0, st, ad, as, aa, bd, bs, ba, n, k, R, ntm,
                     ntn, out);
  return hip_status();
}

int check_fwd(int64_t rows, int64_t n, int64_t k, int32_t E) {
  if (k <= 0 || k % kBK != 0 || k > kMaxK) return NVFP4G_EINVAL;
  if (n <= 0 || n % 16 != 0 || n > kGemmMaxN) return NVFP4G_EINVAL;
  if (rows < 0 || rows > kMaxRows || E < 1) return NVFP4G_EINVAL;
  // tile count fits the 1-D grid
  if ((rows / kBM) * ((n + kBN - 1) / kBN) > (int64_t)INT32_MAX) return NVFP4G_EINVAL;
  return NVFP4G_OK;
}

}  // namespace

extern "C" {

int nvfp4_group_gemm(const uint8_t* a_data, const uint8_t* a_scale, const float* a_amax, const uint8_t* b_data,
                     const uint8_t* b_scale, const float* b_amax, int64_t sum_m, int64_t n, int64_t k,
                     int32_t num_experts, const int64_t* h_splits, float* out, void* stream) {
  int rc = check_fwd(sum_m, n, k, num_experts);
  if (rc) return rc;
  if ((rc = check_gemm_ptrs(a_data, a_scale, a_amax, b_data, b_scale, b_amax, out))) return rc;
  Routing R;
  R.num_experts = num_experts;
  R.m_capacity = (int32_t)sum_m;
  R.d_offs = nullptr;
  R.d_status = nullptr;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  return launch_fwd(a_data, a_scale, a_amax, b_data, b_scale, b_amax, sum_m, n, k, R, out, (hipStream_t)stream);
}

int nvfp4_group_gemm_graphsafe(const uint8_t* a_data, const uint8_t* a_scale, const float* a_amax,
                               const uint8_t* b_data, const uint8_t* b_scale, const float* b_amax,
                               int64_t m_capacity, int64_t n, int64_t k, int32_t num_experts,
                               const int32_t* d_offs, float* out, int32_t* d_status, void* stream) {
  int rc = check_fwd(m_capacity, n, k, num_experts);
  if (rc) return rc;
  if ((rc = check_gemm_ptrs(a_data, a_scale, a_amax, b_data, b_scale, b_amax, out))) return rc;
  Routing R;
  R.num_experts = num_experts;
  R.m_capacity = (int32_t)m_capacity;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  return launch_fwd(a_data, a_scale, a_amax, b_data, b_scale, b_amax, m_capacity, n, k, R, out,
                    (hipStream_t)stream);
}

int nvfp4_group_gemm_wgrad(const uint8_t* a_col_data, const uint8_t* a_col_scale, const float* a_col_amax,
                           const uint8_t* b_col_data, const uint8_t* b_col_scale, const float* b_col_amax,
                           int64_t sum_m, int64_t n, int64_t k, int32_t num_experts, const int64_t* h_splits,
                           float* out, void* stream) {
  if (n <= 0 || n % 16 != 0 || n > kGemmMaxN || k <= 0 || k % 16 != 0 || k > kGemmMaxN) return NVFP4G_EINVAL;
  if (sum_m < 0 || sum_m > kMaxRows || num_experts < 1) return NVFP4G_EINVAL;
  const int64_t ntm = (n + kBM - 1) / kBM, ntn = (k + kBN - 1) / kBN;
  if (ntm * ntn * num_experts > (int64_t)INT32_MAX) return NVFP4G_EINVAL;
  int rc = check_gemm_ptrs(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, out);
  if (rc) return rc;
  Routing R;
  R.num_experts = num_experts;
  R.m_capacity = (int32_t)sum_m;
  R.d_offs = nullptr;
  R.d_status = nullptr;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  hipLaunchKernelGGL(gemm_wgrad_kernel, dim3((uint32_t)(ntm * ntn * num_experts)), dim3(kThreads), 0,
                     (hipStream_t)stream, a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax,
                     n, k, R, (uint32_t)ntm, (uint32_t)ntn, out);
  return hip_status();
}

}  // extern "C"
