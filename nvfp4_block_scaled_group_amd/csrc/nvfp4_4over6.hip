// nvfp4_4over6.hip -- grouped row-scaled NVFP4 cast with four-over-six block
// scaling on MI355X (gfx950), behind the C ABI of include/nvfp4_group.h.
//
// Operation: the "four_over_six" recipe named on the torchtitan converter
// page ("[NVFP4 4over6] Add the grouped-experts four-over-six converter",
// Summary and Review pass: knobs err_mode, e4m3_scale_bound, row_scaled).
// The page does not spell out the block rule; it is read from the published
// method of that name ("Four Over Six: More Accurate NVFP4 Quantization with
// Adaptive Block Scaling"): each 16-element block is encoded twice, with its
// amax mapped to 6 and to 4, and the encoding with the smaller error (sum of
// squared or of absolute element errors, accumulated in element order) is
// kept; ties keep 6.  The line scale is A / (6 * bound) with bound =
// e4m3_scale_bound.  Everything else -- per-row and per-(expert, column)
// line amax (from nvfp4_group_amax), layouts, routing, graph-safe twin --
// is the grouped cast's.
//
// Design: the grouped cast's tiles (128 x 256, one expert per tile, XCD-aware
// order), lane layout (lane = 16 rows x 8 columns), staged rowwise lines and
// scales, and streaming transposed stores.  The difference is arithmetic:
// per block two scale steps (fast quotients proved to give what the IEEE
// divisions give on every input they get) and, per element and candidate,
// the code, its dequantised value and the error term -- about fifteen VALU
// operations per element and direction, so the kernel is bound by the
// vector ALUs rather than by HBM.
//  * Columnwise blocks lie in one lane (16 rows of one column): both error
//    sums run in the lane in row order.
//  * Rowwise blocks are split over the lane pair (L, L^8) (8 columns each).
//    The even lane owns row i of the pair of rows (i, 8+i) it serves with
//    its partner and the odd lane row 8+i; two masked DPP moves per data
//    word give each lane the 16 values of its own row's block in element
//    order, and it then encodes the block alone, like a columnwise one.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>

#include "../../include/nvfp4_group.h"
#include "nvfp4_numerics.hpp"
#include "nvfp4_common.hpp"

namespace {

using namespace nvfp4g;

// One candidate's block step, in the order of the method: t = u_k / s with
// u_k = b / k, S = E4M3(t), d = value(S) * s, m = 1 / d (0 when d == 0, at
// most FLT_MAX).  Returns S; *sv = value(S).  The fast forms give what the
// IEEE divisions give on every input they are used for (exhaustive GPU
// self-tests): b / 6 by div6_bf16 (b is a bf16 value; b / 4 is exact), the
// E4M3 code of t by quot_fast with ys = RN(1/s) on lines with s >= 2^-112,
// and 1 / d by rcp_rn where d and 1 / d are normal; the IEEE division
// elsewhere.
__device__ __forceinline__ uint32_t cand_step(float u, float s, float ys, float* sv, float* m) {
  const float t = (s >= kFastMinLineScale) ? quot_fast(u, s, ys) : ((s == 0.0f) ? 0.0f : u / s);
  const uint32_t S = e4m3_code(t);
  const float v = e4m3_value(S);
  const float d = v * s;
  *sv = v;
  const bool fast = d >= 0x1p-126f && d < 0x1p126f;
  *m = (d == 0.0f) ? 0.0f : (fast ? rcp_rn(d) : fminf(1.0f / d, FLT_MAX));
  return S;
}

// The two E2M1 values of byte SEL of a packed code word: the hardware
// FP4 -> fp32 convert with unit scale (exact, signed).
#define FP4X2_VALUE(w, SEL) __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((w), 1.0f, (SEL))

// Error term of element x whose code has value q, for a candidate with scale
// value sv on a line with scale s: the dequantised value is (q * sv) * s
// (the first product is exact), the term its squared (MODE 0) or absolute
// (MODE 1) difference from x.
template <int MODE>
__device__ __forceinline__ float err_term(float x, float q, float sv, float s) {
  const float diff = x - (q * sv) * s;
  return MODE == 0 ? diff * diff : fabsf(diff);
}

// The 8 values of a packed code word, in element order.
__device__ __forceinline__ void decode8(uint32_t p, float (&q)[8]) {
  const auto q0 = FP4X2_VALUE(p, 0), q1 = FP4X2_VALUE(p, 1), q2 = FP4X2_VALUE(p, 2), q3 = FP4X2_VALUE(p, 3);
  q[0] = q0[0]; q[1] = q0[1]; q[2] = q1[0]; q[3] = q1[1];
  q[4] = q2[0]; q[5] = q2[1]; q[6] = q3[0]; q[7] = q3[1];
}

// Codes of the 8 values x[0..7] times m, 2 per byte.
__device__ __forceinline__ uint32_t encode8f(const float* x, float m) {
  uint32_t p = 0;
  p = FP4X2(p, x[0] * m, x[1] * m, 0);
  p = FP4X2(p, x[2] * m, x[3] * m, 1);
  p = FP4X2(p, x[4] * m, x[5] * m, 2);
  p = FP4X2(p, x[6] * m, x[7] * m, 3);
  return p;
}

// Error sum of one candidate over a block of 16 values x (element order),
// codes c_lo (elements 0-7) and c_hi (8-15), scale value sv, line scale s:
// ((0 + r_0) + r_1) + ... + r_15.
template <int MODE>
__device__ __forceinline__ float block_err(const float (&x)[16], uint32_t c_lo, uint32_t c_hi, float sv, float s) {
  float q[16];
  decode8(c_lo, *reinterpret_cast<float(*)[8]>(&q[0]));
  decode8(c_hi, *reinterpret_cast<float(*)[8]>(&q[8]));
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) e = e + err_term<MODE>(x[i], q[i], sv, s);
  return e;
}

// Four-over-six step of one block of 16 values x (element order) with block
// amax b on a line with scale sl.x (sl.y = RN(1/sl.x)): both candidates,
// the one with the smaller error kept (6 on a tie).  Returns its scale code;
// *lo, *hi = its codes of elements 0-7 and 8-15 (element 2j in the low
// nibble of byte j).
template <int MODE>
__device__ __forceinline__ uint32_t block_4o6(const float (&x)[16], float b, float2 sl, uint32_t* lo, uint32_t* hi) {
  const float s = sl.x;
  float sv6, m6, sv4, m4;
  const uint32_t S6 = cand_step(div6_bf16(b), s, sl.y, &sv6, &m6);
  const uint32_t S4 = cand_step(b * 0.25f, s, sl.y, &sv4, &m4);
  const uint32_t c6_lo = encode8f(x, m6), c6_hi = encode8f(x + 8, m6);
  const uint32_t c4_lo = encode8f(x, m4), c4_hi = encode8f(x + 8, m4);
  const float e6 = block_err<MODE>(x, c6_lo, c6_hi, sv6, s);
  const float e4 = block_err<MODE>(x, c4_lo, c4_hi, sv4, s);
  const bool use4 = e4 < e6;
  *lo = use4 ? c4_lo : c6_lo;
  *hi = use4 ? c4_hi : c6_hi;
  return use4 ? S4 : S6;
}

// DPP row_ror:8 (lane ^ 8 inside a 16-lane row) written only to the lanes
// 0-7 (BANKS = 0x3) or 8-15 (BANKS = 0xC) of each row; the other lanes keep
// `old`.
template <int BANKS>
__device__ __forceinline__ uint32_t swap8_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x128, 0xF, BANKS, false);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void group_cast_4o6_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, uint32_t nrow_tiles, float line_div,
    const float* __restrict__ row_amax, const float* __restrict__ col_amax, uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale, uint8_t* __restrict__ col_data,
    uint8_t* __restrict__ col_scale) {
  __shared__ float2 l_row[kTileRows];  // (s, 1/s) per row of the tile
  __shared__ float2 l_col[kTileCols];  // (s, 1/s) per column of the tile
  __shared__ StagedRowScales l_rs;
  __shared__ StagedColScales l_cs;
  __shared__ StagedRowData l_rd;
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const TileCoord tc = tile_coord(nrow_tiles);
  const int32_t row0 = (int32_t)tc.row_tile * kTileRows;
  if (row0 >= total) return;
  const int64_t col_base = (int64_t)tc.chunk * kTileCols;
  const uint32_t ncols = (uint32_t)min<int64_t>(k - col_base, kTileCols);
  const uint32_t ku = (uint32_t)k;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rb = lane & 7, cg = lane >> 3;
  const uint32_t lcol = wave * 64 + cg * 8;
  const bool active = lcol < ncols;
  const uint32_t vo_x = active ? (16u * rb * ku + lcol) * 2u : kOutOfRange;

  int32_t rbeg, rend;
  const int e = find_expert(R, row0, &rbeg, &rend);
  const uint32_t me = (uint32_t)(rend - rbeg);

  const float a_row = row_data && tid < kTileRows ? row_amax[row0 + tid] : 0.0f;
  const float a_col = col_data && (uint32_t)tid < ncols ? col_amax[(int64_t)e * k + col_base + tid] : 0.0f;
  uint32_t v[16][4];
  load_tile(x + (int64_t)row0 * k + col_base, ku, vo_x, v);
  if (row_data && tid < kTileRows) {
    const float s = a_row / line_div;
    l_row[tid] = make_float2(s, 1.0f / s);
  }
  if (col_data) {
    const float s = a_col / line_div;
    l_col[tid] = make_float2(s, 1.0f / s);
  }
  __syncthreads();

  if (row_data) {
    // The lane pair (lane, lane^8) holds the two 8-column halves of each
    // 16-column block of its 16 rows.  Iteration i serves rows i and 8+i:
    // the even lane takes row i's block (its own half, then the partner's),
    // the odd lane row 8+i's (the partner's half, then its own), by two
    // masked DPP moves per word, and each lane encodes its block alone.
    const bool odd = cg & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = swap8_into<0xC>(v[i][q], v[8 + i][q]);      // elements 0-7
        w[4 + q] = swap8_into<0x3>(v[8 + i][q], v[i][q]);  // elements 8-15
      }
      uint32_t mx = 0;
      float xv[16];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mx = pkmax(mx, w[q] & 0x7FFF7FFFu);
        xv[2 * q] = bf16lo(w[q]);
        xv[2 * q + 1] = bf16hi(w[q]);
      }
      const int ri = odd ? 8 + i : i;
      uint32_t lo, hi;
      const uint32_t S = block_4o6<MODE>(xv, __uint_as_float(hmax(mx) << 16), l_row[16 * rb + ri], &lo, &hi);
      reinterpret_cast<uint8_t*>(&l_rs[16 * rb + ri][0])[wave * 4 + (cg >> 1)] = (uint8_t)S;
      // bytes of columns 8*(cg & ~1) .. +15: dwords 8*wave + (cg & ~1), +1 of the row
      *reinterpret_cast<u32x2*>(&l_rd[16 * rb + ri][row_slot(rb, wave, cg & ~1)]) = u32x2{lo, hi};
    }
  }

  if (col_data) {
    const rsrc_t cd = make_rsrc(col_data + k * (int64_t)rbeg / 2 + col_base * (me / 2) + (row0 - rbeg) / 2);
    const uint32_t vo = active ? lcol * (me / 2) + 8u * rb : kOutOfRange;
    uint32_t mxw[4] = {0, 0, 0, 0};  // column maxima, two columns per word
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) mxw[q] = pkmax(mxw[q], v[i][q] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column lcol + j of the lane's 16 rows
      float xv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) xv[i] = (j & 1) ? bf16hi(v[i][j >> 1]) : bf16lo(v[i][j >> 1]);
      const uint32_t b16 = (j & 1) ? (mxw[j >> 1] >> 16) : (mxw[j >> 1] & 0xFFFFu);
      uint32_t lo, hi;
      const uint32_t S = block_4o6<MODE>(xv, __uint_as_float(b16 << 16), l_col[lcol + j], &lo, &hi);
      reinterpret_cast<uint8_t*>(&l_cs[lcol + j][0])[rb] = (uint8_t)S;
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, cd, vo, (uint32_t)j * (me / 2), kStoreStream);
    }
  }

  __syncthreads();
  store_staged_tile(l_rd, l_rs, l_cs, k, row0, col_base, ncols, rbeg, me, row_data, row_scale,
                    col_data ? col_scale : nullptr);
}

int launch_cast_4o6(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, int32_t bound, int32_t err_mode,
                    const float* row_amax, const float* col_amax, uint8_t* row_data, uint8_t* row_scale,
                    uint8_t* col_data, uint8_t* col_scale, hipStream_t st) {
  if ((!row_data && !col_data) || rows == 0) return NVFP4G_OK;
  const float line_div = 6.0f * (float)bound;  // exact: at most 2688
  if (err_mode == NVFP4G_4O6_ERR_MSE)
    hipLaunchKernelGGL(group_cast_4o6_kernel<0>, tile_grid(rows, k), dim3(kThreads), 0, st, x, k, R,
                       num_row_tiles(rows), line_div, row_amax, col_amax, row_data, row_scale, col_data,
                       col_scale);
  else
    hipLaunchKernelGGL(group_cast_4o6_kernel<1>, tile_grid(rows, k), dim3(kThreads), 0, st, x, k, R,
                       num_row_tiles(rows), line_div, row_amax, col_amax, row_data, row_scale, col_data,
                       col_scale);
  return hip_status();
}

int check_4o6(int32_t bound, int32_t err_mode) {
  if (bound < 1 || bound > NVFP4G_4O6_MAX_BOUND) return NVFP4G_EINVAL;
  if (err_mode != NVFP4G_4O6_ERR_MSE && err_mode != NVFP4G_4O6_ERR_MAE) return NVFP4G_EINVAL;
  return NVFP4G_OK;
}

}  // namespace

extern "C" {

int nvfp4_group_cast_4over6(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts,
                            const int64_t* h_splits, const float* row_amax, const float* col_amax,
                            int32_t scale_bound, int32_t err_mode, uint8_t* row_data, uint8_t* row_scale,
                            uint8_t* col_data, uint8_t* col_scale, void* stream) {
  Routing R;
  int rc = check_common(x, sum_m, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  if ((rc = check_4o6(scale_bound, err_mode))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  return launch_cast_4o6(x, sum_m, k, R, scale_bound, err_mode, row_amax, col_amax, row_data, row_scale, col_data,
                         col_scale, (hipStream_t)stream);
}

int nvfp4_group_cast_4over6_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                                      const int32_t* d_offs, const float* row_amax, const float* col_amax,
                                      int32_t scale_bound, int32_t err_mode, uint8_t* row_data,
                                      uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale,
                                      int32_t* d_status, void* stream) {
  Routing R;
  int rc = check_common(x, m_capacity, k, num_experts, &R);
  if (rc) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  if ((rc = check_4o6(scale_bound, err_mode))) return rc;
  if ((rc = check_cast_outputs(row_amax, col_amax, row_data, row_scale, col_data, col_scale))) return rc;
  return launch_cast_4o6(x, m_capacity, k, R, scale_bound, err_mode, row_amax, col_amax, row_data, row_scale,
                         col_data, col_scale, (hipStream_t)stream);
}

}  // extern "C"
