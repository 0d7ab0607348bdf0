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
// per block two scale steps with IEEE divisions and, per element and
// candidate, the code, its dequantised value and the error term -- about
// fifteen VALU operations per element and direction, so the kernel is bound
// by the vector ALUs rather than by HBM.
//  * Columnwise blocks lie in one lane (16 rows of one column): both error
//    sums run in the lane in row order.
//  * Rowwise blocks are split over the lane pair (L, L^8) (8 columns each).
//    The even lane owns row i of the pair of rows (i, 8+i) it serves with
//    its partner and the odd lane row 8+i; each lane computes the error terms
//    of its 8 columns of both rows, then two masked DPP moves per term give
//    each lane all 16 terms of its own row in element order (the even lane
//    takes its partner's second half, the odd lane its partner's first
//    half), and the lane sums them in order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>

#include "../../include/nvfp4_group.h"
#include "nvfp4_numerics.hpp"
#include "nvfp4_common.hpp"

namespace {

using namespace nvfp4g;

// The two candidates' divisors.
constexpr float kK6 = 6.0f;
constexpr float kK4 = 4.0f;

// One candidate's block step with IEEE divisions, in the order of the
// method: t = (b / k) / s, S = E4M3(t), d = value(S) * s, m = 1 / d (0 when
// d == 0, at most FLT_MAX).  Returns S; *sv = value(S).
__device__ __forceinline__ uint32_t cand_step(float b, float kdiv, float s, float* sv, float* m) {
  const float t = (s == 0.0f) ? 0.0f : (b / kdiv) / s;
  const uint32_t S = e4m3_code(t);
  const float v = e4m3_value(S);
  const float d = v * s;
  *sv = v;
  *m = (d == 0.0f) ? 0.0f : fminf(1.0f / d, FLT_MAX);
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

// Codes of 8 values (v = 4 words of bf16 pairs) times m, 2 per byte.
__device__ __forceinline__ uint32_t encode8(const uint32_t (&v)[4], float m) {
  uint32_t p = 0;
  p = FP4X2(p, bf16lo(v[0]) * m, bf16hi(v[0]) * m, 0);
  p = FP4X2(p, bf16lo(v[1]) * m, bf16hi(v[1]) * m, 1);
  p = FP4X2(p, bf16lo(v[2]) * m, bf16hi(v[2]) * m, 2);
  p = FP4X2(p, bf16lo(v[3]) * m, bf16hi(v[3]) * m, 3);
  return p;
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

// The 8 error terms of the values v (codes p) for one candidate.
template <int MODE>
__device__ __forceinline__ void terms8(const uint32_t (&v)[4], uint32_t p, float sv, float s, float (&t)[8]) {
  float q[8];
  decode8(p, q);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t[2 * j] = err_term<MODE>(bf16lo(v[j]), q[2 * j], sv, s);
    t[2 * j + 1] = err_term<MODE>(bf16hi(v[j]), q[2 * j + 1], sv, s);
  }
}

// DPP row_ror:8 (lane ^ 8 inside a 16-lane row) written only to the lanes
// 0-7 (BANKS = 0x3) or 8-15 (BANKS = 0xC) of each row; the other lanes keep
// `old`.
template <int BANKS>
__device__ __forceinline__ float swap8_into(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), 0x128, 0xF, BANKS, false));
}

// Error sum, in element order, of the rowwise block this lane owns: a = the
// lane's terms of row i (elements 0-7 in the even lane, 8-15 in the odd
// lane), c = those of row 8+i.  The even lane owns row i: its own a, then the
// partner's a.  The odd lane owns row 8+i: the partner's c, then its own c.
__device__ __forceinline__ float row_block_sum(const float (&a)[8], const float (&c)[8]) {
  float e = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) e = e + swap8_into<0xC>(a[j], c[j]);  // first half
#pragma unroll
  for (int j = 0; j < 8; ++j) e = e + swap8_into<0x3>(c[j], a[j]);  // second half
  return e;
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void group_cast_4o6_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, uint32_t nrow_tiles, float line_div, const float* __restrict__ row_amax, const float* __restrict__ col_amax,
    uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale, uint8_t* __restrict__ col_data,
    uint8_t* __restrict__ col_scale) {
  __shared__ float l_row[kTileRows];  // line scale per row of the tile
  __shared__ float l_col[kTileCols];  // line scale per column of the tile
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
  if (row_data && tid < kTileRows) l_row[tid] = a_row / line_div;
  if (col_data) l_col[tid] = a_col / line_div;
  __syncthreads();

  if (row_data) {
    const bool odd = cg & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // block amax of the owned row (as in the grouped cast)
      const uint32_t lo = hmax(pkmax(pkmax(v[i][0] & 0x7FFF7FFFu, v[i][1] & 0x7FFF7FFFu),
                                     pkmax(v[i][2] & 0x7FFF7FFFu, v[i][3] & 0x7FFF7FFFu)));
      const uint32_t hi = hmax(pkmax(pkmax(v[8 + i][0] & 0x7FFF7FFFu, v[8 + i][1] & 0x7FFF7FFFu),
                                     pkmax(v[8 + i][2] & 0x7FFF7FFFu, v[8 + i][3] & 0x7FFF7FFFu)));
      const uint32_t b16 = max(odd ? hi : lo, swap8(odd ? lo : hi));
      const float b = __uint_as_float(b16 << 16);
      const float s_lo = l_row[16 * rb + i], s_hi = l_row[16 * rb + 8 + i];
      const float s_own = odd ? s_hi : s_lo;
      float sv6, m6, sv4, m4;
      const uint32_t S6 = cand_step(b, kK6, s_own, &sv6, &m6);
      const uint32_t S4 = cand_step(b, kK4, s_own, &sv4, &m4);
      // the partner's candidates serve this lane's half of the other row
      const float psv6 = __uint_as_float(swap8(__float_as_uint(sv6)));
      const float pm6 = __uint_as_float(swap8(__float_as_uint(m6)));
      const float psv4 = __uint_as_float(swap8(__float_as_uint(sv4)));
      const float pm4 = __uint_as_float(swap8(__float_as_uint(m4)));
      const float m6_lo = odd ? pm6 : m6, m6_hi = odd ? m6 : pm6;
      const float m4_lo = odd ? pm4 : m4, m4_hi = odd ? m4 : pm4;
      const float sv6_lo = odd ? psv6 : sv6, sv6_hi = odd ? sv6 : psv6;
      const float sv4_lo = odd ? psv4 : sv4, sv4_hi = odd ? sv4 : psv4;

      const uint32_t p6_lo = encode8(v[i], m6_lo), p6_hi = encode8(v[8 + i], m6_hi);
      const uint32_t p4_lo = encode8(v[i], m4_lo), p4_hi = encode8(v[8 + i], m4_hi);
      float e6, e4;
      {
        float a[8], c[8];
        terms8<MODE>(v[i], p6_lo, sv6_lo, s_lo, a);
        terms8<MODE>(v[8 + i], p6_hi, sv6_hi, s_hi, c);
        e6 = row_block_sum(a, c);
      }
      {
        float a[8], c[8];
        terms8<MODE>(v[i], p4_lo, sv4_lo, s_lo, a);
        terms8<MODE>(v[8 + i], p4_hi, sv4_hi, s_hi, c);
        e4 = row_block_sum(a, c);
      }
      const uint32_t use4 = e4 < e6 ? 1u : 0u;  // this lane's row
      const uint32_t puse4 = swap8(use4);       // the partner's row
      const bool use4_lo = odd ? puse4 : use4, use4_hi = odd ? use4 : puse4;
      const int ri = odd ? 8 + i : i;
      reinterpret_cast<uint8_t*>(&l_rs[16 * rb + ri][0])[wave * 4 + (cg >> 1)] = (uint8_t)(use4 ? S4 : S6);
      l_rd[16 * rb + i][row_slot(rb, wave, cg)] = use4_lo ? p4_lo : p6_lo;
      l_rd[16 * rb + 8 + i][row_slot(rb, wave, cg)] = use4_hi ? p4_hi : p6_hi;
    }
  }

  if (col_data) {
    const rsrc_t cd = make_rsrc(col_data + k * (int64_t)rbeg / 2 + col_base * (me / 2) + (row0 - rbeg) / 2);
    const uint32_t vo = active ? lcol * (me / 2) + 8u * rb : kOutOfRange;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // column lcol + j of the lane's 16 rows
      float xv[16];
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w = (j & 1) ? (v[i][j >> 1] >> 16) : (v[i][j >> 1] & 0xFFFFu);
        xv[i] = __uint_as_float(w << 16);
        mx = max(mx, w & 0x7FFFu);
      }
      const float b = __uint_as_float(mx << 16);
      const float s = l_col[lcol + j];
      float sv6, m6, sv4, m4;
      const uint32_t S6 = cand_step(b, kK6, s, &sv6, &m6);
      const uint32_t S4 = cand_step(b, kK4, s, &sv4, &m4);
      const uint32_t c6_lo = encode8f(xv, m6), c6_hi = encode8f(xv + 8, m6);
      const uint32_t c4_lo = encode8f(xv, m4), c4_hi = encode8f(xv + 8, m4);
      float e6 = 0.0f, e4 = 0.0f;
      {
        float q[16];
        decode8(c6_lo, *reinterpret_cast<float(*)[8]>(&q[0]));
        decode8(c6_hi, *reinterpret_cast<float(*)[8]>(&q[8]));
#pragma unroll
        for (int i = 0; i < 16; ++i) e6 = e6 + err_term<MODE>(xv[i], q[i], sv6, s);
      }
      {
        float q[16];
        decode8(c4_lo, *reinterpret_cast<float(*)[8]>(&q[0]));
        decode8(c4_hi, *reinterpret_cast<float(*)[8]>(&q[8]));
#pragma unroll
        for (int i = 0; i < 16; ++i) e4 = e4 + err_term<MODE>(xv[i], q[i], sv4, s);
      }
      const bool use4 = e4 < e6;
      reinterpret_cast<uint8_t*>(&l_cs[lcol + j][0])[rb] = (uint8_t)(use4 ? S4 : S6);
      __builtin_amdgcn_raw_buffer_store_b64(use4 ? u32x2{c4_lo, c4_hi} : u32x2{c6_lo, c6_hi}, cd, vo,
                                            (uint32_t)j * (me / 2), kStoreStream);
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
