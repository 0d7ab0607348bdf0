// mxfp4_group.hip -- grouped MXFP4 cast of a packed MoE activation buffer,
// rowwise and columnwise (transposed per expert), behind the C ABI of
// include/nvfp4_group.h.
//
// MXFP4 is the power-of-two-scaled sibling of NVFP4 named on the
// TransformerEngine PR 3824 page (Changes item 1, Testing): E2M1 elements,
// blocks of 32, one E8M0 scale byte per block.  The scale rule is the OCP
// Microscaling (MX) v1.0 one: for a block with amax A,
//     shared = floor(log2 A) - 2, clamped to [-127, 127] (-127 for A == 0),
//     byte   = shared + 127,
//     code   = E2M1(x / 2^shared), nearest, ties to even, saturating.
// Every block is independent, so there is no amax pass: one kernel reads x
// once and writes both directions.
//
// The block amax is an integer max over abs-bf16 bit patterns, and for a
// finite bf16 amax with exponent field e, floor(log2 A) = e - 127 (0 for a
// subnormal or zero amax, which the clamp maps to byte 0), so
//     byte = max(e - 2, 0).
// 1/2^shared = 2^(127 - byte) is an exact fp32 power of two (byte <= 252 for
// finite bf16, so it is never subnormal), x * 2^(127 - byte) is exact
// whenever it is not subnormal, and |x * 2^(127 - byte)| < 8.  Values so
// small that the product is subnormal all encode to a signed zero, as they
// do under exact division.  Codes come from the hardware FP4 conversion at
// scale 1.0 (identical to the nearest-even E2M1 rule on every fp32 input).
//
// Tiles, lane layout and expert routing are those of the NVFP4 cast kernel:
// a 128 x 256 tile per work-group, lane (rb, cg) = (lane & 7, lane >> 3)
// holding rows 16rb..16rb+15 and columns 64*wave + 8cg .. +7.  A rowwise
// 32-block is the 8 columns of lanes cg = 4q..4q+3 (lane, lane^8, lane^16,
// lane^24); a columnwise 32-block is the 16 rows of lanes rb = 2p, 2p+1
// (lane, lane^1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_common.hpp"
#include "nvfp4_numerics.hpp"

namespace {

using namespace nvfp4g;

// E8M0 scale byte of a block from its abs-bf16 amax bits (finite input).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t a16) {
  return (uint32_t)max((int)(a16 >> 7) - 2, 0);
}
// 1 / 2^(byte - 127) as an fp32 power of two.
__device__ __forceinline__ float mx_multiplier(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

__global__ __launch_bounds__(kThreads) void mxfp4_group_cast_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, uint32_t nrow_tiles,
    uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scale) {
  __shared__ uint32_t l_rs[kTileRows][kTileCols / 128];  // row scales, 8 per row
  __shared__ uint32_t l_cs[kTileCols];                   // column scales, 4 per column
  __shared__ uint32_t l_rd[kTileRows][kTileCols / 8];    // row data, 128 bytes per row (swizzled)
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const TileCoord tc = tile_coord(nrow_tiles);
  const int32_t row0 = (int32_t)tc.row_tile * kTileRows;
  if (row0 >= total) return;
  const int64_t col_base = (int64_t)tc.chunk * kTileCols;
  const uint32_t ncols = (uint32_t)min<int64_t>(k - col_base, kTileCols);  // a multiple of 32
  const uint32_t ku = (uint32_t)k;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rb = lane & 7, cg = lane >> 3;
  const uint32_t lcol = wave * 64 + cg * 8;
  const bool active = lcol < ncols;  // the same for all four lanes of a rowwise block
  const uint32_t vo_x = active ? (16u * rb * ku + lcol) * 2u : kOutOfRange;

  int32_t rbeg, rend;
  find_expert(R, row0, &rbeg, &rend);
  const uint32_t me = (uint32_t)(rend - rbeg);

  uint32_t v[16][4];
  load_tile(x + (int64_t)row0 * k + col_base, ku, vo_x, v);

  if (row_data) {
    // abs amax of rows (2p, 2p+1) over the lane's 8 columns, packed, then
    // over the block's four lanes
    uint32_t rp[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t a0 = hmax(pkmax(pkmax(v[2 * p][0] & 0x7FFF7FFFu, v[2 * p][1] & 0x7FFF7FFFu),
                                     pkmax(v[2 * p][2] & 0x7FFF7FFFu, v[2 * p][3] & 0x7FFF7FFFu)));
      const uint32_t a1 = hmax(pkmax(pkmax(v[2 * p + 1][0] & 0x7FFF7FFFu, v[2 * p + 1][1] & 0x7FFF7FFFu),
                                     pkmax(v[2 * p + 1][2] & 0x7FFF7FFFu, v[2 * p + 1][3] & 0x7FFF7FFFu)));
      uint32_t r = a0 | (a1 << 16);
      r = pkmax(r, swap8(r));
      rp[p] = swap16_max(r, r);
    }
    const int q = cg & 3;  // the four lanes of a block share its scale writes
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = mx_scale_byte((i & 1) ? rp[i >> 1] >> 16 : rp[i >> 1] & 0xFFFFu);
      const float m = mx_multiplier(byte);
      uint32_t packed = 0;
      packed = FP4X2(packed, bf16lo(v[i][0]) * m, bf16hi(v[i][0]) * m, 0);
      packed = FP4X2(packed, bf16lo(v[i][1]) * m, bf16hi(v[i][1]) * m, 1);
      packed = FP4X2(packed, bf16lo(v[i][2]) * m, bf16hi(v[i][2]) * m, 2);
      packed = FP4X2(packed, bf16lo(v[i][3]) * m, bf16hi(v[i][3]) * m, 3);
      // bytes lcol/2 .. +3 of row 16*rb + i: dword 8*wave + cg; granule q
      // of row r sits at slot q ^ ((r / 16) % 8), so the wave's writes (eight
      // rows 16 apart, same dword column) fall in distinct banks
      l_rd[16 * rb + i][(8 * wave + cg) ^ (rb << 2)] = packed;
      if ((i & 3) == q)
        reinterpret_cast<uint8_t*>(&l_rs[16 * rb + i][0])[wave * 2 + (cg >> 2)] = (uint8_t)byte;
    }
  }

  if (col_data) {
    // abs amax of columns (2w, 2w+1) over the lane's 16 rows, packed, then
    // over the lane pair rb, rb^1
    uint32_t cp[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t mx = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = pkmax(mx, v[i][w] & 0x7FFF7FFFu);
      cp[w] = pkmax(mx, dpp_x1(mx));
    }
    const rsrc_t cd = make_rsrc(col_data + k * (int64_t)rbeg / 2 + col_base * (me / 2) + (row0 - rbeg) / 2);
    const uint32_t vo = active ? lcol * (me / 2) + 8u * rb : kOutOfRange;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t byte = mx_scale_byte((j & 1) ? cp[j >> 1] >> 16 : cp[j >> 1] & 0xFFFFu);
      const float m = mx_multiplier(byte);
#define XCOL(i) (((j & 1) ? bf16hi(v[i][j >> 1]) : bf16lo(v[i][j >> 1])) * m)
      uint32_t lo = 0, hi = 0;
      lo = FP4X2(lo, XCOL(0), XCOL(1), 0);
      lo = FP4X2(lo, XCOL(2), XCOL(3), 1);
      lo = FP4X2(lo, XCOL(4), XCOL(5), 2);
      lo = FP4X2(lo, XCOL(6), XCOL(7), 3);
      hi = FP4X2(hi, XCOL(8), XCOL(9), 0);
      hi = FP4X2(hi, XCOL(10), XCOL(11), 1);
      hi = FP4X2(hi, XCOL(12), XCOL(13), 2);
      hi = FP4X2(hi, XCOL(14), XCOL(15), 3);
#undef XCOL
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, cd, vo, (uint32_t)j * (me / 2), kStoreStream);
      if ((j >> 2) == (rb & 1))  // the lane pair splits the 8 columns' scale writes
        reinterpret_cast<uint8_t*>(&l_cs[lcol + j])[rb >> 1] = (uint8_t)byte;
    }
  }

  // rowwise data and scales: staged in LDS, then one store per 16-byte
  // granule of a row line, one per row (8 scale bytes) / column (4 bytes)
  __syncthreads();
  if (row_data) {
    // thread t writes granule t % 8 (32 columns; ncols is a multiple of 32)
    // of rows t / 8 + 32 * it
    const rsrc_t rd = make_rsrc(row_data + (int64_t)row0 * (k / 2) + col_base / 2);
    const uint32_t g = tid & 7;
#pragma unroll
    for (int it = 0; it < kTileRows / 32; ++it) {
      const uint32_t r = 32 * it + (tid >> 3);
      const u32x4 v4 = *reinterpret_cast<const u32x4*>(&l_rd[r][4 * (g ^ ((r >> 4) & 7))]);
      if (32 * g < ncols) __builtin_amdgcn_raw_buffer_store_b128(v4, rd, r * (ku / 2) + 16 * g, 0, kStoreAux);
    }
  }
  if (row_data && tid < kTileRows) {
    uint8_t* dst = row_scale + ((int64_t)row0 + tid) * (k / 32) + col_base / 32;
    if (ncols == kTileCols && (k & 255) == 0) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&l_rs[tid][0]);
    } else {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(&l_rs[tid][0]);
      for (uint32_t b = 0; b < ncols / 32; ++b) dst[b] = src[b];
    }
  }
  if (col_data && (uint32_t)tid < ncols) {
    uint8_t* dst = col_scale + k * (int64_t)rbeg / 32 + (col_base + tid) * (int64_t)(me / 32) + (row0 - rbeg) / 32;
    *reinterpret_cast<uint32_t*>(dst) = l_cs[tid];
  }
}

int check_mx(const void* x, int64_t rows, int64_t k, int32_t E, Routing* R, const uint8_t* row_data,
             const uint8_t* row_scale, const uint8_t* col_data, const uint8_t* col_scale) {
  int rc = check_common(x, rows, k, E, R);
  if (rc) return rc;
  if (k % 32 != 0) return NVFP4G_EINVAL;
  if ((row_data && !row_scale) || (col_data && !col_scale)) return NVFP4G_EINVAL;
  if (!aligned(row_data, 16) || !aligned(row_scale, 16) || !aligned(col_data, 16) || !aligned(col_scale, 16))
    return NVFP4G_EALIGN;
  return NVFP4G_OK;
}

// Residency cap: at most four work-groups (four tiles in flight) per CU.
// The kernel needs 94 VGPRs (five waves per SIMD).  On the 32-expert K=7168
// sum_M=65536 workload one launch takes ~315 us at three work-groups per CU
// and ~266-276 us at four or five; before the rowwise data was staged in LDS
// (four 32-byte pieces per 128-byte line instead of one 16-byte store per
// granule) more tiles in flight made it slower, and the cap was two.
// Reserving a quarter of the CU's 160 KB of LDS per work-group (dynamic LDS
// the kernel does not touch) enforces the cap.
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr int kMxGroupsPerCu = 4;
constexpr size_t kMxStaticLds =
    kTileRows * (kTileCols / 128) * 4 + kTileCols * 4 + kTileRows * (kTileCols / 8) * 4;  // l_rs + l_cs + l_rd
constexpr size_t kMxLdsReserve = kLdsPerCu / kMxGroupsPerCu - kMxStaticLds;

int launch_mx(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, uint8_t* row_data,
              uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale, hipStream_t st) {
  if ((!row_data && !col_data) || rows == 0) return NVFP4G_OK;
  hipLaunchKernelGGL(mxfp4_group_cast_kernel, tile_grid(rows, k), dim3(kThreads), kMxLdsReserve, st, x, k, R,
                     num_row_tiles(rows), row_data, row_scale, col_data, col_scale);
  return hip_status();
}

}  // namespace

extern "C" {

int mxfp4_group_cast(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts, const int64_t* h_splits,
                     uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale, void* stream) {
  Routing R;
  int rc = check_mx(x, sum_m, k, num_experts, &R, row_data, row_scale, col_data, col_scale);
  if (rc) return rc;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  return launch_mx(x, sum_m, k, R, row_data, row_scale, col_data, col_scale, (hipStream_t)stream);
}

int mxfp4_group_cast_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k, int32_t num_experts,
                               const int32_t* d_offs, uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                               uint8_t* col_scale, int32_t* d_status, void* stream) {
  Routing R;
  int rc = check_mx(x, m_capacity, k, num_experts, &R, row_data, row_scale, col_data, col_scale);
  if (rc) return rc;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  return launch_mx(x, m_capacity, k, R, row_data, row_scale, col_data, col_scale, (hipStream_t)stream);
}

}  // extern "C"
