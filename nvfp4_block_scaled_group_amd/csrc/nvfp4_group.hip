// nvfp4_group.hip -- grouped, row-scaled (per-token) NVFP4 amax + cast for
// packed MoE activations on MI355X (gfx950), behind the C ABI declared in
// include/nvfp4_group.h.
//
// Operation (cited by page title and section):
//  * the TransformerEngine issue 3649 page (single-launch grouped
//    row-scaled NVFP4 cast), Description: a grouped amax over the packed (sum_M, K)
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
//    floats), reduced across lanes, then atomic max into zero-initialised
//    outputs: one per row per 512-column chunk, and one per column each time
//    a workgroup's run of tiles leaves an (expert, chunk) pair (atomic max of
//    the fp32 bit patterns of non-negative values is order independent, so
//    results are deterministic).  For K <= 2048 the tiles are whole rows
//    instead (one plain store per row; column maxima flushed per expert).
//  * cast: the rowwise data is staged in LDS and written as whole 128-byte
//    lines, the scales are staged and written one piece per line per tile,
//    and the transposed data goes out directly (see the kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <float.h>

#include <algorithm>

#include "../../include/nvfp4_group.h"
#include "nvfp4_numerics.hpp"
#include "nvfp4_common.hpp"

namespace {

using namespace nvfp4g;

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

// Grouped amax, persistent: a grid of G workgroups, workgroup g walks the
// contiguous range [g*T/G, (g+1)*T/G) of the T tiles of 64 rows x 512
// columns, ordered row tile fastest within each 512-column chunk (so a
// workgroup mostly walks down one chunk).  A wave covers 16 rows x 512
// columns: lane L holds columns 8L..8L+7 of the wave's 16 rows, so each wave
// load reads 1 KB of one row.  The next tile's loads are issued before the
// current tile is reduced.  Column maxima stay in registers while the
// (expert, chunk) pair is unchanged and are flushed with one atomic max per
// column when it changes; each row gets one atomic max per 512-column chunk.
constexpr int kAmaxRows = 64;
constexpr int kAmaxCols = 512;

struct AmaxTile {
  int32_t row0;   // first row
  int32_t chunk;  // 512-column chunk
};

__device__ __forceinline__ void amax_load(const uint16_t* x, uint32_t ku, int32_t row0, int32_t chunk,
                                          uint32_t lane_off, uint32_t (&v)[16][4]) {
  const rsrc_t xr = make_rsrc(x + (int64_t)row0 * ku + (int64_t)chunk * kAmaxCols);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(xr, lane_off, (uint32_t)i * ku * 2u, kAmaxLoadAux);
    v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
  }
}

__global__ __launch_bounds__(kThreads) void group_amax_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R,
    uint32_t* __restrict__ row_amax, uint32_t* __restrict__ col_amax) {
  __shared__ uint32_t l_col[4][kAmaxCols / 2];  // per wave, column pairs
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const uint32_t ku = (uint32_t)k;
  const uint32_t nchunks = (ku + kAmaxCols - 1) / kAmaxCols;
  const uint32_t nrt = (uint32_t)total / kAmaxRows;  // total is a multiple of 128
  const uint32_t T = nrt * nchunks;
  const uint32_t t_begin = uni((uint32_t)(((uint64_t)blockIdx.x * T) / gridDim.x));
  const uint32_t t_end = uni((uint32_t)(((uint64_t)(blockIdx.x + 1) * T) / gridDim.x));
  if (t_begin >= t_end) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t lcol = lane * 8;  // within the chunk
  auto tile_of = [&](uint32_t t) {
    return AmaxTile{(int32_t)uni(t % nrt) * kAmaxRows, (int32_t)uni(t / nrt)};
  };
  auto lane_off = [&](int32_t chunk) -> uint32_t {
    return (uint32_t)chunk * kAmaxCols + lcol < ku ? (16u * wave * ku + lcol) * 2u : kOutOfRange;
  };

  uint32_t c[4] = {0, 0, 0, 0};  // running column maxima (2 bf16 columns per word)
  int key_e = -1, key_chunk = -1;

  auto flush_cols = [&]() {
    __syncthreads();  // previous readers of l_col are done
#pragma unroll
    for (int j = 0; j < 4; ++j) l_col[wave][lane * 4 + j] = c[j];
    __syncthreads();
    const int p = threadIdx.x;  // one column pair per thread
    const uint32_t m = pkmax(pkmax(l_col[0][p], l_col[1][p]), pkmax(l_col[2][p], l_col[3][p]));
    const uint32_t col = (uint32_t)key_chunk * kAmaxCols + 2 * p;
    if (col < ku) {
      uint32_t* dst = col_amax + (int64_t)key_e * k + col;
      atomicMax(dst, m << 16);
      atomicMax(dst + 1, m & 0xFFFF0000u);
    }
  };

  uint32_t va[16][4], vb[16][4];
  AmaxTile cur = tile_of(t_begin);
  amax_load(x, ku, cur.row0, cur.chunk, lane_off(cur.chunk), va);

  auto process = [&](uint32_t (&v)[16][4], AmaxTile tl) {
    int32_t rbeg, rend;
    const int e = find_expert(R, tl.row0, &rbeg, &rend);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i][j] &= 0x7FFF7FFFu;
    if (col_amax) {
      if (e != key_e || tl.chunk != key_chunk) {
        if (key_e >= 0) flush_cols();
        c[0] = c[1] = c[2] = c[3] = 0;
        key_e = e;
        key_chunk = tl.chunk;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) c[j] = pkmax(c[j], v[i][j]);
    }
    if (row_amax) {
      // rows (2p, 2p+1) of the wave packed in one word, p = 0..7
      uint32_t rp[8];
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) {
        const uint32_t a = pkmax(pkmax(v[2 * pr][0], v[2 * pr][1]), pkmax(v[2 * pr][2], v[2 * pr][3]));
        const uint32_t b = pkmax(pkmax(v[2 * pr + 1][0], v[2 * pr + 1][1]),
                                 pkmax(v[2 * pr + 1][2], v[2 * pr + 1][3]));
        rp[pr] = pkmax((a & 0xFFFFu) | (b << 16), (a >> 16) | (b & 0xFFFF0000u));
      }
      const uint32_t g = wave_reduce_scatter8(rp, lane);  // pair lane/8, all 64 lanes reduced
      if ((lane & 7) == 0) {
        const int64_t row = (int64_t)tl.row0 + 16 * wave + 2 * (lane >> 3);
        atomicMax(row_amax + row, g << 16);
        atomicMax(row_amax + row + 1, g & 0xFFFF0000u);
      }
    }
  };

#pragma unroll 1
  for (uint32_t t = t_begin; t < t_end; t += 2) {
    AmaxTile nxt = tile_of(t + 1);
    if (t + 1 < t_end) amax_load(x, ku, nxt.row0, nxt.chunk, lane_off(nxt.chunk), vb);
    process(va, cur);
    if (t + 1 >= t_end) break;
    cur = tile_of(t + 2);
    if (t + 2 < t_end) amax_load(x, ku, cur.row0, cur.chunk, lane_off(cur.chunk), va);
    process(vb, nxt);
  }
  if (col_amax && key_e >= 0) flush_cols();
}

// Grouped amax for K <= 2048 (NCH = ceil(K/512) column chunks): tiles of
// whole rows.  Wave w of a workgroup covers RPW rows x all NCH chunks (lane L
// holds columns 512c + 8L .. +7 of each), at most 16 loads of 1 KB, so
// consecutive tiles of a workgroup's range are consecutive rows and
// contiguous memory.  Walking down 512-column chunks instead reads 1 KB
// pieces at the row pitch, which for K = 2048 is 4 KB: 16% slower loads.
// Each row lies in one tile, so row maxima are plain stores; column maxima
// stay in registers (per chunk) while the expert is unchanged and are then
// flushed with one atomic max per column.
template <int NCH>
__global__ __launch_bounds__(kThreads) void group_amax_rows_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R,
    uint32_t* __restrict__ row_amax, uint32_t* __restrict__ col_amax) {
  constexpr int RPW = NCH == 1 ? 16 : NCH == 2 ? 8 : 4;  // rows per wave
  constexpr int TR = 4 * RPW;                            // rows per tile (divides 128)
  __shared__ uint32_t l_col[4][NCH * kAmaxCols / 2];     // per wave, column pairs
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  const uint32_t ku = (uint32_t)k;
  const uint32_t T = (uint32_t)total / TR;
  const uint32_t t_begin = uni((uint32_t)(((uint64_t)blockIdx.x * T) / gridDim.x));
  const uint32_t t_end = uni((uint32_t)(((uint64_t)(blockIdx.x + 1) * T) / gridDim.x));
  if (t_begin >= t_end) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t off[NCH];  // lane offset of chunk c in the wave's first row, or out of range
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t col = 512u * c + 8u * lane;
    off[c] = col < ku ? ((uint32_t)(wave * RPW) * ku + col) * 2u : kOutOfRange;
  }
  auto load = [&](uint32_t t, uint32_t (&v)[RPW][NCH][4]) {
    const rsrc_t xr = make_rsrc(x + (int64_t)t * TR * k);
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(xr, off[c], (uint32_t)r * ku * 2u, kAmaxLoadAux);
        v[r][c][0] = q.x; v[r][c][1] = q.y; v[r][c][2] = q.z; v[r][c][3] = q.w;
      }
  };

  uint32_t cm[NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c) cm[c][0] = cm[c][1] = cm[c][2] = cm[c][3] = 0;
  int key_e = -1;
  auto flush_cols = [&]() {
    __syncthreads();  // previous readers of l_col are done
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) l_col[wave][c * (kAmaxCols / 2) + lane * 4 + j] = cm[c][j];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int p = c * (kAmaxCols / 2) + threadIdx.x;  // one column pair per thread and chunk
      const uint32_t m = pkmax(pkmax(l_col[0][p], l_col[1][p]), pkmax(l_col[2][p], l_col[3][p]));
      const uint32_t col = 2u * p;
      if (col < ku) {
        uint32_t* dst = col_amax + (int64_t)key_e * k + col;
        atomicMax(dst, m << 16);
        atomicMax(dst + 1, m & 0xFFFF0000u);
      }
    }
  };
  auto process = [&](uint32_t t, uint32_t (&v)[RPW][NCH][4]) {
    const int32_t row0 = (int32_t)(t * TR);
    int32_t rbeg, rend;
    const int e = find_expert(R, row0, &rbeg, &rend);
    if (col_amax && e != key_e) {
      if (key_e >= 0) flush_cols();
#pragma unroll
      for (int c = 0; c < NCH; ++c) cm[c][0] = cm[c][1] = cm[c][2] = cm[c][3] = 0;
      key_e = e;
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[r][c][j] &= 0x7FFF7FFFu;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < RPW; ++r) cm[c][j] = pkmax(cm[c][j], v[r][c][j]);
    uint32_t rw[RPW];  // per row: max over the lane's columns, two halves
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      uint32_t m = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        m = pkmax(m, pkmax(pkmax(v[r][c][0], v[r][c][1]), pkmax(v[r][c][2], v[r][c][3])));
      rw[r] = m;
    }
    if (row_amax) {
      // rows (2p, 2p+1) of the wave packed in one word, p < RPW/2; the rest 0
      uint32_t rp[8];
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) {
        if (2 * pr + 1 < RPW) {
          const uint32_t a = rw[2 * pr], b = rw[2 * pr + 1];
          rp[pr] = pkmax((a & 0xFFFFu) | (b << 16), (a >> 16) | (b & 0xFFFF0000u));
        } else {
          rp[pr] = 0;
        }
      }
      const uint32_t g = wave_reduce_scatter8(rp, lane);  // pair lane/8, all 64 lanes reduced
      if ((lane & 7) == 0 && 2 * (lane >> 3) < RPW) {
        const int64_t row = (int64_t)row0 + RPW * wave + 2 * (lane >> 3);
        row_amax[row] = g << 16;
        row_amax[row + 1] = g & 0xFFFF0000u;
      }
    }
  };

  uint32_t va[RPW][NCH][4], vb[RPW][NCH][4];
  load(t_begin, va);
#pragma unroll 1
  for (uint32_t t = t_begin; t < t_end; t += 2) {
    if (t + 1 < t_end) load(t + 1, vb);
    process(t, va);
    if (t + 1 >= t_end) break;
    if (t + 2 < t_end) load(t + 2, va);
    process(t + 1, vb);
  }
  if (col_amax && key_e >= 0) flush_cols();
}

// Grouped cast of one 128 x 256 tile; rowwise and/or columnwise.
//
// Rowwise data is staged in LDS and written a whole 128-byte row line per
// eight lanes (16 bytes each): written straight from the lane layout, a line
// would be assembled from four waves' 32-byte pieces, four times the store
// requests.  In LDS, the 16-byte granule q of row r sits at slot
// q ^ ((r / 16) % 8), so the 4-byte writes of a wave (lanes on eight rows
// 16 apart, same dword column) fall in distinct banks.
//
// Addressing: every tensor is reached through a raw buffer descriptor whose
// base is the tile's first element, a per-lane 32-bit offset and a scalar
// per-row (or per-column) offset, so no per-store 64-bit address arithmetic
// is done on the vector ALUs.  Lanes whose columns lie beyond K get an offset
// past the descriptor's range: their loads return 0 and their stores are
// dropped by the hardware range check.
__global__ __launch_bounds__(kThreads) void group_cast_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, uint32_t nrow_tiles,
    const float* __restrict__ row_amax, const float* __restrict__ col_amax,
    uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scale) {
  __shared__ float2 l_row[kTileRows];                   // (s, 1/s) per row of the tile
  __shared__ float2 l_col[kTileCols];                   // (s, 1/s) per column of the tile
  __shared__ StagedRowScales l_rs;
  __shared__ StagedColScales l_cs;
  __shared__ StagedRowData l_rd;
  __shared__ uint32_t l_slow[kThreads / 64];            // per wave: a line needs the exact block step
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
  const uint32_t lcol = wave * 64 + cg * 8;  // lane's first column within the tile
  const bool active = lcol < ncols;
  const uint32_t vo_x = active ? (16u * rb * ku + lcol) * 2u : kOutOfRange;
  {
    int32_t rbeg, rend;
    const int e = find_expert(R, row0, &rbeg, &rend);
    const uint32_t me = (uint32_t)(rend - rbeg);

    // the line amax loads go first: the line scales are then computed while
    // the tile's loads are in flight
    const float a_row = row_data && tid < kTileRows ? row_amax[row0 + tid] : 0.0f;
    const float a_col = col_data && (uint32_t)tid < ncols ? col_amax[(int64_t)e * k + col_base + tid] : 0.0f;
    uint32_t v[16][4];
    load_tile(x + (int64_t)row0 * k + col_base, ku, vo_x, v);
    bool slow_line = false;
    if (row_data && tid < kTileRows) {
      const float s = a_row / 2688.0f;
      l_row[tid] = make_float2(s, 1.0f / s);
      slow_line = !(s >= kFastMinLineScale);
    }
    if (col_data) {
      const float s = a_col / 2688.0f;
      l_col[tid] = make_float2(s, 1.0f / s);
      slow_line = slow_line || ((uint32_t)tid < ncols && !(s >= kFastMinLineScale));
    }
    const bool wave_slow = __ballot(slow_line) != 0;
    if (lane == 0) l_slow[wave] = wave_slow;
    __syncthreads();
    // When every line of the tile has s >= 2^-112 (the usual case) the block
    // steps take the fast path without a per-lane test; otherwise each block
    // step picks its path from its own line scale.
    const bool all_fast = uni((uint32_t)(l_slow[0] | l_slow[1] | l_slow[2] | l_slow[3])) == 0u;

    auto encode = [&](auto fast_tag) {
      constexpr bool kAllFast = decltype(fast_tag)::value;
      if (row_data) {
        // The lane pair (lane, lane^8) holds the two 8-column halves of each
        // 16-column block of its 16 rows.  Iteration i serves rows i and 8+i:
        // the even lane derives the scale of row i, the odd lane that of row
        // 8+i; each sends the partner the half amax it needs, then the two
        // multipliers are swapped back, and both rows are encoded.
        const bool odd = cg & 1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo = hmax(pkmax(pkmax(v[i][0] & 0x7FFF7FFFu, v[i][1] & 0x7FFF7FFFu),
                                         pkmax(v[i][2] & 0x7FFF7FFFu, v[i][3] & 0x7FFF7FFFu)));
          const uint32_t hi = hmax(pkmax(pkmax(v[8 + i][0] & 0x7FFF7FFFu, v[8 + i][1] & 0x7FFF7FFFu),
                                         pkmax(v[8 + i][2] & 0x7FFF7FFFu, v[8 + i][3] & 0x7FFF7FFFu)));
          const uint32_t b16 = max(odd ? hi : lo, swap8(odd ? lo : hi));
          const int ri = odd ? 8 + i : i;
          const float2 sl = l_row[16 * rb + ri];
          float m;
          const uint32_t S = kAllFast ? block_scale_fast(__uint_as_float(b16 << 16), sl.x, sl.y, &m)
                                      : block_step(__uint_as_float(b16 << 16), sl.x, sl.y, &m);
          const float mo = __uint_as_float(swap8(__float_as_uint(m)));
          reinterpret_cast<uint8_t*>(&l_rs[16 * rb + ri][0])[wave * 4 + (cg >> 1)] = (uint8_t)S;
          // bytes lcol/2 .. +3 of rows 16*rb + i and 16*rb + 8 + i: dword
          // 8*wave + cg of the row, swizzled
          const float m_lo = odd ? mo : m, m_hi = odd ? m : mo;
          uint32_t packed = 0;
          packed = FP4X2(packed, bf16lo(v[i][0]) * m_lo, bf16hi(v[i][0]) * m_lo, 0);
          packed = FP4X2(packed, bf16lo(v[i][1]) * m_lo, bf16hi(v[i][1]) * m_lo, 1);
          packed = FP4X2(packed, bf16lo(v[i][2]) * m_lo, bf16hi(v[i][2]) * m_lo, 2);
          packed = FP4X2(packed, bf16lo(v[i][3]) * m_lo, bf16hi(v[i][3]) * m_lo, 3);
          l_rd[16 * rb + i][row_slot(rb, wave, cg)] = packed;
          packed = 0;
          packed = FP4X2(packed, bf16lo(v[8 + i][0]) * m_hi, bf16hi(v[8 + i][0]) * m_hi, 0);
          packed = FP4X2(packed, bf16lo(v[8 + i][1]) * m_hi, bf16hi(v[8 + i][1]) * m_hi, 1);
          packed = FP4X2(packed, bf16lo(v[8 + i][2]) * m_hi, bf16hi(v[8 + i][2]) * m_hi, 2);
          packed = FP4X2(packed, bf16lo(v[8 + i][3]) * m_hi, bf16hi(v[8 + i][3]) * m_hi, 3);
          l_rd[16 * rb + 8 + i][row_slot(rb, wave, cg)] = packed;
        }
      }

      if (col_data) {
        const rsrc_t cd = make_rsrc(col_data + k * (int64_t)rbeg / 2 + col_base * (me / 2) + (row0 - rbeg) / 2);
        const uint32_t vo = active ? lcol * (me / 2) + 8u * rb : kOutOfRange;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t mx = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = pkmax(mx, v[i][j >> 1] & 0x7FFF7FFFu);
          const uint32_t b16 = (j & 1) ? (mx >> 16) : (mx & 0xFFFFu);
          const float2 sl = l_col[lcol + j];
          float m;
          const uint32_t S = kAllFast ? block_scale_fast(__uint_as_float(b16 << 16), sl.x, sl.y, &m)
                                      : block_step(__uint_as_float(b16 << 16), sl.x, sl.y, &m);
          reinterpret_cast<uint8_t*>(&l_cs[lcol + j][0])[rb] = (uint8_t)S;
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
        }
      }
    };
    if (all_fast)
      encode(BoolTag<true>{});
    else
      encode(BoolTag<false>{});

    __syncthreads();
    store_staged_tile(l_rd, l_rs, l_cs, k, row0, col_base, ncols, rbeg, me, row_data, row_scale,
                      col_data ? col_scale : nullptr);
  }
}

// Rowwise-only amax + cast in one pass over x (the per-row form of "Implement
// per-token NVFP4 fprop recipe", Important Files Changed: the row amax and the
// quantisation of the row in one go).  A wave owns whole rows: lane L holds
// columns 512*g + 8L .. +7 for the row's segments g < NSEG (K <= 512*NSEG),
// so each segment load reads 1 KB of the row; the row amax is a wave
// reduction, and a 16-column block is the values of lanes 2j and 2j+1.  The
// next row's loads are in flight while the current row is encoded.  Rows only
// need the routed row count: expert boundaries do not affect rowwise output.
template <int NSEG>
__global__ __launch_bounds__(kThreads) void group_quantize_rowwise_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, float* __restrict__ row_amax,
    uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale) {
  if (!routing_ok(R)) return;
  const uint32_t total = (uint32_t)route_end(R, R.num_experts - 1);
  const uint32_t ku = (uint32_t)k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const uint32_t w0 = blockIdx.x * (kThreads / 64) + wave;
  uint32_t off[NSEG];  // lane's byte offset of each segment within a row (or out of range)
#pragma unroll
  for (int g = 0; g < NSEG; ++g) off[g] = (uint32_t)g * 512u + lane * 8u < ku ? ((uint32_t)g * 512u + lane * 8u) * 2u : kOutOfRange;

  // row indices are wave-uniform: readfirstlane keeps the 64-bit row base in
  // scalar registers, and only the small lane offsets are per lane
  auto load_row = [&](uint32_t r, uint32_t (&v)[NSEG][4]) {
    const rsrc_t xr = make_rsrc(x + (int64_t)__builtin_amdgcn_readfirstlane(r) * k);
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
      const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(xr, off[g], 0, kLoadStream);
      v[g][0] = q.x; v[g][1] = q.y; v[g][2] = q.z; v[g][3] = q.w;
    }
  };
  auto do_row = [&](uint32_t r, uint32_t (&v)[NSEG][4]) {
    // row amax: lane max, then the max over the 64 lanes
    uint32_t a = 0;
#pragma unroll
    for (int g = 0; g < NSEG; ++g)
      a = pkmax(a, pkmax(pkmax(v[g][0] & 0x7FFF7FFFu, v[g][1] & 0x7FFF7FFFu),
                         pkmax(v[g][2] & 0x7FFF7FFFu, v[g][3] & 0x7FFF7FFFu)));
    a = hmax(a);
    a = max(a, dpp_x1(a));
    a = max(a, dpp_x2(a));
    a = max(a, dpp_hmirror(a));
    a = max(a, swap8(a));
    a = max(a, swap32_max(a, a) & 0xFFFFu);
    a = max(a, swap16_max(a, a) & 0xFFFFu);
    const float A = __uint_as_float(a << 16);
    if (lane == 0) row_amax[r] = A;
    const float s = A / 2688.0f, ys = 1.0f / s;
    const rsrc_t rd = make_rsrc(row_data + (int64_t)__builtin_amdgcn_readfirstlane(r) * (k / 2));
    auto encode = [&](auto fast_tag) {
      constexpr bool kFast = decltype(fast_tag)::value;
#pragma unroll
      for (int g = 0; g < NSEG; ++g) {
        uint32_t b = hmax(pkmax(pkmax(v[g][0] & 0x7FFF7FFFu, v[g][1] & 0x7FFF7FFFu),
                                pkmax(v[g][2] & 0x7FFF7FFFu, v[g][3] & 0x7FFF7FFFu)));
        b = max(b, dpp_x1(b));  // the block is lanes 2j, 2j+1
        float m;
        const uint32_t S = kFast ? block_scale_fast(__uint_as_float(b << 16), s, ys, &m)
                                 : block_scale(__uint_as_float(b << 16), s, &m);
        uint32_t packed = 0;
        packed = FP4X2(packed, bf16lo(v[g][0]) * m, bf16hi(v[g][0]) * m, 0);
        packed = FP4X2(packed, bf16lo(v[g][1]) * m, bf16hi(v[g][1]) * m, 1);
        packed = FP4X2(packed, bf16lo(v[g][2]) * m, bf16hi(v[g][2]) * m, 2);
        packed = FP4X2(packed, bf16lo(v[g][3]) * m, bf16hi(v[g][3]) * m, 3);
        const uint32_t c = (uint32_t)g * 512u + lane * 8u;
        __builtin_amdgcn_raw_buffer_store_b32(packed, rd, off[g] == kOutOfRange ? kOutOfRange : c / 2u, 0,
                                              kStoreAux);
        if (!(lane & 1) && c < ku) row_scale[(int64_t)r * (k / 16) + c / 16] = (uint8_t)S;
      }
    };
    // the row's line scale is the same in every lane: one wave-uniform choice
    // between the fast block step and the exact one (block_step's rule)
    if (uni((uint32_t)(s >= kFastMinLineScale)))
      encode(BoolTag<true>{});
    else
      encode(BoolTag<false>{});
  };

  uint32_t va[NSEG][4], vb[NSEG][4];
  uint32_t r = w0;
  if (r < total) load_row(r, va);
#pragma unroll 1
  for (; r < total; r += 2 * nwaves) {
    const uint32_t r1 = r + nwaves;
    if (r1 < total) load_row(r1, vb);
    do_row(r, va);
    if (r1 >= total) break;
    const uint32_t r2 = r1 + nwaves;
    if (r2 < total) load_row(r2, va);
    do_row(r1, vb);
  }
}

// Small inputs in one launch.  When every expert holds at most
// kSmallMaxExpertElems elements (K <= kSmallMaxK follows, an expert having
// 128 rows or none), the general path's three launches (zero-fill, amax,
// cast; ~6 us each, mostly launch latency) cost more than the work.
// kSmallSplit workgroups per expert each run the whole path: copy the
// expert's rows (one contiguous slice of x, at most 128 KB) into LDS with
// every load in flight at once, take the row and column amax there, then
// encode their share of the rowwise and columnwise blocks from LDS -- the
// cast kernel's line scales, block step and FP4 converts, so the bytes are
// the same.  The first of them writes the amax outputs (each element once,
// so with no zero-fill and no atomics); computing the amax in each one costs
// less than leaving all the encoding to one workgroup on one CU.
constexpr int64_t kSmallMaxExpertElems = NVFP4G_SMALL_MAX_EXPERT_ELEMS;
constexpr int64_t kSmallMaxK = NVFP4G_SMALL_MAX_K;
static_assert(kSmallMaxK * 128 == kSmallMaxExpertElems, "K limit = elements of a 128-row expert");
constexpr int kSmallThreads = 1024;                                // 16 waves
constexpr int kSmallSplit = 8;  // workgroups per expert (4 and 16 measured within 5% on the tiny workload)
constexpr int kSmallMaxRows = (int)(kSmallMaxExpertElems / 16);  // K >= 16
constexpr int kSmallLoads = (int)(kSmallMaxExpertElems / 8 / kSmallThreads);  // 16-byte loads per thread

__global__ __launch_bounds__(kSmallThreads) void group_quantize_small_kernel(
    const uint16_t* __restrict__ x, int64_t k, Routing R, float* __restrict__ row_amax,
    float* __restrict__ col_amax, uint8_t* __restrict__ row_data, uint8_t* __restrict__ row_scale,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scale) {
  __shared__ u32x4 l_x[kSmallMaxExpertElems / 8];       // the expert's rows, row-major bf16
  __shared__ uint16_t l_bm[kSmallMaxExpertElems / 16];  // amax of each rowwise 16-block (bf16 bits)
  __shared__ uint16_t l_ra[kSmallMaxRows];              // row amax (bf16 bits)
  __shared__ uint32_t l_cp[kSmallThreads];              // column maxima: partial, then final pairs
  if (!routing_ok(R)) return;
  // The kSmallSplit work-groups of an expert share one XCD (work-groups are
  // dealt to the XCDs round-robin by index): the expert's rows then come
  // from HBM once and from that XCD's L2 for the others.  Indexes past the
  // last expert (E not a multiple of kNumXcd) exit.
  const uint32_t L = blockIdx.x;
  const int e = (int)(kNumXcd * (L / (kNumXcd * kSmallSplit)) + L % kNumXcd);
  const int g = (int)((L / kNumXcd) % kSmallSplit);
  if (e >= R.num_experts) return;
  const int32_t rend = route_end(R, e), rbeg = e ? route_end(R, e - 1) : 0;
  const uint32_t me = (uint32_t)(rend - rbeg);
  const int tid = threadIdx.x;
  const bool writer = g == 0;  // the one workgroup of the expert that writes its amax
  const uint32_t ku = (uint32_t)k, kp = ku / 2, kq = ku / 8;  // bf16 pairs, 16-byte pieces per row
  const uint16_t* lx16 = reinterpret_cast<const uint16_t*>(l_x);
  const uint32_t* lx32 = reinterpret_cast<const uint32_t*>(l_x);

  // the expert's slice: me * k contiguous bf16, all loads issued before any store
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)rbeg * k);
    const uint32_t n = me * kq;
    u32x4 v[kSmallLoads];
#pragma unroll
    for (int u = 0; u < kSmallLoads; ++u) {
      const uint32_t i = tid + u * kSmallThreads;
      v[u] = i < n ? src[i] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kSmallLoads; ++u) {
      const uint32_t i = tid + u * kSmallThreads;
      if (i < n) l_x[i] = v[u];
    }
  }
  __syncthreads();

  // the amax of every rowwise 16-block (magnitude bits: bf16 magnitudes
  // order as their bit patterns)
  const uint32_t nb = ku / 16;
  for (uint32_t q = tid; q < me * nb; q += kSmallThreads) {
    const u32x4 q0 = l_x[2 * q], q1 = l_x[2 * q + 1];
    l_bm[q] = (uint16_t)hmax(pkmax(pkmax(pkmax(q0.x & 0x7FFF7FFFu, q0.y & 0x7FFF7FFFu),
                                         pkmax(q0.z & 0x7FFF7FFFu, q0.w & 0x7FFF7FFFu)),
                                   pkmax(pkmax(q1.x & 0x7FFF7FFFu, q1.y & 0x7FFF7FFFu),
                                         pkmax(q1.z & 0x7FFF7FFFu, q1.w & 0x7FFF7FFFu))));
  }
  // column amax: thread t takes column pair t % kp over rows t / kp + nseg * j
  const uint32_t nseg = kSmallThreads / kp;
  {
    uint32_t m = 0;
    if ((uint32_t)tid < nseg * kp) {
      const uint32_t p = tid % kp;
      for (uint32_t r = tid / kp; r < me; r += nseg) m = pkmax(m, lx32[r * kp + p] & 0x7FFF7FFFu);
    }
    l_cp[tid] = m;
  }
  __syncthreads();
  // row amax: the max of the row's block maxima, a thread per row
  for (uint32_t r = tid; r < me; r += kSmallThreads) {
    uint32_t m = 0;
    for (uint32_t b = 0; b < nb; ++b) m = max(m, (uint32_t)l_bm[r * nb + b]);
    l_ra[r] = (uint16_t)m;
    if (row_amax && writer) row_amax[rbeg + r] = __uint_as_float(m << 16);
  }
  uint32_t cpair = 0;
  if ((uint32_t)tid < kp) {
    for (uint32_t sg = 0; sg < nseg; ++sg) cpair = pkmax(cpair, l_cp[sg * kp + tid]);
    if (col_amax && writer) {
      col_amax[(int64_t)e * k + 2 * tid] = __uint_as_float(cpair << 16);
      col_amax[(int64_t)e * k + 2 * tid + 1] = __uint_as_float(cpair & 0xFFFF0000u);
    }
  }
  __syncthreads();  // every partial read before the final pairs replace them
  if ((uint32_t)tid < kp) l_cp[tid] = cpair;
  __syncthreads();

  // rowwise: a 16-element block per thread and pass (block q of the slice
  // is elements 16q .. 16q+15: row q / nb, block q % nb)
  if (row_data) {
    for (uint32_t q = tid + g * kSmallThreads; q < me * nb; q += kSmallSplit * kSmallThreads) {
      const uint32_t i = q / nb, b = q % nb;
      const u32x4 q0 = l_x[2 * q], q1 = l_x[2 * q + 1];
      const uint32_t bm = l_bm[q];
      const float s = __uint_as_float((uint32_t)l_ra[i] << 16) / 2688.0f;
      float m;
      const uint32_t S = block_step(__uint_as_float(bm << 16), s, 1.0f / s, &m);
      uint32_t p0 = 0, p1 = 0;
      p0 = FP4X2(p0, bf16lo(q0.x) * m, bf16hi(q0.x) * m, 0);
      p0 = FP4X2(p0, bf16lo(q0.y) * m, bf16hi(q0.y) * m, 1);
      p0 = FP4X2(p0, bf16lo(q0.z) * m, bf16hi(q0.z) * m, 2);
      p0 = FP4X2(p0, bf16lo(q0.w) * m, bf16hi(q0.w) * m, 3);
      p1 = FP4X2(p1, bf16lo(q1.x) * m, bf16hi(q1.x) * m, 0);
      p1 = FP4X2(p1, bf16lo(q1.y) * m, bf16hi(q1.y) * m, 1);
      p1 = FP4X2(p1, bf16lo(q1.z) * m, bf16hi(q1.z) * m, 2);
      p1 = FP4X2(p1, bf16lo(q1.w) * m, bf16hi(q1.w) * m, 3);
      *reinterpret_cast<u32x2*>(row_data + (int64_t)(rbeg + i) * (k / 2) + 8 * b) = u32x2{p0, p1};
      row_scale[(int64_t)(rbeg + i) * (k / 16) + b] = (uint8_t)S;
    }
  }
  // columnwise: a 16-row block of a column per thread and pass (adjacent
  // threads take adjacent columns)
  if (col_data) {
    const uint32_t nrb = me / 16;
    uint8_t* cd = col_data + (int64_t)k * rbeg / 2;
    uint8_t* cs = col_scale + (int64_t)k * rbeg / 16;
    for (uint32_t q = tid + g * kSmallThreads; q < ku * nrb; q += kSmallSplit * kSmallThreads) {
      const uint32_t c = q % ku, rb = q / ku;
      uint32_t w[16], bm = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        w[i] = lx16[(16 * rb + i) * ku + c];
        bm = max(bm, w[i] & 0x7FFFu);
      }
      const uint32_t pm = l_cp[c >> 1];
      const float s = __uint_as_float(((c & 1) ? (pm >> 16) : (pm & 0xFFFFu)) << 16) / 2688.0f;
      float m;
      const uint32_t S = block_step(__uint_as_float(bm << 16), s, 1.0f / s, &m);
      uint32_t p0 = 0, p1 = 0;
      p0 = FP4X2(p0, __uint_as_float(w[0] << 16) * m, __uint_as_float(w[1] << 16) * m, 0);
      p0 = FP4X2(p0, __uint_as_float(w[2] << 16) * m, __uint_as_float(w[3] << 16) * m, 1);
      p0 = FP4X2(p0, __uint_as_float(w[4] << 16) * m, __uint_as_float(w[5] << 16) * m, 2);
      p0 = FP4X2(p0, __uint_as_float(w[6] << 16) * m, __uint_as_float(w[7] << 16) * m, 3);
      p1 = FP4X2(p1, __uint_as_float(w[8] << 16) * m, __uint_as_float(w[9] << 16) * m, 0);
      p1 = FP4X2(p1, __uint_as_float(w[10] << 16) * m, __uint_as_float(w[11] << 16) * m, 1);
      p1 = FP4X2(p1, __uint_as_float(w[12] << 16) * m, __uint_as_float(w[13] << 16) * m, 2);
      p1 = FP4X2(p1, __uint_as_float(w[14] << 16) * m, __uint_as_float(w[15] << 16) * m, 3);
      *reinterpret_cast<u32x2*>(cd + (int64_t)c * (me / 2) + 8 * rb) = u32x2{p0, p1};
      cs[(int64_t)c * (me / 16) + rb] = (uint8_t)S;
    }
  }
}

// ------------------------------------------------------------- host side

// Persistent amax grid: enough resident workgroups to cover the device
// (at most the number of 64 x 512 tiles of the buffers).
#ifndef NVFP4G_AMAX_WGS
#define NVFP4G_AMAX_WGS 768
#endif
unsigned amax_grid(int64_t rows, int64_t k) {
  const int64_t tiles = (rows / kAmaxRows) * ((k + kAmaxCols - 1) / kAmaxCols);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(tiles, NVFP4G_AMAX_WGS));
}

int launch_amax(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, float* row_amax,
                float* col_amax, hipStream_t st) {
  if (!row_amax && !col_amax) return NVFP4G_OK;
  const int64_t n = (row_amax ? rows : 0) + (col_amax ? (int64_t)R.num_experts * k : 0);
  const unsigned init_blocks = (unsigned)std::min<int64_t>(std::max<int64_t>((n + kThreads - 1) / kThreads, 1), 4096);
  hipLaunchKernelGGL(amax_init_kernel, dim3(init_blocks), dim3(kThreads), 0, st, R, k, row_amax, col_amax);
  if (rows > 0) {
    uint32_t* ra = reinterpret_cast<uint32_t*>(row_amax);
    uint32_t* ca = reinterpret_cast<uint32_t*>(col_amax);
    // K <= 2048: tiles of whole rows (16 - 64 rows); up to 175 VGPRs, two workgroups per CU
    const unsigned g = (unsigned)std::max<int64_t>(1, std::min<int64_t>(rows / 16, 512));
    if (k <= 512)
      hipLaunchKernelGGL(group_amax_rows_kernel<1>, dim3(g), dim3(kThreads), 0, st, x, k, R, ra, ca);
    else if (k <= 1024)
      hipLaunchKernelGGL(group_amax_rows_kernel<2>, dim3(g), dim3(kThreads), 0, st, x, k, R, ra, ca);
    else if (k <= 1536)
      hipLaunchKernelGGL(group_amax_rows_kernel<3>, dim3(g), dim3(kThreads), 0, st, x, k, R, ra, ca);
    else if (k <= 2048)
      hipLaunchKernelGGL(group_amax_rows_kernel<4>, dim3(g), dim3(kThreads), 0, st, x, k, R, ra, ca);
    else
      hipLaunchKernelGGL(group_amax_kernel, dim3(amax_grid(rows, k)), dim3(kThreads), 0, st, x, k, R, ra, ca);
  }
  return hip_status();
}

int launch_cast(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, const float* row_amax,
                const float* col_amax, uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                uint8_t* col_scale, hipStream_t st) {
  if ((!row_data && !col_data) || rows == 0) return NVFP4G_OK;
  hipLaunchKernelGGL(group_cast_kernel, tile_grid(rows, k), dim3(kThreads), 0, st, x, k, R, num_row_tiles(rows), row_amax,
                     col_amax, row_data, row_scale, col_data, col_scale);
  return hip_status();
}

// Fused rowwise amax + cast (K <= 8192): one wave per row at a time over a
// grid of resident workgroups.
constexpr int64_t kRowFusedMaxK = 8192;

int launch_rowwise_fused(const uint16_t* x, int64_t rows, int64_t k, const Routing& R, float* row_amax,
                         uint8_t* row_data, uint8_t* row_scale, hipStream_t st) {
  if (rows == 0) return NVFP4G_OK;
  // 4 waves per workgroup, one row per wave up to 2048 workgroups (a small
  // problem then has every load in flight at once; 8192 x 2048: 10.5 us
  // against 11.8 us with 4 rows per wave), more rows per wave beyond
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((rows + 3) / 4, 2048));
  if (k <= 2048)
    hipLaunchKernelGGL(group_quantize_rowwise_kernel<4>, dim3(grid), dim3(kThreads), 0, st, x, k, R, row_amax,
                       row_data, row_scale);
  else if (k <= 4096)
    hipLaunchKernelGGL(group_quantize_rowwise_kernel<8>, dim3(grid), dim3(kThreads), 0, st, x, k, R, row_amax,
                       row_data, row_scale);
  else
    hipLaunchKernelGGL(group_quantize_rowwise_kernel<16>, dim3(grid), dim3(kThreads), 0, st, x, k, R, row_amax,
                       row_data, row_scale);
  return hip_status();
}

// One launch for small inputs with a columnwise output (see the kernel):
// every expert's rows times k within the limit -- for host splits the
// largest expert, for device routing the capacity (any expert may hold it).
bool small_input(int64_t max_expert_rows, int64_t k) {
  return max_expert_rows * k <= kSmallMaxExpertElems && k <= kSmallMaxK;
}
int64_t max_expert_rows(const Routing& R) {
  int64_t mx = 0;
  for (int e = 0; e < R.num_experts; ++e)
    mx = std::max<int64_t>(mx, (int64_t)R.h_offs[e] - (e ? R.h_offs[e - 1] : 0));
  return mx;
}

int launch_small(const uint16_t* x, int64_t k, const Routing& R, float* row_amax, float* col_amax,
                 uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale, hipStream_t st) {
  const unsigned groups = (unsigned)((R.num_experts + kNumXcd - 1) / kNumXcd);  // of kNumXcd experts
  hipLaunchKernelGGL(group_quantize_small_kernel, dim3(groups * kNumXcd * kSmallSplit), dim3(kSmallThreads), 0, st, x,
                     k, R, row_data ? row_amax : nullptr, col_amax, row_data, row_scale, col_data, col_scale);
  return hip_status();
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
  if (row_data && !col_data && k <= kRowFusedMaxK)
    return launch_rowwise_fused(x, sum_m, k, R, row_amax, row_data, row_scale, st);
  if (col_data && small_input(max_expert_rows(R), k))
    return launch_small(x, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale, st);
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
  if (row_data && !col_data && k <= kRowFusedMaxK)
    return launch_rowwise_fused(x, m_capacity, k, R, row_amax, row_data, row_scale, st);
  if (col_data && small_input(m_capacity, k))
    return launch_small(x, k, R, row_amax, col_amax, row_data, row_scale, col_data, col_scale, st);
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
