// nvfp4_common.hpp -- routing, buffer addressing and host-side argument
// checks shared by the HIP sources of libnvfp4g.so.
//
// Routing: expert e owns rows [end(e-1), end(e)) of the packed buffer, with
// end() the inclusive row ends, taken from the kernel arguments for host
// splits or from device memory for the graph-safe calls (TransformerEngine
// issue 3649 page, Description: the graph-safe twins read the routing from
// device offsets and share the device body).  Every expert's row count is a
// multiple of 128 (the token dispatcher pads groups to 128 rows, torchtitan
// PR 14 page, Design notes).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4_group.h"

namespace nvfp4g {

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

// Values that are uniform over a workgroup (routing, tile coordinates) are
// passed through readfirstlane so the compiler keeps them, and the buffer
// descriptors built from them, in scalar registers.
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint32_t lo = uni((uint32_t)v), hi = uni((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Inclusive row end of expert e, for an e that is the same in every lane.
__device__ __forceinline__ int32_t route_end(const Routing& R, int e) {
  return uni(R.d_offs ? R.d_offs[e] : R.h_offs[e]);
}
// The same for an e that may differ between lanes.
__device__ __forceinline__ int32_t route_end_lane(const Routing& R, int e) {
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

// ------------------------------------------------------------ addressing

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor (gfx9 layout: 32-bit data format word) over `base`.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
// Offset of a lane that must not touch memory: beyond the descriptor range.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache policy bits: streaming (non-temporal) loads of x; plain stores.
constexpr int kLoadStream = 2;
// Load policy of the amax pass and of the cast's tile loads (both streaming
// by default; overridable at build time for measurements).
#ifndef NVFP4G_AMAX_LOAD_AUX
#define NVFP4G_AMAX_LOAD_AUX 2
#endif
#ifndef NVFP4G_CAST_LOAD_AUX
#define NVFP4G_CAST_LOAD_AUX 2
#endif
constexpr int kAmaxLoadAux = NVFP4G_AMAX_LOAD_AUX;
constexpr int kCastLoadAux = NVFP4G_CAST_LOAD_AUX;
#ifndef NVFP4G_STORE_AUX
#define NVFP4G_STORE_AUX 0
#endif
constexpr int kStoreAux = NVFP4G_STORE_AUX;
// Streaming (non-temporal) stores, for the transposed (columnwise) data: its
// two 64-byte halves of a 128-byte line come from vertically adjacent tiles
// processed together on one XCD, and writing them past the caches' normal
// retention measured faster than plain stores (plain stores stay better for
// the rowwise data and for the small scale stores).
constexpr int kStoreStream = 2;

// Compile-time flag passed to a generic lambda (one instantiation per value).
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// ------------------------------------------------------------- tiles

// Tile order of the cast kernel.  Work-groups are dispatched round-robin
// over the 8 XCDs, each with its own L2; the linear block id is remapped so
// that each XCD gets a contiguous run of logical tiles, ordered row tile
// first within a 256-column chunk.  Vertically adjacent tiles, which write
// the two 64-byte halves of each 128-byte line of the transposed output, then
// go through the same L2 at about the same time.
constexpr int kNumXcd = 8;

struct TileCoord {
  uint32_t row_tile, chunk;
};

__device__ __forceinline__ TileCoord tile_coord(uint32_t nrow_tiles) {
  const uint32_t nb = gridDim.x, L = blockIdx.x;
  const uint32_t xcd = L % kNumXcd, q = nb / kNumXcd, r = nb % kNumXcd;
  const uint32_t lt = xcd * q + min(xcd, r) + L / kNumXcd;  // a permutation of 0..nb-1
  return TileCoord{uni(lt % nrow_tiles), uni(lt / nrow_tiles)};
}

// Loads the lane's 16 rows x 8 columns (16 x 16 bytes) of a 128 x 256 tile
// whose first element is `tile`; `vo` is the lane's byte offset (or
// kOutOfRange), row i adds i*K*2 bytes as a scalar offset.
__device__ __forceinline__ void load_tile(const uint16_t* tile, uint32_t ku, uint32_t vo,
                                          uint32_t (&v)[16][4]) {
  const rsrc_t xr = make_rsrc(tile);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(xr, vo, (uint32_t)i * ku * 2u, kCastLoadAux);
    v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
  }
}

// --------------------------------------------------- staged tile outputs

// The NVFP4 cast kernels stage a tile's rowwise codes and both directions'
// scales in LDS and write them after a barrier.  Rowwise codes: 128 rows x
// 128 bytes; the lane holding rows 16*rb.. and columns 8*cg.. of wave w
// writes dword 8*w + cg of a row, at slot (8*w + cg) ^ (4*rb): the 16-byte
// granule q of row r sits at granule slot q ^ ((r / 16) % 8), so the 4-byte
// writes of a wave (lanes on eight rows 16 apart, same dword column) fall in
// distinct banks.  Scales: 16 bytes per row, 8 per column (one per 16-row
// block).
typedef uint32_t StagedRowData[kTileRows][kTileCols / 8];
typedef uint32_t StagedRowScales[kTileRows][kTileCols / 64];
typedef uint32_t StagedColScales[kTileCols][2];

__device__ __forceinline__ uint32_t row_slot(int rb, int wave, int cg) { return (uint32_t)((8 * wave + cg) ^ (rb << 2)); }

// Writes a staged 128 x 256 tile (ncols <= 256 valid columns from col_base,
// rows row0.. of the expert owning rows [rbeg, rbeg + me)): whole 128-byte
// row lines, 16 bytes per thread (thread t: granule t % 8 of rows t / 8 +
// 32 * it; a granule of a ragged last chunk may hold only 16 valid columns),
// one 16-byte row-scale piece per row and one 8-byte column-scale piece per
// column.  row_data == nullptr skips the rowwise output, col_scale ==
// nullptr the column scales.
__device__ __forceinline__ void store_staged_tile(const StagedRowData& l_rd, const StagedRowScales& l_rs,
                                                  const StagedColScales& l_cs, int64_t k, int32_t row0,
                                                  int64_t col_base, uint32_t ncols, int32_t rbeg, uint32_t me,
                                                  uint8_t* row_data, uint8_t* row_scale, uint8_t* col_scale) {
  const int tid = threadIdx.x;
  const uint32_t ku = (uint32_t)k;
  if (row_data) {
    const rsrc_t rd = make_rsrc(row_data + (int64_t)row0 * (k / 2) + col_base / 2);
    const uint32_t g = tid & 7;
#pragma unroll
    for (int it = 0; it < kTileRows / 32; ++it) {
      const uint32_t r = 32 * it + (tid >> 3);
      const u32x4 q = *reinterpret_cast<const u32x4*>(&l_rd[r][4 * (g ^ ((r >> 4) & 7))]);
      if (32 * g + 32 <= ncols)
        __builtin_amdgcn_raw_buffer_store_b128(q, rd, r * (ku / 2) + 16 * g, 0, kStoreAux);
      else if (32 * g < ncols)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, rd, r * (ku / 2) + 16 * g, 0, kStoreAux);
    }
  }
  if (row_data && tid < kTileRows) {
    uint8_t* dst = row_scale + ((int64_t)row0 + tid) * (k / 16) + col_base / 16;
    if (ncols == kTileCols && (k & 255) == 0) {
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&l_rs[tid][0]);
    } else {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(&l_rs[tid][0]);
      for (uint32_t b = 0; b < ncols / 16; ++b) dst[b] = src[b];
    }
  }
  if (col_scale && (uint32_t)tid < ncols) {
    uint8_t* dst = col_scale + k * (int64_t)rbeg / 16 + (col_base + tid) * (int64_t)(me / 16) + (row0 - rbeg) / 16;
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&l_cs[tid][0]);
  }
}

// ------------------------------------------------------------- host side

constexpr int64_t kMaxK = NVFP4G_MAX_K;
constexpr int64_t kMaxRows = NVFP4G_MAX_ROWS;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int hip_status() {
  return hipGetLastError() == hipSuccess ? NVFP4G_OK : NVFP4G_EHIP;
}

// Common static checks; fills R (all but the offsets).
inline int check_common(const void* x, int64_t rows, int64_t k, int32_t E, Routing* R) {
  // size limits keep every per-lane and per-row buffer offset below 2^31
  if (k <= 0 || k % 16 != 0 || k > kMaxK) return NVFP4G_EINVAL;
  if (rows < 0 || rows > kMaxRows) return NVFP4G_EINVAL;
  if (rows > 0 && x == nullptr) return NVFP4G_EINVAL;
  if (!aligned(x, 16)) return NVFP4G_EALIGN;
  R->num_experts = E;
  R->m_capacity = (int32_t)rows;
  R->d_offs = nullptr;
  R->d_status = nullptr;
  return NVFP4G_OK;
}

inline int host_routing(const int64_t* h_splits, int64_t sum_m, int32_t E, Routing* R) {
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

inline int graph_routing(const int32_t* d_offs, int32_t* d_status, int32_t E, int64_t m_capacity, Routing* R) {
  if (E < 1 || E > NVFP4G_MAX_EXPERTS_DEVICE) return NVFP4G_EINVAL;
  if (!d_offs || !d_status || m_capacity % kTileRows != 0) return NVFP4G_EINVAL;
  if (!aligned(d_offs, 4) || !aligned(d_status, 4)) return NVFP4G_EALIGN;
  R->d_offs = d_offs;
  R->d_status = d_status;
  return NVFP4G_OK;
}

// Outputs of a cast: a direction is produced when its data pointer is set,
// and then needs its scales and amax.
inline int check_cast_outputs(const float* row_amax, const float* col_amax, const uint8_t* row_data,
                              const uint8_t* row_scale, const uint8_t* col_data, const uint8_t* col_scale) {
  if (row_data && (!row_scale || !row_amax)) return NVFP4G_EINVAL;
  if (col_data && (!col_scale || !col_amax)) return NVFP4G_EINVAL;
  if (!aligned(row_data, 16) || !aligned(row_scale, 16) || !aligned(col_data, 16) ||
      !aligned(col_scale, 16) || !aligned(row_amax, 4) || !aligned(col_amax, 4))
    return NVFP4G_EALIGN;
  return NVFP4G_OK;
}

// 1-D grid of 128-row tiles x 256-column chunks for the cast kernel.
inline uint32_t num_row_tiles(int64_t rows) { return (uint32_t)((rows + kTileRows - 1) / kTileRows); }
inline dim3 tile_grid(int64_t rows, int64_t k) {
  return dim3(num_row_tiles(rows) * (unsigned)((k + kTileCols - 1) / kTileCols));
}

}  // namespace nvfp4g
