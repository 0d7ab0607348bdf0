// hbm_probe.hip -- measurement kernels for the benchmark's memory ceiling
// (libhbmprobe.so; not part of the C ABI of libnvfp4g.so).
//
// What the memory system of one MI355X moves when nothing but memory
// traffic is asked of it, measured with kernels written the way the cast
// kernels are (16-byte buffer loads and stores, streaming cache policy):
//   hbm_probe_read   -- a read-only stream (non-temporal loads);
//   hbm_probe_fill   -- a write-only stream;
//   hbm_probe_copy   -- a copy (non-temporal loads, streaming stores);
//   hbm_probe_mix    -- each work-group iteration reads 64 KB and writes
//                       w KB contiguous (streaming stores), the read/write
//                       ratio of the grouped cast in its simplest layout;
//   hbm_probe_cast_pattern -- the grouped cast's own loads and stores (same
//                       tiles, tile order, addresses, sizes and cache bits)
//                       with the arithmetic removed: each stored word is an
//                       XOR of loaded words.
// Every kernel's indexes are bounded by the sizes passed in; the host entry
// points check those sizes before launching.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
constexpr int kNt = 2;              // non-temporal / streaming cache policy
constexpr uint32_t kOut = 0x80000000u;  // offset beyond any descriptor range: dropped
constexpr int kChunk = 256 * 16 * 8;    // bytes a work-group moves per iteration (8 x 16 B per thread)

__global__ __launch_bounds__(256) void read_kernel(const uint8_t* __restrict__ src, uint64_t niter, uint32_t* sink) {
  uint32_t acc = 0;
  for (uint64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const rsrc_t r = make_rsrc(src + it * kChunk);
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + threadIdx.x) * 16, 0, kNt);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;  // keeps the loads; practically never taken
}

__global__ __launch_bounds__(256) void fill_kernel(uint8_t* __restrict__ dst, uint64_t niter) {
  const u32x4 v = {threadIdx.x, blockIdx.x, 0x5A5A5A5Au, 0xA5A5A5A5u};
  for (uint64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const rsrc_t w = make_rsrc(dst + it * kChunk);
#pragma unroll
    for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(v, w, (u * 256 + threadIdx.x) * 16, 0, kNt);
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   uint64_t niter) {
  for (uint64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const rsrc_t r = make_rsrc(src + it * kChunk);
    const rsrc_t w = make_rsrc(dst + it * kChunk);
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + threadIdx.x) * 16, 0, kNt);
#pragma unroll
    for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], w, (u * 256 + threadIdx.x) * 16, 0, kNt);
  }
}

// one work-group per 64 KB of src; writes W 4-KB units (W of 16) contiguously
template <int W>
__global__ __launch_bounds__(256) void mix_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  const uint64_t it = blockIdx.x;
  const rsrc_t r = make_rsrc(src + it * 65536);
  u32x4 v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (u * 256 + threadIdx.x) * 16, 0, kNt);
  const rsrc_t w = make_rsrc(dst + it * (4096u * W));
#pragma unroll
  for (int s = 0; s < W; ++s) {
    u32x4 o = v[s];
#pragma unroll
    for (int q = s + W; q < 16; q += W) o ^= v[q];
    __builtin_amdgcn_raw_buffer_store_b128(o, w, (s * 256 + threadIdx.x) * 16, 0, kNt);
  }
}

// The grouped cast's memory pattern (see the cast kernel): 128 x 256 tiles,
// the XCD-contiguous tile order, lane L holding rows 16*(L%8)..+15 and
// columns 8*(L/8)..+7 of its wave's 64 columns; transposed data as 8-byte
// streaming stores per lane and column; after a work-group barrier, rowwise
// data as 16-byte stores (whole 128-byte lines per row), 16 bytes of row
// scales per row and 8 bytes of column scales per column.
constexpr int kMaxExperts = 512;
struct Splits {
  int32_t n;
  int32_t end[kMaxExperts];  // inclusive row ends
};

__global__ __launch_bounds__(256) void cast_pattern_kernel(
    const uint16_t* __restrict__ x, int64_t k, Splits S, uint32_t nrt, uint8_t* __restrict__ row_data,
    uint8_t* __restrict__ row_scale, uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scale) {
  const uint32_t nb = gridDim.x, L = blockIdx.x;
  const uint32_t xcd = L % 8, q = nb / 8, r = nb % 8;
  const uint32_t lt = xcd * q + min(xcd, r) + L / 8;
  const uint32_t rt = lt % nrt, chunk = lt / nrt;
  const int32_t row0 = (int32_t)rt * 128;
  const int64_t col_base = (int64_t)chunk * 256;
  const uint32_t ncols = (uint32_t)min<int64_t>(k - col_base, 256);
  const uint32_t ku = (uint32_t)k;
  int lo = 0, hi = S.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (S.end[mid] > row0) hi = mid; else lo = mid + 1;
  }
  const int32_t rend = S.end[lo], rbeg = lo ? S.end[lo - 1] : 0;
  const uint32_t me = (uint32_t)(rend - rbeg);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, rb = lane & 7, cg = lane >> 3;
  const uint32_t lcol = wave * 64 + cg * 8;
  const bool active = lcol < ncols;
  const rsrc_t xr = make_rsrc(x + (int64_t)row0 * k + col_base);
  const uint32_t vo = active ? (16u * rb * ku + lcol) * 2u : kOut;
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, vo, (uint32_t)i * ku * 2u, kNt);
  u32x4 f = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) f ^= v[i];
  // transposed data: column lcol + j of the tile, 16 rows of this lane
  const rsrc_t cd = make_rsrc(col_data + k * (int64_t)rbeg / 2 + col_base * (me / 2) + (row0 - rbeg) / 2);
  const uint32_t vc = active ? lcol * (me / 2) + 8u * rb : kOut;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{f.x ^ v[2 * j].y, f.y ^ v[2 * j + 1].z}, cd, vc, (uint32_t)j * (me / 2), kNt);
  __syncthreads();
  // rowwise data: granule tid % 8 of rows tid / 8 + 32 * it
  const rsrc_t rd = make_rsrc(row_data + (int64_t)row0 * (k / 2) + col_base / 2);
  const uint32_t g = tid & 7;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint32_t row = 32 * it + (tid >> 3);
    const uint32_t off = 32 * g + 32 <= ncols ? row * (ku / 2) + 16 * g : kOut;
    __builtin_amdgcn_raw_buffer_store_b128(f ^ v[4 * it], rd, off, 0, 0);
  }
  if (tid < 128 && ncols == 256)
    *reinterpret_cast<u32x4*>(row_scale + ((int64_t)row0 + tid) * (k / 16) + col_base / 16) = f ^ v[15];
  if ((uint32_t)tid < ncols)
    *reinterpret_cast<u32x2*>(col_scale + k * (int64_t)rbeg / 16 + (col_base + tid) * (int64_t)(me / 16) +
                              (row0 - rbeg) / 16) = u32x2{f.z, f.w};
}

int status() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

// nbytes: a positive multiple of 32 KB (one work-group iteration); grid > 0.
int hbm_probe_read(const void* src, int64_t nbytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || nbytes <= 0 || nbytes % kChunk || grid <= 0) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src,
                     (uint64_t)nbytes / kChunk, sink);
  return status();
}

int hbm_probe_fill(void* dst, int64_t nbytes, int grid, void* stream) {
  if (!dst || nbytes <= 0 || nbytes % kChunk || grid <= 0) return -1;
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint8_t*)dst,
                     (uint64_t)nbytes / kChunk);
  return status();
}

int hbm_probe_copy(const void* src, void* dst, int64_t nbytes, int grid, void* stream) {
  if (!src || !dst || nbytes <= 0 || nbytes % kChunk || grid <= 0) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src,
                     (uint8_t*)dst, (uint64_t)nbytes / kChunk);
  return status();
}

// Reads read_bytes (a multiple of 64 KB) of src and writes
// read_bytes / 16 * w4k bytes to dst (w4k = 4-KB units per 64 KB read, one of
// 4, 8, 9, 16); dst must hold that many bytes.
int hbm_probe_mix(const void* src, void* dst, int64_t read_bytes, int w4k, void* stream) {
  if (!src || !dst || read_bytes <= 0 || read_bytes % 65536) return -1;
  const unsigned n = (unsigned)(read_bytes / 65536);
  hipStream_t st = (hipStream_t)stream;
  switch (w4k) {
    case 4: hipLaunchKernelGGL((mix_kernel<4>), dim3(n), dim3(256), 0, st, (const uint8_t*)src, (uint8_t*)dst); break;
    case 8: hipLaunchKernelGGL((mix_kernel<8>), dim3(n), dim3(256), 0, st, (const uint8_t*)src, (uint8_t*)dst); break;
    case 9: hipLaunchKernelGGL((mix_kernel<9>), dim3(n), dim3(256), 0, st, (const uint8_t*)src, (uint8_t*)dst); break;
    case 16: hipLaunchKernelGGL((mix_kernel<16>), dim3(n), dim3(256), 0, st, (const uint8_t*)src, (uint8_t*)dst); break;
    default: return -1;
  }
  return status();
}

// The grouped cast's loads and stores on the buffers of nvfp4_group_cast
// (both directions), host splits as there.  k: a positive multiple of 256.
int hbm_probe_cast_pattern(const uint16_t* x, int64_t sum_m, int64_t k, int32_t num_experts, const int64_t* h_splits,
                           uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data, uint8_t* col_scale,
                           void* stream) {
  if (!x || !h_splits || !row_data || !row_scale || !col_data || !col_scale) return -1;
  if (k <= 0 || k % 256 || k > (1 << 22) || sum_m <= 0 || sum_m % 128 || sum_m > (1 << 24)) return -1;
  if (num_experts < 1 || num_experts > kMaxExperts) return -1;
  Splits S;
  S.n = num_experts;
  int64_t acc = 0;
  for (int e = 0; e < num_experts; ++e) {
    if (h_splits[e] < 0 || h_splits[e] % 128) return -1;
    acc += h_splits[e];
    S.end[e] = (int32_t)acc;
  }
  if (acc != sum_m) return -1;
  const uint32_t nrt = (uint32_t)(sum_m / 128);
  hipLaunchKernelGGL(cast_pattern_kernel, dim3(nrt * (unsigned)(k / 256)), dim3(256), 0, (hipStream_t)stream, x, k,
                     S, nrt, row_data, row_scale, col_data, col_scale);
  return status();
}

}  // extern "C"
