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
//  * Work-group tile 128 (i) x 256 (j); 4 wave64s in a 2 x 2 grid, each
//    computing 64 x 128 with 2 x 4 v_mfma_f32_32x32x16_f16 (128 fp32
//    accumulators per lane), two work-groups per CU so one's barrier and
//    LDS phase overlaps the other's MFMAs; the contraction advances 128
//    elements per step.
//  * LDS holds the raw FP4 bytes of the step's A and B lines (double-buffered;
//    the next step is copied by direct global -> LDS loads while the current
//    one is multiplied) and, apart, the E4M3 scale bytes of four steps at a
//    time (32 bytes per line, 16 per lane, double-buffered): copied per step
//    (8 bytes per line, 4 per lane) the scales took a third of the copy
//    instructions for a ninth of the bytes.  Each wave decodes its own
//    fragments one sub-step ahead of the MFMAs, interleaved with them
//    (one MFMA to six VALU instructions): v_cvt_scalef32_pk_f16_fp4 with unit
//    scale gives the exact E2M1 values two at a time, one packed fp16
//    multiply applies value(S) (converted once per block pair by
//    v_cvt_scalef32_pk_f16_fp8).
//  * Global loads are buffer loads: lines beyond an operand read as zero.
//    The 16-byte granules of a line are XOR-swizzled in LDS so that a
//    fragment read (32 consecutive lines, same granule) spreads over the
//    banks.
//  * Tile order: groups of 8 row tiles sweep the column tiles together, and
//    super-tiles of 64 tiles are dealt round-robin to the 8 XCDs, so each XCD
//    shares operand slices through its L2 and the XCDs share the work evenly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/nvfp4_group.h"
#include "nvfp4_common.hpp"
#include "nvfp4_numerics.hpp"

namespace {

using namespace nvfp4g;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWavesM = 2, kWavesN = 2;  // wave grid of a work-group
constexpr int kWM = 2, kWN = 4;          // 32 x 32 MFMA tiles per wave (i, j)
constexpr int kBM = kWavesM * kWM * 32;  // tile rows (i): 128
constexpr int kBN = kWavesN * kWN * 32;  // tile columns (j): 256
static_assert(kBM == 128, "row tiles must be the 128-row expert granule");
static_assert(kBN % kThreads == 0, "each thread copies whole B lines");
constexpr int kBK = 128;            // contraction step
constexpr int kGroupRows = 8;       // row tiles per column sweep

// One NT operand tile: `rows` lines of length L starting at the tile's first
// line; lines at or beyond `valid` read as zero.
struct OperandTile {
  const uint8_t* data;   // first line's codes; line pitch L/2 bytes
  const uint8_t* scale;  // first line's scales; line pitch L/16 bytes
  uint32_t valid;        // lines that exist
};

// Logical tile of this work-group.  Work-group i runs on XCD i % 8 (each
// XCD has its own L2).  Super-tiles of 64 consecutive logical tiles are dealt
// round-robin to the XCDs, so each XCD works through whole super-tiles
// (whose operand slices its L2 shares) and the XCDs share the work evenly
// even when tiles differ in cost (the weight-gradient tiles of a large expert
// are longer).  Work-groups past the last full round keep their index.
__device__ __forceinline__ uint32_t xcd_supertile_id() {
  const uint32_t id = blockIdx.x, T = gridDim.x;
  const uint32_t round = kNumXcd * 64, full = (T / round) * round;
  if (id >= full) return uni(id);
  const uint32_t j = id / kNumXcd, x = id % kNumXcd;
  return uni((kNumXcd * (j / 64) + x) * 64 + j % 64);
}

// Grouped order inside `ntm` x `ntn` tiles: groups of kGroupRows row tiles
// walk the column tiles together.
__device__ __forceinline__ void grouped_tile(uint32_t t, uint32_t ntm, uint32_t ntn, uint32_t* tm, uint32_t* tn) {
  const uint32_t g = t / (kGroupRows * ntn), in = t % (kGroupRows * ntn);
  const uint32_t first = g * kGroupRows, gm = min((uint32_t)kGroupRows, ntm - first);
  *tm = uni(first + in % gm);
  *tn = uni(in / gm);
}

// LDS stage: the raw FP4 bytes of one contraction step, [line][64 bytes] for
// A, then for B.
constexpr uint32_t kRowBytes = kBK / 2, kRowScales = kBK / 16;
constexpr uint32_t kStA = 0, kStB = kBM * kRowBytes;
constexpr uint32_t kStageBytes = kStB + kBN * kRowBytes;  // 24 KB
// Scale block: the E4M3 scale bytes of kScSteps consecutive steps, 32 bytes
// per line ([line][32] for A, then for B), double-buffered apart from the
// code stages.  Block b holds steps 4b .. 4b+3; a line's piece of the last
// block may run past the line's scales when the step count is not a multiple
// of 4: those bytes are the next line's (or read as zero past the operand,
// buffer loads being range-checked per dword) and are never used.
constexpr uint32_t kScSteps = 4, kScLine = kScSteps * kRowScales;
constexpr uint32_t kScA = 0, kScB = kBM * kScLine, kScBlockBytes = kScB + kBN * kScLine;  // 12 KB
// copies per thread (direct global -> LDS loads, 16 bytes each): code
// granules of A and B per stage, scale halves of A and B per scale block
constexpr int kCpA = kBM * kRowBytes / 16 / kThreads, kCpB = kBN * kRowBytes / 16 / kThreads;
constexpr int kCpAS = kBM * kScLine / 16 / kThreads, kCpBS = kBN * kScLine / 16 / kThreads;
static_assert(kCpA * 16 * kThreads == kBM * kRowBytes && kCpB * 16 * kThreads == kBN * kRowBytes &&
              kCpAS * 16 * kThreads == kBM * kScLine && kCpBS * 16 * kThreads == kBN * kScLine,
              "every thread issues the same copies");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS slot of 16-byte granule q (0..3) of a line's 64-byte step chunk.  A
// fragment read has lanes 0-31 on 32 consecutive lines at the same granule;
// XOR-ing the granule with bits 2-3 of the line spreads lines r, r+4, r+8,
// r+12 over different banks (an involution: the copy fetches granule
// swz(line, slot) into each slot, the reader finds granule q at slot
// swz(line, q)).
__device__ __forceinline__ uint32_t swz(uint32_t line, uint32_t q) { return q ^ ((line >> 2) & 3u); }

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (and nothing else).
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Two E4M3 codes (low byte first) -> their fp16 values (exact: the fp8
// convert with unit scale).
__device__ __forceinline__ h2_t scales_h2(uint32_t two_codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_codes, 1.0f, false);
}

// One MFMA operand fragment: the 8 codes of `w` (element 2j in the low
// nibble of byte j) times value(S), as 8 fp16.
__device__ __forceinline__ h8_t decode8(uint32_t w, _Float16 S) {
  const h2_t ss = {S, S};
  const h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return h8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// acc[im][in] += A[lines of the wave] x B[lines of the wave]^T over the
// contraction length L (a multiple of kBK).
//
// Contraction order: the MFMA's 16 k-slots of sub-step s (0..7) are, for
// lanes 0-31 (h = 0) and 32-63 (h = 1), the 8 elements of 4-byte word
// 8h + s of the line's 64-byte step chunk.  A and B use the same
// assignment, so the sum is unchanged; each lane reads its words of all
// eight sub-steps with two 16-byte LDS reads and the four block scales it
// needs (blocks 4h .. 4h+3) with one 4-byte read.
//
// Pipeline (double-buffered LDS, the two stages in separate arrays): each
// step starts with the wave waiting for its own copies of the step (issued
// one step earlier) and a work-group barrier, so the step is complete in LDS
// and the other stage is no longer being read; every wave then issues the
// direct global -> LDS copies of the next step into the other stage, reads
// all its fragments of the step and multiplies while the copies are in
// flight.  The loop is unrolled by two so that every copy and every read
// names its stage array: the compiler can then tell that a read of one stage
// need not wait for copies into the other (with one array and a computed
// offset it makes every LDS read wait for every copy in flight).  The scale
// blocks share one array, so each step reads its scales before it issues
// any copy: no copy into that array is then in flight (the step's wait has
// drained them), and the read of block b and the copy of block b + 1 (issued
// by the last step of block b, into the other half) never overlap.
__device__ __forceinline__ void gemm_tile(const OperandTile& A, const OperandTile& B, uint32_t L,
                                          f32x16 (&acc)[kWM][kWN], uint8_t* lds0, uint8_t* lds1,
                                          uint8_t* lsc) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // every descriptor field is work-group uniform: keep them in scalar registers
  const uint32_t dpitch = uni(L / 2), spitch = uni(L / 16);
  const uint32_t av = uni(A.valid), bv = uni(B.valid);
  auto rsrc = [](const uint8_t* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(uni(reinterpret_cast<int64_t>(p))), 0, bytes, 0x00020000);
  };
  const rsrc_t ad = rsrc(A.data, av * dpitch), as = rsrc(A.scale, av * spitch);
  const rsrc_t bd = rsrc(B.data, bv * dpitch), bs = rsrc(B.scale, bv * spitch);
  const uint32_t nk = L / kBK;
  if (nk == 0) return;

  // Copy the codes of step ks into a stage.  Copy c of a thread moves
  // granule g = c * kThreads + tid; a wave's lanes land contiguously in LDS.
  auto issue = [&](uint32_t ks, uint8_t* base) {
    const uint32_t sd = ks * kRowBytes;
#pragma unroll
    for (int c = 0; c < kCpA; ++c) {
      const uint32_t g = c * kThreads + tid;  // LDS slot g % 4 of line g / 4
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ad, (lds_ptr_t)(base + kStA + 16 * (c * kThreads + wave * 64)), 16,
                                               (g >> 2) * dpitch + 16 * swz(g >> 2, g & 3), sd, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kCpB; ++c) {
      const uint32_t g = c * kThreads + tid;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bd, (lds_ptr_t)(base + kStB + 16 * (c * kThreads + wave * 64)), 16,
                                               (g >> 2) * dpitch + 16 * swz(g >> 2, g & 3), sd, 0, 0);
    }
  };
  // Copy the scales of steps kScSteps * blk .. + kScSteps - 1 into a scale
  // block: lane g moves 16-byte half g % 2 of line g / 2's 32-byte piece.
  auto issue_scales = [&](uint32_t blk, uint8_t* sbase) {
    const uint32_t so = blk * kScLine;
#pragma unroll
    for (int c = 0; c < kCpAS; ++c) {
      const uint32_t g = c * kThreads + tid;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(as, (lds_ptr_t)(sbase + kScA + 16 * (c * kThreads + wave * 64)), 16,
                                               (g >> 1) * spitch + 16 * (g & 1), so, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kCpBS; ++c) {
      const uint32_t g = c * kThreads + tid;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bs, (lds_ptr_t)(sbase + kScB + 16 * (c * kThreads + wave * 64)), 16,
                                               (g >> 1) * spitch + 16 * (g & 1), so, 0, 0);
    }
  };

  const int wm = wave / kWavesN, wn = wave % kWavesN, h = lane >> 5;
  auto step = [&](uint32_t ks, const uint8_t* base, uint8_t* next) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies of step ks
    __syncthreads();
    // scales first (see above), two E4M3 codes -> fp16 pairs per line
    h2_t sa[kWM][2], sb[kWN][2];
    const uint8_t* scb = lsc + ((ks / kScSteps) & 1) * kScBlockBytes + kRowScales * (ks % kScSteps) + 4 * h;
#pragma unroll
    for (int im = 0; im < kWM; ++im) {
      const uint32_t line = wm * (kWM * 32) + im * 32 + (lane & 31);
      const uint32_t sc = *reinterpret_cast<const uint32_t*>(scb + kScA + kScLine * line);
      sa[im][0] = scales_h2(sc & 0xFFFFu);
      sa[im][1] = scales_h2(sc >> 16);
    }
#pragma unroll
    for (int in = 0; in < kWN; ++in) {
      const uint32_t line = wn * (kWN * 32) + in * 32 + (lane & 31);
      const uint32_t sc = *reinterpret_cast<const uint32_t*>(scb + kScB + kScLine * line);
      sb[in][0] = scales_h2(sc & 0xFFFFu);
      sb[in][1] = scales_h2(sc >> 16);
    }
    if (ks + 1 < nk) {
      issue(ks + 1, next);
      const uint32_t nb = (ks + 1) / kScSteps;
      if ((ks + 1) % kScSteps == 0) issue_scales(nb, lsc + (nb & 1) * kScBlockBytes);
    }
    u32x4 wa[kWM][2], wb[kWN][2];
#pragma unroll
    for (int im = 0; im < kWM; ++im) {
      const uint32_t line = wm * (kWM * 32) + im * 32 + (lane & 31);
      wa[im][0] = *reinterpret_cast<const u32x4*>(base + kStA + kRowBytes * line + 16 * swz(line, 2 * h));
      wa[im][1] = *reinterpret_cast<const u32x4*>(base + kStA + kRowBytes * line + 16 * swz(line, 2 * h + 1));
    }
#pragma unroll
    for (int in = 0; in < kWN; ++in) {
      const uint32_t line = wn * (kWN * 32) + in * 32 + (lane & 31);
      wb[in][0] = *reinterpret_cast<const u32x4*>(base + kStB + kRowBytes * line + 16 * swz(line, 2 * h));
      wb[in][1] = *reinterpret_cast<const u32x4*>(base + kStB + kRowBytes * line + 16 * swz(line, 2 * h + 1));
    }
    // Sub-step s+1's fragments are decoded while sub-step s's MFMAs run, and
    // the scheduler is told to alternate one MFMA with six VALU instructions
    // (the decode is 48 per sub-step for 8 MFMAs), so each wave keeps its own
    // matrix core busy during its decode instead of leaving that to the other
    // wave on the SIMD.
    h8_t af[2][kWM], bf[2][kWN];
#pragma unroll
    for (int im = 0; im < kWM; ++im) af[0][im] = decode8(wa[im][0][0], sa[im][0][0]);
#pragma unroll
    for (int in = 0; in < kWN; ++in) bf[0][in] = decode8(wb[in][0][0], sb[in][0][0]);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int cu = s & 1, nx = cu ^ 1, t = s + 1;
      if (t < kBK / 16) {
#pragma unroll
        for (int im = 0; im < kWM; ++im) af[nx][im] = decode8(wa[im][t >> 2][t & 3], sa[im][t >> 2][(t >> 1) & 1]);
#pragma unroll
        for (int in = 0; in < kWN; ++in) bf[nx][in] = decode8(wb[in][t >> 2][t & 3], sb[in][t >> 2][(t >> 1) & 1]);
      }
#pragma unroll
      for (int im = 0; im < kWM; ++im)
#pragma unroll
        for (int in = 0; in < kWN; ++in)
          acc[im][in] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cu][im], bf[cu][in], acc[im][in], 0, 0, 0);
      if (t < kBK / 16) {
#pragma unroll
        for (int i = 0; i < kWM * kWN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
        }
      }
    }
  };
  issue(0, lds0);
  issue_scales(0, lsc);
#pragma unroll 1
  for (uint32_t ks = 0; ks < nk; ks += 2) {
    step(ks, lds0, lds1);
    if (ks + 1 >= nk) break;
    step(ks + 1, lds1, lds0);
  }
  // the stages are reused by the epilogue's staging only after every wave is done
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
}

// out[i, j] = (acc * sa[i]) * sb[j] for i < rows_i, j < rows_j; the line
// scales of the tile are staged in LDS first.  The fp32 output is written
// with streaming stores (the weight gradient's [E, N, K] output is 1.9 GB at
// the expert-share shapes: 1881 -> 1833 us).
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[kWM][kWN], const float* a_amax, uint32_t rows_i,
                                         const float* b_amax, uint32_t rows_j, float* out, int64_t ldo,
                                         float* lsa, float* lsb) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < kBM) lsa[tid] = (uint32_t)tid < rows_i ? a_amax[tid] / 2688.0f : 0.0f;
#pragma unroll
  for (int c = 0; c < kBN / kThreads; ++c) {
    const uint32_t j = tid + kThreads * c;
    lsb[j] = j < rows_j ? b_amax[j] / 2688.0f : 0.0f;
  }
  __syncthreads();
  const int wm = wave / kWavesN, wn = wave % kWavesN;
#pragma unroll
  for (int in = 0; in < kWN; ++in) {
    const uint32_t j = wn * (kWN * 32) + in * 32 + (lane & 31);
    const float sb = lsb[j];
#pragma unroll
    for (int im = 0; im < kWM; ++im)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t i = wm * (kWM * 32) + im * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (i < rows_i && j < rows_j)  // streaming store: the output is not read again here
          __builtin_nontemporal_store((acc[im][in][v] * lsa[i]) * sb, &out[(int64_t)i * ldo + j]);
      }
  }
}

// Forward form: expert e's rows of a times b_e^T.  Tiles: 128-row tiles of
// the routed rows (each inside one expert) x 256-column tiles of n.
__global__ __launch_bounds__(kThreads, 2) void gemm_fwd_kernel(
    const uint8_t* __restrict__ a_data, const uint8_t* __restrict__ a_scale, const float* __restrict__ a_amax,
    const uint8_t* __restrict__ b_data, const uint8_t* __restrict__ b_scale, const float* __restrict__ b_amax,
    int64_t n, int64_t k, Routing R, uint32_t ntm, uint32_t ntn, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[2 * kScBlockBytes];
  __shared__ float lsa[kBM], lsb[kBN];
  if (!routing_ok(R)) return;
  const int32_t total = route_end(R, R.num_experts - 1);
  uint32_t tm, tn;
  grouped_tile(xcd_supertile_id(), ntm, ntn, &tm, &tn);
  const int32_t row0 = (int32_t)(tm * kBM);
  if (row0 >= total) return;
  int32_t rbeg, rend;
  const int e = find_expert(R, row0, &rbeg, &rend);
  const int64_t col0 = (int64_t)tn * kBN;
  const uint32_t cols = (uint32_t)min<int64_t>(n - col0, kBN);
  const int64_t brow0 = (int64_t)e * n + col0;  // first line of b in this tile
  const OperandTile A{a_data + (int64_t)row0 * (k / 2), a_scale + (int64_t)row0 * (k / 16), (uint32_t)kBM};
  const OperandTile B{b_data + brow0 * (k / 2), b_scale + brow0 * (k / 16), cols};
  f32x16 acc[kWM][kWN];
#pragma unroll
  for (int im = 0; im < kWM; ++im)
#pragma unroll
    for (int in = 0; in < kWN; ++in) acc[im][in] = f32x16{};
  gemm_tile(A, B, (uint32_t)k, acc, lds0, lds1, lsc);
  epilogue(acc, a_amax + row0, kBM, b_amax + brow0, cols, out + (int64_t)row0 * n + col0, n, lsa, lsb);
}

// Expert order of the weight-gradient tiles: the experts with the most rows
// (the longest contractions) first, so the long tiles do not form the tail.
struct ExpertOrder {
  uint16_t e[NVFP4G_MAX_EXPERTS_HOST];
};

// Weight-gradient form: for expert e, out_e[i, j] = sum over its rows r of
// xa_e[i, r] * xb_e[j, r], with a and b columnwise cast outputs (expert e's
// lines at byte n*r_e/2 resp. k*r_e/2, line length M_e).  Tiles: per expert,
// 128-line tiles of a x 256-line tiles of b.
__global__ __launch_bounds__(kThreads, 2) void gemm_wgrad_kernel(
    const uint8_t* __restrict__ a_data, const uint8_t* __restrict__ a_scale, const float* __restrict__ a_amax,
    const uint8_t* __restrict__ b_data, const uint8_t* __restrict__ b_scale, const float* __restrict__ b_amax,
    int64_t n, int64_t k, Routing R, ExpertOrder order, bool ordered, uint32_t ntm, uint32_t ntn,
    float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lsc[2 * kScBlockBytes];
  __shared__ float lsa[kBM], lsb[kBN];
  if (!routing_ok(R)) return;
  const uint32_t t = xcd_supertile_id(), per = ntm * ntn;
  const int e = (int)uni(ordered ? (uint32_t)order.e[t / per] : t / per);
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
  f32x16 acc[kWM][kWN];
#pragma unroll
  for (int im = 0; im < kWM; ++im)
#pragma unroll
    for (int in = 0; in < kWN; ++in) acc[im][in] = f32x16{};
  gemm_tile(A, B, me, acc, lds0, lds1, lsc);
  epilogue(acc, a_amax + (int64_t)e * n + i0, rows_i, b_amax + (int64_t)e * k + j0, rows_j,
           out + (int64_t)e * n * k + i0 * k + j0, k, lsa, lsb);
}

// ------------------------------------------------------------- host side

constexpr int64_t kGemmMaxN = 1 << 20;
constexpr int64_t kGemmMaxExpertRows = 1 << 22;  // weight gradient: rows of one expert

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

int check_wgrad(int64_t rows, int64_t n, int64_t k, int32_t E) {
  if (n <= 0 || n % 16 != 0 || n > kGemmMaxN || k <= 0 || k % 16 != 0 || k > kGemmMaxN) return NVFP4G_EINVAL;
  if (rows < 0 || rows > kMaxRows || E < 1) return NVFP4G_EINVAL;
  const int64_t tiles = ((n + kBM - 1) / kBM) * ((k + kBN - 1) / kBN);
  if (tiles * E > (int64_t)INT32_MAX) return NVFP4G_EINVAL;
  return NVFP4G_OK;
}

int launch_wgrad(const uint8_t* ad, const uint8_t* as, const float* aa, const uint8_t* bd, const uint8_t* bs,
                 const float* ba, int64_t n, int64_t k, const Routing& R, const ExpertOrder& order, bool ordered,
                 float* out, hipStream_t st) {
  const uint32_t ntm = (uint32_t)((n + kBM - 1) / kBM), ntn = (uint32_t)((k + kBN - 1) / kBN);
  hipLaunchKernelGGL(gemm_wgrad_kernel, dim3(ntm * ntn * (uint32_t)R.num_experts), dim3(kThreads), 0, st, ad, as,
                     aa, bd, bs, ba, n, k, R, order, ordered, ntm, ntn, out);
  return hip_status();
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
  int rc = check_wgrad(sum_m, n, k, num_experts);
  if (rc) return rc;
  if ((rc = check_gemm_ptrs(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, out))) return rc;
  Routing R;
  R.num_experts = num_experts;
  R.m_capacity = (int32_t)sum_m;
  R.d_offs = nullptr;
  R.d_status = nullptr;
  if ((rc = host_routing(h_splits, sum_m, num_experts, &R))) return rc;
  // a work-group's operand lines are addressed with 32-bit byte offsets
  for (int32_t e = 0; e < num_experts; ++e)
    if (h_splits[e] > kGemmMaxExpertRows) return NVFP4G_EINVAL;
  ExpertOrder order;
  for (int32_t e = 0; e < num_experts; ++e) order.e[e] = (uint16_t)e;
  std::stable_sort(order.e, order.e + num_experts,
                   [&](uint16_t a, uint16_t b) { return h_splits[a] > h_splits[b]; });
  return launch_wgrad(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, n, k, R, order,
                      true, out, (hipStream_t)stream);
}

int nvfp4_group_gemm_wgrad_graphsafe(const uint8_t* a_col_data, const uint8_t* a_col_scale,
                                     const float* a_col_amax, const uint8_t* b_col_data,
                                     const uint8_t* b_col_scale, const float* b_col_amax, int64_t m_capacity,
                                     int64_t n, int64_t k, int32_t num_experts, const int32_t* d_offs, float* out,
                                     int32_t* d_status, void* stream) {
  int rc = check_wgrad(m_capacity, n, k, num_experts);
  if (rc) return rc;
  // the routing is only known on the device: bound every expert by the capacity
  if (m_capacity > kGemmMaxExpertRows) return NVFP4G_EINVAL;
  if ((rc = check_gemm_ptrs(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, out))) return rc;
  Routing R;
  R.num_experts = num_experts;
  R.m_capacity = (int32_t)m_capacity;
  if ((rc = graph_routing(d_offs, d_status, num_experts, m_capacity, &R))) return rc;
  ExpertOrder order;  // unused: experts in index order
  return launch_wgrad(a_col_data, a_col_scale, a_col_amax, b_col_data, b_col_scale, b_col_amax, n, k, R, order,
                      false, out, (hipStream_t)stream);
}

}  // extern "C"
