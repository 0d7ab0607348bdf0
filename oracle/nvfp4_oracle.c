/*
 * nvfp4_oracle.c -- CPU oracle for the grouped, row-scaled (per-token) NVFP4
 * amax + cast of packed MoE activations.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU path must compute, used by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg.  Nothing on the
 * product path may link, load or call it, and it shares no code, header,
 * table or helper with the HIP library.  It is compiled with
 * `gcc -O2 -ffp-contract=off` (no -ffast-math, no FMA contraction), so every
 * float expression below is exactly one IEEE-754 binary32 operation with
 * round-to-nearest-even, as written.
 *
 * Sources (the pages this follows; cited by page title and section):
 *  - the TransformerEngine issue 3649 page (single-launch grouped
 *    row-scaled NVFP4 cast), Description: a grouped amax over the packed (sum_M, K)
 *    buffer yields a rowwise [sum_M] and a columnwise [num_tensors*K] amax,
 *    then a grouped cast consumes them; a graph-safe twin reads the routing
 *    from device offsets and is byte-identical.
 *  - "Implement per-token NVFP4 fprop recipe" (TransformerEngine PR 2931),
 *    Description and Important Files Changed: one amax per row replaces the
 *    per-tensor amax; FP4 data with FP8 (E4M3) block scales; the dequant
 *    looks the amax up by row index.
 *  - "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
 *    GroupedLinear" (TransformerEngine PR 3324), Greptile Summary: the
 *    columnwise (transposed) operand carries a per-column amax.
 *  - the TransformerEngine PR 3824 page (CustomRecipe for grouped GEMM and
 *    the MXFP4 reference quantizer), Changes item 2: a 0-element split must
 *    not fail.
 *
 * The numerics (the pages print no formula; this is the project's fixed
 * reading, stated once here and in the design notes):
 *   line scale        s = A / (6 * 448)            (A = the line's amax)
 *   block decode      t = (b / 6) / s              (b = the block's amax)
 *                     S = E4M3FN(t), round to nearest, ties to even,
 *                         saturating at 448
 *                     d = value(S) * s
 *                     m = 1 / d  (0 when d == 0; clamped to FLT_MAX)
 *   element           v = x * m,  code = sign(v) | E2M1(|v|), nearest with
 *                         ties to the even code, saturating at 6
 *   dequant           x^ = (value(code) * value(S)) * (A / (6 * 448))
 * A "line" is a row of X (rowwise) or one column of one expert's rows
 * (columnwise); blocks are 16 consecutive elements of a line.
 *
 * Further sections below: the MXFP4 sibling cast (OCP MX scale rule), the
 * four-over-six block scaling (a reading of the recipe the torchtitan
 * converter page names; the selection rule comes from the published method
 * of that name, so its agreement with that method's own code is not
 * pinned), and the per-tensor amax for casts with row scaling off.
 *
 * Parity pins: every function here is pinned by the CPU tests (exhaustive
 * and special-case checks of the two conversions against their definitions
 * and against torch's float8_e4m3fn cast, closed-form round trips, an
 * independent numpy brute force, grouped == per-expert loop, the half-gap
 * error bound, hand-worked golden rows, and mutations of the oracle that the
 * pins must catch).  No function is left unpinned against its own
 * definition.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* FP4 (E2M1) and FP8 (E4M3) maxima; their product is the line-scale divisor. */
static const float kFp4Max = 6.0f;
static const float kE4m3Max = 448.0f;

/* ---------------------------------------------------------------- widening */

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
static float bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ------------------------------------------------------------- E4M3FN code */

/* Value of an E4M3FN code (sign 0): 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals when the exponent field is 0; code 0x7F is NaN and is
 * never produced here. */
double oracle_e4m3_value(int code) {
  int e = (code >> 3) & 15;
  int f = code & 7;
  if (e == 0) return ldexp((double)f, -9);          /* f/8 * 2^(1-7) */
  return ldexp(1.0 + f / 8.0, e - 7);
}

/* Nearest E4M3FN code to t >= 0, ties to the even code, saturating: any t at
 * or above the largest finite value 448 gives 0x7E.  Written as a scan over
 * the 127 non-negative finite codes so that it can be checked by eye. */
int oracle_e4m3_encode(float t) {
  if (!(t >= 0.0f)) return -1; /* negative or NaN: outside the contract */
  if (t >= kE4m3Max) return 0x7E;
  double td = (double)t;
  for (int c = 0; c < 0x7E; ++c) {
    double lo = oracle_e4m3_value(c), hi = oracle_e4m3_value(c + 1);
    if (td > hi) continue;
    double mid = 0.5 * (lo + hi); /* exact in double */
    if (td < mid) return c;
    if (td > mid) return c + 1;
    return (c % 2 == 0) ? c : c + 1; /* tie: even code */
  }
  return 0x7E;
}

/* ------------------------------------------------------------- E2M1 code */

/* The eight non-negative E2M1 values, indexed by the 3-bit magnitude code. */
static const double kE2m1Grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(int code) {
  double v = kE2m1Grid[code & 7];
  return (code & 8) ? -v : v;
}

/* Magnitude code of the nearest E2M1 value to a >= 0, ties to the even code,
 * saturating: a >= 6 (including +inf) gives 7. */
int oracle_e2m1_encode_mag(float a) {
  if (!(a >= 0.0f)) return -1;
  if (a >= 6.0f) return 7;
  double ad = (double)a;
  for (int c = 0; c < 7; ++c) {
    double lo = kE2m1Grid[c], hi = kE2m1Grid[c + 1];
    if (ad > hi) continue;
    double mid = 0.5 * (lo + hi);
    if (ad < mid) return c;
    if (ad > mid) return c + 1;
    return (c % 2 == 0) ? c : c + 1;
  }
  return 7;
}

/* 4-bit code of v: sign bit of v in bit 3, magnitude code in bits 0..2. */
int oracle_e2m1_encode(float v) {
  int sign = signbit(v) ? 8 : 0;
  return sign | oracle_e2m1_encode_mag(fabsf(v));
}

/* ------------------------------------------------------------ line encode */

/* Line scale s = A / (6*448): the per-row (or per-column) scale that replaces
 * the per-tensor one. */
float oracle_line_scale(float amax) { return amax / (kFp4Max * kE4m3Max); }

/* Block step for block amax b on a line with scale s: returns the E4M3 code
 * and writes the element multiplier m = 1/d. */
int oracle_block_scale(float b, float s, float* m_out) {
  float t = (s == 0.0f) ? 0.0f : (b / kFp4Max) / s;
  int S = oracle_e4m3_encode(t);
  float d = (float)oracle_e4m3_value(S) * s;
  float m = 0.0f;
  if (d != 0.0f) m = fminf(1.0f / d, FLT_MAX);
  *m_out = m;
  return S;
}

/* Encode one line of n values (n a multiple of 16) with line amax A.
 * codes: n/2 bytes, element 2j in the low nibble of byte j, element 2j+1 in
 * the high nibble.  scales: n/16 E4M3 codes. */
int oracle_encode_line(const float* L, int64_t n, float A, uint8_t* codes,
                       uint8_t* scales) {
  if (n < 0 || n % 16 != 0) return ORACLE_EINVAL;
  float s = oracle_line_scale(A);
  for (int64_t j = 0; j < n / 16; ++j) {
    const float* blk = L + 16 * j;
    float b = 0.0f;
    for (int i = 0; i < 16; ++i) b = fmaxf(b, fabsf(blk[i]));
    float m;
    int S = oracle_block_scale(b, s, &m);
    scales[j] = (uint8_t)S;
    for (int i = 0; i < 16; i += 2) {
      int c0 = oracle_e2m1_encode(blk[i] * m);
      int c1 = oracle_e2m1_encode(blk[i + 1] * m);
      codes[8 * j + i / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
  return ORACLE_OK;
}

/* Dequantize one encoded line back to fp32 with the same A. */
int oracle_decode_line(const uint8_t* codes, const uint8_t* scales, int64_t n,
                       float A, float* out) {
  if (n < 0 || n % 16 != 0) return ORACLE_EINVAL;
  float s = oracle_line_scale(A);
  for (int64_t i = 0; i < n; ++i) {
    int byte = codes[i / 2];
    int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
    float q = (float)oracle_e2m1_value(code);
    float S = (float)oracle_e4m3_value(scales[i / 16]);
    out[i] = (q * S) * s;
  }
  return ORACLE_OK;
}

/* --------------------------------------------------------------- grouping */

/* Validate the host split list: E >= 1, splits >= 0, multiples of 128,
 * summing to sum_m; K a positive multiple of 16. */
static int check_args(int64_t sum_m, int64_t k, int32_t E,
                      const int64_t* splits) {
  if (E < 1 || k <= 0 || k % 16 != 0 || sum_m < 0 || splits == NULL)
    return ORACLE_EINVAL;
  int64_t tot = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (splits[e] < 0 || splits[e] % 128 != 0) return ORACLE_EINVAL;
    tot += splits[e];
  }
  return tot == sum_m ? ORACLE_OK : ORACLE_EINVAL;
}

/* Amax of one row of X (bf16, row-major with row length k). */
float oracle_row_amax(const uint16_t* x, int64_t k, int64_t r) {
  float a = 0.0f;
  for (int64_t c = 0; c < k; ++c) a = fmaxf(a, fabsf(bf16_value(x[r * k + c])));
  return a;
}

/* Amax of column c over rows [r0, r0 + m). */
float oracle_col_amax(const uint16_t* x, int64_t k, int64_t c, int64_t r0,
                      int64_t m) {
  float a = 0.0f;
  for (int64_t r = r0; r < r0 + m; ++r) a = fmaxf(a, fabsf(bf16_value(x[r * k + c])));
  return a;
}

/* Grouped amax: row_amax[r] over each row; col_amax[e*k + c] over the rows of
 * expert e (0 for an expert with no rows).  Either output may be NULL. */
int oracle_group_amax(const uint16_t* x, int64_t sum_m, int64_t k, int32_t E,
                      const int64_t* splits, float* row_amax, float* col_amax) {
  int rc = check_args(sum_m, k, E, splits);
  if (rc != ORACLE_OK) return rc;
  if (row_amax)
    for (int64_t r = 0; r < sum_m; ++r) row_amax[r] = oracle_row_amax(x, k, r);
  if (col_amax) {
    int64_t r0 = 0;
    for (int32_t e = 0; e < E; ++e) {
      for (int64_t c = 0; c < k; ++c)
        col_amax[(int64_t)e * k + c] = oracle_col_amax(x, k, c, r0, splits[e]);
      r0 += splits[e];
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------ per-tensor amax
 *
 * The row_scaled knob of the four-over-six converter page ("[NVFP4 4over6]
 * Add the grouped-experts four-over-six converter", Summary and Review pass)
 * switches the per-row amax off; the per-token page ("Implement per-token
 * NVFP4 fprop recipe", Description) describes the per-row amax as replacing
 * a per-tensor one.  Reading taken: with row scaling off, every line of an
 * expert takes the expert's tensor amax A_e = max |x| over all of its rows
 * and columns (each expert's slice is the tensor its GEMM sees), written as
 * the amax vectors the casts consume: row_amax[r] = A_e for every row r of
 * expert e and col_amax[e*k + c] = A_e for every column c; an expert with no
 * rows gets 0.  Either output may be NULL. */
int oracle_group_amax_tensor(const uint16_t* x, int64_t sum_m, int64_t k, int32_t E,
                             const int64_t* splits, float* row_amax, float* col_amax) {
  int rc = check_args(sum_m, k, E, splits);
  if (rc != ORACLE_OK) return rc;
  int64_t r0 = 0;
  for (int32_t e = 0; e < E; ++e) {
    float A = 0.0f;
    for (int64_t r = r0; r < r0 + splits[e]; ++r)
      for (int64_t c = 0; c < k; ++c) A = fmaxf(A, fabsf(bf16_value(x[r * k + c])));
    if (row_amax)
      for (int64_t r = r0; r < r0 + splits[e]; ++r) row_amax[r] = A;
    if (col_amax)
      for (int64_t c = 0; c < k; ++c) col_amax[(int64_t)e * k + c] = A;
    r0 += splits[e];
  }
  return ORACLE_OK;
}

/* Rowwise cast of row r: k/2 data bytes and k/16 scales. */
int oracle_cast_row(const uint16_t* x, int64_t k, int64_t r, float A,
                    uint8_t* data, uint8_t* scales) {
  float* L = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
  if (!L) return ORACLE_EINVAL;
  for (int64_t c = 0; c < k; ++c) L[c] = bf16_value(x[r * k + c]);
  int rc = oracle_encode_line(L, k, A, data, scales);
  free(L);
  return rc;
}

/* Columnwise cast of column c of the expert owning rows [r0, r0 + m):
 * m/2 data bytes and m/16 scales (one line of the transposed expert). */
int oracle_cast_col(const uint16_t* x, int64_t k, int64_t c, int64_t r0,
                    int64_t m, float A, uint8_t* data, uint8_t* scales) {
  float* L = (float*)malloc(sizeof(float) * (size_t)(m > 0 ? m : 1));
  if (!L) return ORACLE_EINVAL;
  for (int64_t r = 0; r < m; ++r) L[r] = bf16_value(x[(r0 + r) * k + c]);
  int rc = oracle_encode_line(L, m, A, data, scales);
  free(L);
  return rc;
}

/* Grouped cast.  Rowwise outputs: data [sum_m, k/2], scales [sum_m, k/16].
 * Columnwise outputs, expert e owning rows [r_e, r_e + M_e): data [k, M_e/2]
 * at byte k*r_e/2, scales [k, M_e/16] at byte k*r_e/16.  A direction is
 * produced when its data pointer is non-NULL (its scale pointer and amax must
 * then be non-NULL too). */
int oracle_group_cast(const uint16_t* x, int64_t sum_m, int64_t k, int32_t E,
                      const int64_t* splits, const float* row_amax,
                      const float* col_amax, uint8_t* row_data,
                      uint8_t* row_scale, uint8_t* col_data,
                      uint8_t* col_scale) {
  int rc = check_args(sum_m, k, E, splits);
  if (rc != ORACLE_OK) return rc;
  if (row_data) {
    if (!row_scale || !row_amax) return ORACLE_EINVAL;
    for (int64_t r = 0; r < sum_m; ++r) {
      rc = oracle_cast_row(x, k, r, row_amax[r], row_data + r * (k / 2),
                           row_scale + r * (k / 16));
      if (rc != ORACLE_OK) return rc;
    }
  }
  if (col_data) {
    if (!col_scale || !col_amax) return ORACLE_EINVAL;
    int64_t r0 = 0;
    for (int32_t e = 0; e < E; ++e) {
      int64_t m = splits[e];
      uint8_t* d = col_data + k * r0 / 2;
      uint8_t* sc = col_scale + k * r0 / 16;
      for (int64_t c = 0; c < k; ++c) {
        rc = oracle_cast_col(x, k, c, r0, m, col_amax[(int64_t)e * k + c],
                             d + c * (m / 2), sc + c * (m / 16));
        if (rc != ORACLE_OK) return rc;
      }
      r0 += m;
    }
  }
  return ORACLE_OK;
}

/* Batch helpers for the tests (plain loops over the scalar functions). */
void oracle_e4m3_encode_array(const float* t, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(t[i]);
}
void oracle_e2m1_encode_array(const float* v, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(v[i]);
}
void oracle_block_scale_array(const float* b, const float* s, int64_t n,
                              int32_t* S_out, float* m_out) {
  for (int64_t i = 0; i < n; ++i) S_out[i] = oracle_block_scale(b[i], s[i], &m_out[i]);
}

/* ------------------------------------------------------------------ MXFP4
 *
 * The MXFP4 sibling format named on the TransformerEngine PR 3824 page
 * (Changes item 1 and Testing: E2M1 elements, blocks of 32, E8M0
 * power-of-two scales, the "pow_2_scales" branch).  The page gives no scale
 * rule; the reading taken is the OCP Microscaling (MX) v1.0 definition: for
 * a block with amax A,
 *     shared = floor(log2(A)) - 2      (2 = exponent of FP4's largest value, 6 = 1.5 * 2^2)
 *              clamped to [-127, 127]; -127 when A == 0
 *     scale byte (E8M0) = shared + 127
 *     element code = E2M1(x / 2^shared), nearest, ties to the even code,
 *                    saturating at 6, sign of x kept.
 * No amax pass and no line scale: every 32-block is independent.  Rowwise
 * blocks run along the row, columnwise blocks along an expert's rows (the
 * same transposed layout as NVFP4, with 1/32 instead of 1/16 scales).
 */

/* E8M0 byte of a block with amax A >= 0 (finite). */
int oracle_mx_scale_byte(float A) {
  if (!(A >= 0.0f)) return -1;
  int shared = -127;
  if (A > 0.0f) {
    int ex;
    frexp((double)A, &ex); /* A = f * 2^ex, f in [0.5, 1): floor(log2 A) = ex - 1 */
    shared = ex - 1 - 2;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
  }
  return shared + 127;
}

/* Encode one line of n values (n a multiple of 32). */
int oracle_mx_encode_line(const float* L, int64_t n, uint8_t* codes, uint8_t* scales) {
  if (n < 0 || n % 32 != 0) return ORACLE_EINVAL;
  for (int64_t j = 0; j < n / 32; ++j) {
    const float* blk = L + 32 * j;
    float A = 0.0f;
    for (int i = 0; i < 32; ++i) A = fmaxf(A, fabsf(blk[i]));
    int byte = oracle_mx_scale_byte(A);
    scales[j] = (uint8_t)byte;
    double X = ldexp(1.0, byte - 127);
    for (int i = 0; i < 32; i += 2) {
      /* x / 2^shared is exact in double; as float it is exact for every
         |value| >= 2^-126, and smaller ones all encode to a signed zero */
      int c0 = oracle_e2m1_encode((float)((double)blk[i] / X));
      int c1 = oracle_e2m1_encode((float)((double)blk[i + 1] / X));
      codes[16 * j + i / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
  return ORACLE_OK;
}

/* Decode: value(code) * 2^(byte - 127), exact. */
int oracle_mx_decode_line(const uint8_t* codes, const uint8_t* scales, int64_t n, float* out) {
  if (n < 0 || n % 32 != 0) return ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    int byte = codes[i / 2];
    int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
    out[i] = (float)(oracle_e2m1_value(code) * ldexp(1.0, scales[i / 32] - 127));
  }
  return ORACLE_OK;
}

/* Grouped MXFP4 cast.  Rowwise: data [sum_m, k/2], scales [sum_m, k/32].
 * Columnwise, expert e owning rows [r_e, r_e + M_e): data [k, M_e/2] at
 * byte k*r_e/2, scales [k, M_e/32] at byte k*r_e/32.  k a multiple of 32;
 * a direction is produced when its data pointer is non-NULL. */
int oracle_mxfp4_group_cast(const uint16_t* x, int64_t sum_m, int64_t k, int32_t E,
                            const int64_t* splits, uint8_t* row_data, uint8_t* row_scale,
                            uint8_t* col_data, uint8_t* col_scale) {
  int rc = check_args(sum_m, k, E, splits);
  if (rc != ORACLE_OK || k % 32 != 0) return ORACLE_EINVAL;
  float* L = (float*)malloc(sizeof(float) * (size_t)((k > sum_m ? k : sum_m) + 1));
  if (!L) return ORACLE_EINVAL;
  if (row_data) {
    for (int64_t r = 0; r < sum_m && rc == ORACLE_OK; ++r) {
      for (int64_t c = 0; c < k; ++c) L[c] = bf16_value(x[r * k + c]);
      rc = oracle_mx_encode_line(L, k, row_data + r * (k / 2), row_scale + r * (k / 32));
    }
  }
  if (col_data && rc == ORACLE_OK) {
    int64_t r0 = 0;
    for (int32_t e = 0; e < E && rc == ORACLE_OK; ++e) {
      int64_t m = splits[e];
      for (int64_t c = 0; c < k && rc == ORACLE_OK; ++c) {
        for (int64_t r = 0; r < m; ++r) L[r] = bf16_value(x[(r0 + r) * k + c]);
        rc = oracle_mx_encode_line(L, m, col_data + k * r0 / 2 + c * (m / 2),
                                   col_scale + k * r0 / 32 + c * (m / 32));
      }
      r0 += m;
    }
  }
  free(L);
  return rc;
}

void oracle_mx_scale_byte_array(const float* A, int64_t n, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_mx_scale_byte(A[i]);
}

/* ---------------------------------------------------------- four over six
 *
 * Four-over-six block scaling, the NVFP4 recipe named on the torchtitan
 * converter page ("[NVFP4 4over6] Add the grouped-experts four-over-six
 * converter", Summary and Review pass: recipe "four_over_six" with the knobs
 * err_mode, e4m3_scale_bound and row_scaled).  The page gives no rule; the
 * reading taken follows the published method it is named after ("Four Over
 * Six: More Accurate NVFP4 Quantization with Adaptive Block Scaling"): each
 * 16-element block is encoded twice, once with its amax mapped to 6 (the
 * plain NVFP4 block step above) and once mapped to 4 (where the E2M1 grid is
 * finer relative to the block's largest values), and the encoding with the
 * smaller error is kept.  Steps, each one IEEE binary32 operation:
 *   line scale   s = A / (6 * Bnd)       Bnd = e4m3_scale_bound, 1 .. 448
 *   for k = 6, then k = 4:
 *     t_k = (b / k) / s  (0 when s == 0);  S_k = E4M3(t_k);  d_k = value(S_k) * s
 *     m_k = 1 / d_k (0 when d_k == 0, at most FLT_MAX);  c_i = E2M1(x_i * m_k)
 *     x^_i = (value(c_i) * value(S_k)) * s        (the dequant, first product exact)
 *     err_k = e_15 with e_{-1} = 0 and e_i = e_{i-1} + (x_i - x^_i)^2
 *             (err_mode 0, squared error), or + |x_i - x^_i| (err_mode 1)
 *   the block keeps k = 4 when err_4 < err_6, else k = 6.
 * row_scaled: the line scale is per row and per column of an expert, as
 * everywhere in this library.  With Bnd = 448 the k = 6 candidate is exactly
 * the plain block step.  A smaller Bnd leaves room for the k = 4 scale of the
 * line's largest block, (A/4)/s = 1.5 * Bnd, below E4M3's 448; the default
 * taken is 256, the largest power of two with 1.5 * Bnd <= 448.
 */

float oracle_line_scale_b(float amax, int bound) {
  return amax / (kFp4Max * (float)bound);
}

/* One candidate: scale code for divisor k, the 16 codes, and the error. */
static int cand_4o6(const float* blk, float b, float s, float k, int err_mode,
                    int* codes, float* err) {
  float t = (s == 0.0f) ? 0.0f : (b / k) / s;
  int S = oracle_e4m3_encode(t);
  float Sv = (float)oracle_e4m3_value(S);
  float d = Sv * s;
  float m = 0.0f;
  if (d != 0.0f) m = fminf(1.0f / d, FLT_MAX);
  float e = 0.0f;
  for (int i = 0; i < 16; ++i) {
    codes[i] = oracle_e2m1_encode(blk[i] * m);
    float q = (float)oracle_e2m1_value(codes[i]);
    float xh = (q * Sv) * s;
    float diff = blk[i] - xh;
    e = e + (err_mode == 0 ? diff * diff : fabsf(diff));
  }
  *err = e;
  return S;
}

/* Four-over-six step for one block of 16 values on a line with scale s:
 * writes the 16 codes, returns the scale code; *pick = 4 or 6; errs[0..1] =
 * the errors of the k = 6 and k = 4 candidates (either may be NULL). */
int oracle_block_4o6(const float* blk, float s, int err_mode, int* codes,
                     int* pick, float* errs) {
  float b = 0.0f;
  for (int i = 0; i < 16; ++i) b = fmaxf(b, fabsf(blk[i]));
  int c6[16], c4[16];
  float e6, e4;
  int S6 = cand_4o6(blk, b, s, 6.0f, err_mode, c6, &e6);
  int S4 = cand_4o6(blk, b, s, 4.0f, err_mode, c4, &e4);
  int use4 = e4 < e6;
  for (int i = 0; i < 16; ++i) codes[i] = use4 ? c4[i] : c6[i];
  if (pick) *pick = use4 ? 4 : 6;
  if (errs) { errs[0] = e6; errs[1] = e4; }
  return use4 ? S4 : S6;
}

static int check_4o6(int bound, int err_mode) {
  return (bound >= 1 && bound <= 448 && (err_mode == 0 || err_mode == 1)) ? ORACLE_OK : ORACLE_EINVAL;
}

/* Encode one line (n a multiple of 16) with line amax A; picks (n/16 bytes,
 * 4 or 6 per block) may be NULL. */
int oracle_encode_line_4o6(const float* L, int64_t n, float A, int bound,
                           int err_mode, uint8_t* codes, uint8_t* scales,
                           uint8_t* picks) {
  if (n < 0 || n % 16 != 0 || check_4o6(bound, err_mode)) return ORACLE_EINVAL;
  float s = oracle_line_scale_b(A, bound);
  for (int64_t j = 0; j < n / 16; ++j) {
    int c[16], pick;
    scales[j] = (uint8_t)oracle_block_4o6(L + 16 * j, s, err_mode, c, &pick, NULL);
    if (picks) picks[j] = (uint8_t)pick;
    for (int i = 0; i < 16; i += 2) codes[8 * j + i / 2] = (uint8_t)(c[i] | (c[i + 1] << 4));
  }
  return ORACLE_OK;
}

/* Dequantize a line encoded with line scale A / (6 * bound). */
int oracle_decode_line_b(const uint8_t* codes, const uint8_t* scales, int64_t n,
                         float A, int bound, float* out) {
  if (n < 0 || n % 16 != 0 || bound < 1 || bound > 448) return ORACLE_EINVAL;
  float s = oracle_line_scale_b(A, bound);
  for (int64_t i = 0; i < n; ++i) {
    int byte = codes[i / 2];
    int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
    float q = (float)oracle_e2m1_value(code);
    float S = (float)oracle_e4m3_value(scales[i / 16]);
    out[i] = (q * S) * s;
  }
  return ORACLE_OK;
}

/* Grouped four-over-six cast: the layouts, amax inputs and directions of
 * oracle_group_cast. */
int oracle_group_cast_4o6(const uint16_t* x, int64_t sum_m, int64_t k, int32_t E,
                          const int64_t* splits, const float* row_amax,
                          const float* col_amax, int bound, int err_mode,
                          uint8_t* row_data, uint8_t* row_scale,
                          uint8_t* col_data, uint8_t* col_scale) {
  int rc = check_args(sum_m, k, E, splits);
  if (rc != ORACLE_OK) return rc;
  if (check_4o6(bound, err_mode)) return ORACLE_EINVAL;
  int64_t cap = k > sum_m ? k : sum_m;
  float* L = (float*)malloc(sizeof(float) * (size_t)(cap > 0 ? cap : 1));
  if (!L) return ORACLE_EINVAL;
  if (row_data) {
    if (!row_scale || !row_amax) { free(L); return ORACLE_EINVAL; }
    for (int64_t r = 0; r < sum_m; ++r) {
      for (int64_t c = 0; c < k; ++c) L[c] = bf16_value(x[r * k + c]);
      oracle_encode_line_4o6(L, k, row_amax[r], bound, err_mode, row_data + r * (k / 2),
                             row_scale + r * (k / 16), NULL);
    }
  }
  if (col_data) {
    if (!col_scale || !col_amax) { free(L); return ORACLE_EINVAL; }
    int64_t r0 = 0;
    for (int32_t e = 0; e < E; ++e) {
      int64_t m = splits[e];
      for (int64_t c = 0; c < k; ++c) {
        for (int64_t r = 0; r < m; ++r) L[r] = bf16_value(x[(r0 + r) * k + c]);
        oracle_encode_line_4o6(L, m, col_amax[(int64_t)e * k + c], bound, err_mode,
                               col_data + k * r0 / 2 + c * (m / 2),
                               col_scale + k * r0 / 16 + c * (m / 16), NULL);
      }
      r0 += m;
    }
  }
  free(L);
  return ORACLE_OK;
}
