/*
 * nvfp4_group.h -- C ABI of libnvfp4g.so: grouped, row-scaled (per-token)
 * NVFP4 amax + cast of packed MoE expert activations/gradients on MI355X.
 *
 * What is computed (pages cited by title and section):
 *  - the TransformerEngine issue 3649 page (single-launch grouped
 *    row-scaled NVFP4 cast), Description: one grouped amax launch over the packed
 *    (sum_M, K) buffer produces a rowwise [sum_M] and a columnwise
 *    [num_experts * K] amax (both directions in one pass); one grouped cast
 *    launch consumes them; each has a graph-safe twin that reads the routing
 *    from device offsets instead of host split metadata, with the same device
 *    body, so the outputs of the two are byte-identical.
 *  - "Implement per-token NVFP4 fprop recipe" (TransformerEngine PR 2931),
 *    Description / Important Files Changed: one fp32 amax per row (token)
 *    replaces the per-tensor amax; data is FP4 (E2M1) with one FP8 (E4M3)
 *    scale per 16-element block; dequantisation looks up the amax by row.
 *  - "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
 *    GroupedLinear" (TransformerEngine PR 3324), Greptile Summary: the
 *    columnwise (transposed) operand is quantised with a per-column amax.
 *
 * Numerics, per line (a row of X, or one column of one expert's rows) with
 * amax A, and per 16-element block of the line with block amax b; every step
 * is one IEEE binary32 operation, round to nearest even, no FMA contraction,
 * denormals kept:
 *     s = A / 2688            (2688 = 6 * 448)
 *     t = (b / 6) / s         (0 when s == 0)
 *     S = E4M3FN(t)           nearest, ties to even, saturating at 448 (0x7E)
 *     d = value(S) * s
 *     m = 1 / d               (0 when d == 0, at most FLT_MAX)
 *     code = sign(x*m) << 3 | E2M1(|x*m|)   nearest on {0,.5,1,1.5,2,3,4,6},
 *                                           ties to the even code, saturating
 * x must be finite: a NaN or infinite element gives unspecified codes and
 * scales for its lines (no error is reported).
 *
 * Layouts (all row-major, unswizzled; expert e owns rows [r_e, r_e + M_e),
 * M_e a multiple of 128, experts packed in order):
 *     x          bf16 bits, [sum_m, k], contiguous, 16-byte aligned
 *     row_amax   fp32 [sum_m]
 *     col_amax   fp32 [E * k], expert-major (0 for an expert with no rows)
 *     row_data   u8 [sum_m, k/2]: element 2j in the low nibble of byte j
 *     row_scale  u8 [sum_m, k/16]: E4M3FN codes
 *     col_data   u8, per expert a [k, M_e/2] block (line c = column c of the
 *                expert, packed along its rows) at byte offset k*r_e/2
 *     col_scale  u8, per expert a [k, M_e/16] block at byte offset k*r_e/16
 *
 * Conventions: every pointer except h_splits is a device pointer owned by
 * the caller; `stream` is a hipStream_t (NULL = the default stream).  Calls
 * only enqueue work on `stream` and never synchronise, allocate or read
 * device memory on the host.  Arguments are checked on the host first and a
 * call that fails a check enqueues nothing and returns a negative status;
 * launch failures return NVFP4G_EHIP.  A direction is produced when its data
 * pointer is non-NULL (its scale pointer and amax must then be non-NULL).
 * The library keeps no state between calls: calls from several host threads,
 * on different streams and buffers, are independent of each other.
 */
#ifndef NVFP4_GROUP_H_
#define NVFP4_GROUP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4G_OK 0
#define NVFP4G_EINVAL (-1)  /* bad size, count, NULL pointer or direction */
#define NVFP4G_ESPLITS (-2) /* host splits negative, not %128, or sum != sum_m */
#define NVFP4G_EALIGN (-3)  /* x or an output not suitably aligned */
#define NVFP4G_EHIP (-4)    /* HIP launch/runtime error */

/* Size limits: K <= 2^22 columns and at most 2^24 rows (sum_m, or
 * m_capacity); larger calls return NVFP4G_EINVAL.  Largest expert count of
 * the host-split calls (the splits travel in the kernel arguments) and of the
 * graph-safe calls. */
#define NVFP4G_MAX_K (1 << 22)
#define NVFP4G_MAX_ROWS (1 << 24)
#define NVFP4G_MAX_EXPERTS_HOST 512
#define NVFP4G_MAX_EXPERTS_DEVICE 4096

/* Bits ORed into *d_status by the graph-safe calls when the device routing is
 * invalid; the library never clears them.  With any bit set the call writes
 * nothing else. */
#define NVFP4G_DEV_UNALIGNED 1 /* an expert's row count is not a multiple of 128 */
#define NVFP4G_DEV_NONMONO 2   /* offsets decrease (or the first is negative) */
#define NVFP4G_DEV_OVERFLOW 4  /* offs[E-1] > m_capacity */

/* Grouped amax (TransformerEngine issue 3649 page, single-launch grouped
 * row-scaled NVFP4 cast, Description).  x: [sum_m, k] bf16; h_splits: host array of E row counts
 * (each >= 0, a multiple of 128, summing to sum_m).  Writes
 * row_amax[r] = max_c |x[r, c]| and col_amax[e*k + c] = max over the rows of
 * expert e of |x[r, c]| (0 for an expert with no rows).  Either output may
 * be NULL to skip that direction.  k must be a positive multiple of 16. */
int nvfp4_group_amax(const uint16_t* x, int64_t sum_m, int64_t k,
                     int32_t num_experts, const int64_t* h_splits,
                     float* row_amax, float* col_amax, void* stream);

/* Grouped cast (same page, Description; per-token numerics from "Implement
 * per-token NVFP4 fprop recipe"; columnwise per-column amax from "Enable
 * NVFP4 row-scaled (per-token) backward for GroupedLinear").  Consumes the
 * amax vectors of nvfp4_group_amax and writes the rowwise and/or columnwise
 * FP4 data and E4M3 scales in the layouts above.  The bytes follow the
 * numerics above for amax vectors that nvfp4_group_amax wrote for the same
 * x and routing (each line's max |x|, a bf16 value): the block steps use
 * fast quotients that were checked against the IEEE divisions over exactly
 * such inputs.  Other amax values give finite output that may differ from
 * those numerics in a scale's last rounding. */
int nvfp4_group_cast(const uint16_t* x, int64_t sum_m, int64_t k,
                     int32_t num_experts, const int64_t* h_splits,
                     const float* row_amax, const float* col_amax,
                     uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                     uint8_t* col_scale, void* stream);

/* Graph-safe grouped amax (same page, Description: routing read from device
 * offsets so a captured graph replays under changed routing).  d_offs:
 * device int32[E], inclusive row ends (expert e owns rows
 * [offs[e-1], offs[e]), offs[-1] = 0).  m_capacity (a multiple of 128) sizes
 * the buffers: x and row_amax hold m_capacity rows; rows at or beyond
 * offs[E-1] are neither read nor written.  col_amax is fully written.  The
 * routing is checked on the device; if it is invalid, bits are ORed into
 * *d_status (a device int32 the caller zeroes) and nothing else is written.
 * Output bytes equal those of nvfp4_group_amax for the same routing. */
int nvfp4_group_amax_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k,
                               int32_t num_experts, const int32_t* d_offs,
                               float* row_amax, float* col_amax,
                               int32_t* d_status, void* stream);

/* Per-tensor amax, for casts with row scaling off: the row_scaled knob of
 * the four-over-six converter page ("[NVFP4 4over6] Add the grouped-experts
 * four-over-six converter", Summary and Review pass); the per-token page
 * ("Implement per-token NVFP4 fprop recipe", Description) describes the
 * per-row amax as replacing a per-tensor one.  Every line of expert e gets
 * the expert's tensor amax A_e = max |x| over all of its rows and columns:
 * row_amax[r] = A_e for each row r of expert e and col_amax[e*k + c] = A_e
 * (0 for an expert with no rows).  The vectors feed nvfp4_group_cast and
 * nvfp4_group_cast_4over6 unchanged, which then scale every line of an
 * expert alike.  Arguments as in nvfp4_group_amax; either output may be
 * NULL (at least one is needed for a result).  Runs the grouped amax and
 * one more launch (one work-group per expert). */
int nvfp4_group_amax_tensor(const uint16_t* x, int64_t sum_m, int64_t k,
                            int32_t num_experts, const int64_t* h_splits,
                            float* row_amax, float* col_amax, void* stream);

/* Graph-safe form of nvfp4_group_amax_tensor (routing, buffers and status as
 * in nvfp4_group_amax_graphsafe; rows at or beyond offs[E-1] are neither
 * read nor written).  Output equals nvfp4_group_amax_tensor's for the same
 * routing. */
int nvfp4_group_amax_tensor_graphsafe(const uint16_t* x, int64_t m_capacity,
                                      int64_t k, int32_t num_experts,
                                      const int32_t* d_offs, float* row_amax,
                                      float* col_amax, int32_t* d_status,
                                      void* stream);

/* Graph-safe grouped cast: as nvfp4_group_cast with the routing taken from
 * d_offs (see nvfp4_group_amax_graphsafe).  row_data/row_scale hold
 * m_capacity rows; col_data/col_scale hold k*m_capacity/2 and
 * k*m_capacity/16 bytes, of which the first k*offs[E-1]/2 (/16) are written.
 * Output bytes equal those of nvfp4_group_cast for the same routing. */
int nvfp4_group_cast_graphsafe(const uint16_t* x, int64_t m_capacity, int64_t k,
                               int32_t num_experts, const int32_t* d_offs,
                               const float* row_amax, const float* col_amax,
                               uint8_t* row_data, uint8_t* row_scale,
                               uint8_t* col_data, uint8_t* col_scale,
                               int32_t* d_status, void* stream);

/* Amax + cast in one call (both launches of the grouped cast page's
 * Description, enqueued back to back).  When no columnwise output is
 * requested the rowwise amax and cast run as one fused pass over x, the
 * one-pass-per-row form of "Implement per-token NVFP4 fprop recipe",
 * Important Files Changed; row_amax is still written.  When a columnwise
 * output is requested and every expert is small -- the largest expert's
 * rows times k (m_capacity * k for the graph-safe form, where any expert
 * may hold all rows) at most NVFP4G_SMALL_MAX_EXPERT_ELEMS, and k at most
 * NVFP4G_SMALL_MAX_K -- the whole path runs as one launch with one
 * work-group per expert, where the general path's three launches would
 * cost more than the work.  Every path writes the same bytes. */
#define NVFP4G_SMALL_MAX_EXPERT_ELEMS (1 << 16)
#define NVFP4G_SMALL_MAX_K 512  /* = NVFP4G_SMALL_MAX_EXPERT_ELEMS / 128: an expert has 128 rows or none */
int nvfp4_group_quantize(const uint16_t* x, int64_t sum_m, int64_t k,
                         int32_t num_experts, const int64_t* h_splits,
                         float* row_amax, float* col_amax, uint8_t* row_data,
                         uint8_t* row_scale, uint8_t* col_data,
                         uint8_t* col_scale, void* stream);

/* Graph-safe form of nvfp4_group_quantize. */
int nvfp4_group_quantize_graphsafe(const uint16_t* x, int64_t m_capacity,
                                   int64_t k, int32_t num_experts,
                                   const int32_t* d_offs, float* row_amax,
                                   float* col_amax, uint8_t* row_data,
                                   uint8_t* row_scale, uint8_t* col_data,
                                   uint8_t* col_scale, int32_t* d_status,
                                   void* stream);

/* Dequantisation of row-scaled NVFP4 ("Implement per-token NVFP4 fprop
 * recipe", TransformerEngine PR 2931, Important Files Changed: the dequant
 * looks the amax up by the element's row).  Element i of a line with amax A
 * and block scale S:  out = (value(code) * value(S)) * (A / 2688)  (fp32).
 * Scale bytes are expected to be codes the cast writes (0x00 .. 0x7E); other
 * bytes give unspecified values (no error is reported).
 *
 * Rowwise: row_data [rows, k/2], row_scale [rows, k/16], row_amax [rows]
 * -> out fp32 [rows, k].  Rows are independent (pass the routed row count). */
int nvfp4_group_dequant_rowwise(const uint8_t* row_data, const uint8_t* row_scale,
                                const float* row_amax, int64_t rows, int64_t k,
                                float* out, void* stream);

/* Columnwise: the transposed output of nvfp4_group_cast (per expert [k, M_e]
 * lines with amax col_amax[e*k + c]) -> out fp32 in the same transposed
 * layout: expert e's block of k lines of M_e values at element offset k*r_e. */
int nvfp4_group_dequant_columnwise(const uint8_t* col_data, const uint8_t* col_scale,
                                   const float* col_amax, int64_t sum_m, int64_t k,
                                   int32_t num_experts, const int64_t* h_splits,
                                   float* out, void* stream);

/* Graph-safe columnwise dequant: routing from d_offs as in
 * nvfp4_group_cast_graphsafe; elements beyond k*offs[E-1] are not written. */
int nvfp4_group_dequant_columnwise_graphsafe(const uint8_t* col_data,
                                             const uint8_t* col_scale,
                                             const float* col_amax,
                                             int64_t m_capacity, int64_t k,
                                             int32_t num_experts,
                                             const int32_t* d_offs, float* out,
                                             int32_t* d_status, void* stream);

/* Grouped MXFP4 cast: the power-of-two-scaled sibling format named on the
 * TransformerEngine PR 3824 page (Changes item 1, Testing): E2M1 elements,
 * blocks of 32, one E8M0 scale byte per block.  The scale rule is the OCP
 * Microscaling (MX) v1.0 one: for a block with amax A,
 * shared = floor(log2 A) - 2 clamped to [-127, 127] (-127 for A == 0),
 * byte = shared + 127, code = E2M1(x / 2^shared) (nearest, ties to even,
 * saturating at 6, sign kept).  Each block is independent: no amax pass.
 *
 * x, sum_m, num_experts, h_splits as in nvfp4_group_cast; k > 0 and a
 * multiple of 32 (else NVFP4G_EINVAL).  Outputs (caller-owned, 16-byte
 * aligned; a direction is produced when its data pointer is non-NULL, and
 * then needs its scale pointer):
 *   row_data  [sum_m, k/2]   packed codes, element 2j in the low nibble
 *   row_scale [sum_m, k/32]  E8M0 bytes
 *   col_data  per expert e: [k, M_e/2] at byte k*r_e/2 (column c of expert
 *             e packed along its rows)
 *   col_scale per expert e: [k, M_e/32] at byte k*r_e/32
 * Inputs must be finite.  Stream-ordered; allocates nothing. */
int mxfp4_group_cast(const uint16_t* x, int64_t sum_m, int64_t k,
                     int32_t num_experts, const int64_t* h_splits,
                     uint8_t* row_data, uint8_t* row_scale, uint8_t* col_data,
                     uint8_t* col_scale, void* stream);

/* Graph-safe form of mxfp4_group_cast: routing from the device inclusive
 * row ends d_offs[E] (as in nvfp4_group_cast_graphsafe); buffers sized for
 * m_capacity rows; rows at or beyond offs[E-1] are not written; bad routing
 * sets NVFP4G_DEV_* bits in *d_status and writes nothing. */
int mxfp4_group_cast_graphsafe(const uint16_t* x, int64_t m_capacity,
                               int64_t k, int32_t num_experts,
                               const int32_t* d_offs, uint8_t* row_data,
                               uint8_t* row_scale, uint8_t* col_data,
                               uint8_t* col_scale, int32_t* d_status,
                               void* stream);

/* Row-scaled NVFP4 grouped GEMM, the consumer of the cast ("Implement
 * per-token NVFP4 fprop recipe", TransformerEngine PR 2931, Greptile Summary
 * and sequence diagram: the GEMM runs on the block-scaled FP4 operands with
 * the per-row amax set aside, produces fp32, and its rows are then
 * multiplied by the row amax; grouped, one GEMM per expert).  Forward (and
 * data-gradient) form, both operands stored along the contraction index k:
 * for expert e and each of its rows r,
 *     out[r, j] = sum_{t<k} xa[r, t] * xb_e[j, t],   j < n,
 * where xa is the rowwise cast output (a_data [sum_m, k/2], a_scale
 * [sum_m, k/16], a_amax [sum_m]) and xb_e is expert e's operand in the same
 * rowwise layout (b_data [E, n, k/2], b_scale [E, n, k/16], b_amax [E*n]; a
 * per-tensor-scaled operand is the case of a constant b_amax).  An element
 * decodes to value(code) * value(S) * (A / 2688); the kernel computes
 *     out = (acc * (a_amax[r] / 2688)) * (b_amax[e*n + j] / 2688)
 * with acc the fp32 MFMA sum of the exact products value(code)*value(S)
 * (fp16 operands).  For the data gradient pass the columnwise cast of each
 * expert's weight as b.  Scale bytes are expected to be codes the cast
 * writes (0x00 .. 0x7E); other bytes give unspecified values (no error is
 * reported).  out: fp32 [sum_m, n], row-major, caller-owned.
 * k a positive multiple of 128 (<= 2^22), n a positive multiple of 16
 * (<= 2^20); data pointers 16-byte aligned, scale and amax pointers 4-byte
 * aligned; otherwise NVFP4G_EINVAL / NVFP4G_EALIGN and nothing is enqueued. */
int nvfp4_group_gemm(const uint8_t* a_data, const uint8_t* a_scale,
                     const float* a_amax, const uint8_t* b_data,
                     const uint8_t* b_scale, const float* b_amax, int64_t sum_m,
                     int64_t n, int64_t k, int32_t num_experts,
                     const int64_t* h_splits, float* out, void* stream);

/* Graph-safe form of nvfp4_group_gemm: routing from the device inclusive row
 * ends d_offs[E] (as in nvfp4_group_cast_graphsafe); a and out hold
 * m_capacity rows, of which rows at or beyond offs[E-1] are neither read nor
 * written; bad routing sets NVFP4G_DEV_* bits in *d_status and writes
 * nothing. */
int nvfp4_group_gemm_graphsafe(const uint8_t* a_data, const uint8_t* a_scale,
                               const float* a_amax, const uint8_t* b_data,
                               const uint8_t* b_scale, const float* b_amax,
                               int64_t m_capacity, int64_t n, int64_t k,
                               int32_t num_experts, const int32_t* d_offs,
                               float* out, int32_t* d_status, void* stream);

/* Weight-gradient form ("[PyTorch] Enable NVFP4 row-scaled (per-token)
 * backward for GroupedLinear", TransformerEngine PR 3324, Greptile Summary:
 * an NT GEMM per expert on the columnwise operands, each with a per-column
 * amax): with a = the columnwise cast of dY (per expert [n, M_e] lines at byte
 * n*r_e/2, scales at n*r_e/16, amax a_col_amax[e*n + i]) and b = the
 * columnwise cast of X (per expert [k, M_e] lines, amax b_col_amax[e*k + j]),
 *     out[e, i, j] = sum_{r in expert e} xa_e[i, r] * xb_e[j, r]
 * (dW_e = dY_e^T X_e), computed as in nvfp4_group_gemm; an expert without
 * rows gets zeros.  out: fp32 [E, n, k].  n and k positive multiples of 16
 * (<= 2^20); at most 2^22 rows per expert. */
int nvfp4_group_gemm_wgrad(const uint8_t* a_col_data, const uint8_t* a_col_scale,
                           const float* a_col_amax, const uint8_t* b_col_data,
                           const uint8_t* b_col_scale, const float* b_col_amax,
                           int64_t sum_m, int64_t n, int64_t k,
                           int32_t num_experts, const int64_t* h_splits,
                           float* out, void* stream);

/* Graph-safe weight-gradient form: the routing comes from the device
 * inclusive row ends d_offs[E] (as in nvfp4_group_cast_graphsafe); the
 * columnwise operands are laid out for that routing and out [E, n, k] is
 * fully written (zeros for experts without rows).  m_capacity <= 2^22.  Bad
 * routing sets NVFP4G_DEV_* bits in *d_status and writes nothing. */
int nvfp4_group_gemm_wgrad_graphsafe(const uint8_t* a_col_data,
                                     const uint8_t* a_col_scale,
                                     const float* a_col_amax,
                                     const uint8_t* b_col_data,
                                     const uint8_t* b_col_scale,
                                     const float* b_col_amax, int64_t m_capacity,
                                     int64_t n, int64_t k, int32_t num_experts,
                                     const int32_t* d_offs, float* out,
                                     int32_t* d_status, void* stream);

/* Grouped cast with four-over-six block scaling: the "four_over_six" NVFP4
 * recipe named on the torchtitan converter page ("[NVFP4 4over6] Add the
 * grouped-experts four-over-six converter", Summary and Review pass: knobs
 * err_mode, e4m3_scale_bound, row_scaled).  The page does not state the
 * block rule; the one implemented is that of the published method of the
 * same name ("Four Over Six: More Accurate NVFP4 Quantization with Adaptive
 * Block Scaling"), as a reading, not as a page fact.  Per line with amax A
 * and per 16-element block with block amax b, each step one IEEE binary32
 * operation (round to nearest even, no FMA contraction, denormals kept):
 *     s = A / (6 * scale_bound)
 *     for k = 6 and k = 4:
 *       t_k = (b / k) / s (0 when s == 0);  S_k = E4M3FN(t_k) (as above)
 *       d_k = value(S_k) * s;  m_k = 1 / d_k (0 when d_k == 0, <= FLT_MAX)
 *       c_i = E2M1(x_i * m_k);  x^_i = (value(c_i) * value(S_k)) * s
 *       err_k = (...((0 + r_0) + r_1) + ... ) + r_15, element order, with
 *               r_i = (x_i - x^_i)^2 (err_mode 0) or |x_i - x^_i| (1)
 *     the block keeps k = 4 (codes and scale) when err_4 < err_6, else k = 6.
 * Dequantisation: (value(code) * value(S)) * (A / (6 * scale_bound)).  With
 * scale_bound = 448 the k = 6 candidate is the plain cast's block step.
 * scale_bound: 1 .. NVFP4G_4O6_MAX_BOUND; err_mode: NVFP4G_4O6_ERR_MSE or
 * NVFP4G_4O6_ERR_MAE; anything else returns NVFP4G_EINVAL.  Amax inputs
 * (from nvfp4_group_amax), layouts, directions and the other arguments as
 * in nvfp4_group_cast, including its condition on the amax vectors (the
 * fast quotients here were checked over every bf16 line amax, bound and
 * block amax at most the line amax).  x must be finite. */
#define NVFP4G_4O6_ERR_MSE 0
#define NVFP4G_4O6_ERR_MAE 1
#define NVFP4G_4O6_MAX_BOUND 448
#define NVFP4G_4O6_DEFAULT_BOUND 256 /* largest power of two with 1.5 * bound <= 448 */
int nvfp4_group_cast_4over6(const uint16_t* x, int64_t sum_m, int64_t k,
                            int32_t num_experts, const int64_t* h_splits,
                            const float* row_amax, const float* col_amax,
                            int32_t scale_bound, int32_t err_mode,
                            uint8_t* row_data, uint8_t* row_scale,
                            uint8_t* col_data, uint8_t* col_scale, void* stream);

/* Graph-safe form of nvfp4_group_cast_4over6: routing from d_offs, buffers
 * and status as in nvfp4_group_cast_graphsafe; output bytes equal those of
 * nvfp4_group_cast_4over6 for the same routing. */
int nvfp4_group_cast_4over6_graphsafe(const uint16_t* x, int64_t m_capacity,
                                      int64_t k, int32_t num_experts,
                                      const int32_t* d_offs,
                                      const float* row_amax,
                                      const float* col_amax,
                                      int32_t scale_bound, int32_t err_mode,
                                      uint8_t* row_data, uint8_t* row_scale,
                                      uint8_t* col_data, uint8_t* col_scale,
                                      int32_t* d_status, void* stream);

/* Static description of a status code. */
const char* nvfp4_group_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GROUP_H_ */
