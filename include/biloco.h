/*
 * biloco.h -- C ABI of libbiloco_hip: the decode-time fused product of BiLoCo
 * on AMD Instinct MI355X (gfx950).
 *
 *     y = Q4(x) . deq(R)^T  +  sum_i alpha_i (x . v_i) u_i
 *
 * Source of the operation: "BiLoCo: Binary Low-Rank Corrections for
 * Post-Training Quantization" (project README).  Its intro gives the weight
 * model W ~ U diag(alpha) V^T + R with U in {+-1}^{N x r}, V in {+-1}^{K x r}
 * and R stored in NVFP4; its section "Kernel" gives the fused product, the
 * decode batch limit (M <= 32), z = alpha (.) (V x) computed from the packed
 * signs of V, the expansion of z through the packed signs of U before the
 * bf16 store, and the launcher's operands: NVFP4 codes and block scales of R,
 * the fp32 global scale, pack_signs(V.T), pack_signs(U.T), alpha in bf16, the
 * NVFP4 activation (codes + block scales) and the bf16 activation x.
 *
 * Conventions shared by every entry point
 *  - Memory: every array pointer is DEVICE memory owned by the caller.  The
 *    library allocates nothing on any call path and keeps no pointer after a
 *    call returns.
 *  - Asynchrony: calls are ordered on `stream` (NULL = the null stream) and
 *    return as soon as the work is enqueued.  The status reports host-side
 *    argument checks and the launch itself, never the kernel's completion.
 *  - Errors: arguments are checked on the host BEFORE any HIP call; a bad
 *    argument returns BILOCO_ERR_INVALID_VALUE or BILOCO_ERR_UNSUPPORTED and
 *    enqueues nothing.  No exception crosses the ABI and nothing is printed.
 *  - Layouts are row-major.  "bf16" arrays hold raw bfloat16 bit patterns
 *    (uint16_t); NVFP4 element codes are E2M1, two per byte, element 2j in
 *    the LOW nibble of byte j; block scales are E4M3 (OCP "FN": bias 7, max
 *    448, no infinity), one byte per 16 consecutive elements along K.
 *  - Alignment: every pointer must be 16-byte aligned.  Reads may cover the
 *    rest of the 16-byte block that holds an array's last byte (never more,
 *    never across a page); such bytes do not affect any result.
 *  - Thread safety: the host side keeps no mutable state; concurrent calls
 *    are safe as long as they do not share an output or a workspace.
 */
#ifndef BILOCO_H_
#define BILOCO_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t biloco_status;
#define BILOCO_OK                       0
#define BILOCO_ERR_INVALID_VALUE        1  /* null pointer, bad size, misaligned pointer */
#define BILOCO_ERR_UNSUPPORTED          2  /* well-formed but outside what the kernels handle */
#define BILOCO_ERR_HIP                  3  /* the HIP runtime reported an error at launch */
#define BILOCO_ERR_WORKSPACE_TOO_SMALL  4

/* Schedules of biloco_gemm_lowrank_sched (BiLoCo "Kernel": the launcher picks
 * the fastest mode for batch size and rank, and can list the modes a shape
 * allows).  The modes here are this library's own, designed for gfx950. */
#define BILOCO_SCHED_AUTO        0  /* pick per shape (biloco_default_schedule) */
#define BILOCO_SCHED_UNFUSED     1  /* two launches: z, then a vector-ALU product kernel that
                                       adds the correction before the store (the default at
                                       M <= 2 with r == 0, where it is one launch; a plain,
                                       slow fallback at larger M) */
#define BILOCO_SCHED_FUSED_GEMV  2  /* one launch; vector-ALU dot products; M <= 2, r >= 1
                                       (the default there): its first workgroups compute z
                                       while the others stream R, which apply z through
                                       sign tables in LDS.  Needs every workgroup resident
                                       at once for its speed, not for its results: a wait
                                       for z is bounded, after which the waiting thread
                                       computes the value itself */
#define BILOCO_SCHED_FUSED_MFMA  3  /* matrix-core products for any M <= 32: a z kernel
                                       (skipped when r == 0; for K > 7168 a second launch
                                       sums its K-slices), then one product kernel whose
                                       accumulators take the correction before the store,
                                       then (only when K is split over workgroups) a launch
                                       that sums the K-slices; the default at M >= 3 where
                                       neither BILOCO_SCHED_MFMA_SIDE nor
                                       BILOCO_SCHED_MFMA_ZEPI applies */
#define BILOCO_SCHED_COMPOSED    4  /* separate launches: the plain FP4 product (fp32, in the
                                       workspace), z, then y = bf16(product + z . U^T) by
                                       4-bit sign lookup tables: the unfused form the fused
                                       schedules are timed against; r <= 1024 */
#define BILOCO_SCHED_COMPOSED_MFMA 5 /* as BILOCO_SCHED_COMPOSED, the correction by bf16
                                       MFMAs of z (high + low) against U's +-1 signs
                                       instead of lookup tables; r <= 1024 */
#define BILOCO_SCHED_MFMA_ALLWG  6  /* matrix-core products, r >= 1 (BiLoCo "Kernel": the
                                       mode where every CTA takes part in the correction
                                       at kernel entry): one product launch in which
                                       every workgroup first computes one tile of z
                                       (a 32-index word of V over a K-part), the last
                                       tile of each word finishes it, and the product
                                       applies the finished words after its row blocks;
                                       plus the K-slice sum launch when K is split.
                                       Needs every workgroup of the launch resident at
                                       once for its speed, not for its results: a wait
                                       for z is bounded, after which the waiting wave
                                       computes the word itself */
#define BILOCO_SCHED_MFMA_SIDE   7  /* matrix-core products, r >= 1, x of at most 96 KiB
                                       (BiLoCo "Kernel": side CTAs compute z while the
                                       others stream R): one product launch whose first
                                       8 to 32 workgroups stream no rows and compute z,
                                       a word or half a word of K each; the others apply
                                       the published words after their row blocks; plus
                                       the K-slice sum launch when K is split.  Needs
                                       every workgroup resident at once for its speed, not
                                       for its results (bounded waits, as above) */
#define BILOCO_SCHED_MFMA_ZEPI   8  /* matrix-core products, 1 <= r <= 1024, K split over
                                       workgroups (the default at M >= 3 there, unless
                                       BILOCO_SCHED_MFMA_SIDE applies): one product launch
                                       whose first 8 to 32 workgroups stream no rows and
                                       compute z, a K-part of every word each, then
                                       finish its words; the
                                       product takes no correction; the launch that sums
                                       the K-slices adds z . U^T (bf16 MFMAs of z's high
                                       and low parts against U's signs) before the store.
                                       The side workgroups' wait for one another is
                                       bounded, after which the words still missing are
                                       computed from x and V (slow) */

/* Human-readable name of a status code (static string, never NULL). */
const char *biloco_status_string(biloco_status s);

/* pack_signs (BiLoCo "Kernel": the launcher receives pack_signs(V.T) and
 * pack_signs(U.T)).  Packs a sign matrix along its FIRST axis, 32 signs per
 * 32-bit word:
 *   signs  int8 [rows][cols]; an entry < 0 means -1, any other value +1.
 *          Pass V^T ([r][K]) or U^T ([r][N]): rows is the rank axis.
 *   packed uint32 [ceil(rows/32)][cols]; bit b of word (w, c) is 1 when
 *          signs[32w+b][c] < 0; bits for 32w+b >= rows are written as 0.
 * rows >= 1, cols >= 1.  Bit-exact; one launch. */
biloco_status biloco_pack_signs(const int8_t *signs, int64_t rows, int64_t cols,
                                uint32_t *packed, hipStream_t stream);

/* Activation FP4 quantisation (BiLoCo "Kernel": the fused product takes
 * FP4(x) as NVFP4 codes and block scales).  For each row m and each block of
 * 16 consecutive k: amax = max |x|; scale = E4M3(amax / 6) rounded to
 * nearest-even (saturating at 448); code = E2M1(x / scale) rounded to
 * nearest-even (saturating at 6) with the sign of x kept, also for values
 * that round to zero; a zero scale gives signed-zero codes.
 *   x_bf16   [M][K] bf16
 *   a_codes  [M][K/2] uint8  (E2M1 pairs, even k in the low nibble)
 *   a_scales [M][K/16] uint8 (E4M3)
 * M >= 1, K >= 32, K % 32 == 0.  Inputs must be finite.  Bit-exact. */
biloco_status biloco_quant_act_fp4(const uint16_t *x_bf16, int32_t M, int32_t K,
                                   uint8_t *a_codes, uint8_t *a_scales, hipStream_t stream);

/* NVFP4 quantisation of a weight matrix, the residual R (BiLoCo intro and
 * section "Decomposition": R is stored in NVFP4; section "Kernel": the
 * product takes R's E2M1 codes, its E4M3 block scales and an fp32 global
 * scale).  The pages give no rounding recipe; this one puts the largest
 * block scale on the largest E4M3 value:
 *   g = fp32(max|w| / 2688)   (2688 = 6 * 448; g = 1 when every w is 0)
 *   per row n and block b of 16 consecutive k, with a = max |w| over it:
 *     scale[n][b] = E4M3(fp32(fp32(a / 6) / g)), nearest, ties to even,
 *                   saturating at 448
 *     d = fp32(e4m3(scale[n][b]) * g)
 *     code = E2M1(fp32(|w| / d)), nearest, ties to the even code, saturating
 *            at 6, sign of w kept (also for values that round to zero);
 *            d == 0 gives signed-zero codes
 *   each fp32(...) one correctly rounded single-precision operation, so that
 *   w ~ g * e4m3(scale) * e2m1(code), the operand form biloco_gemm_lowrank
 *   takes as (w_codes, w_scales, w_global_scale).
 *   w        [N][K] fp32, finite (input)
 *   codes    [N][K/2] uint8  (even k in the low nibble)
 *   scales   [N][K/16] uint8 (E4M3)
 *   g_out    one fp32 (device memory)
 *   workspace >= biloco_quant_weight_workspace_bytes(...) bytes of device
 *          memory; no fill needed (every call writes it before reading it);
 *          not shared by calls that can run at the same time.
 * N >= 1, K >= 16, K % 16 == 0 (biloco_gemm_lowrank further needs K % 32 == 0);
 * N * K <= 2^38.  No two of the five arrays may overlap.  Two launches on
 * `stream`.  Bit-exact. */
biloco_status biloco_quant_weight_nvfp4(const float *w, int64_t N, int64_t K, uint8_t *codes,
                                        uint8_t *scales, float *g_out, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace biloco_quant_weight_nvfp4 needs (a few KiB, never 0).
 * Same shape rules. */
biloco_status biloco_quant_weight_workspace_bytes(int64_t N, int64_t K, size_t *bytes);

/* Greedy sign peeling with the joint coefficient refit (BiLoCo intro and
 * section "Decomposition"): W ~ U diag(alpha) V^T + R with U in {+-1}^{m x r},
 * V in {+-1}^{n x r}.  Term i (i = 0 .. r-1) starts from the signs v_init[i],
 * then T times: u = sign(R v), v = sign(R^T u), with R = W minus the terms
 * found so far and sign(0) = +1; its greedy coefficient is u^T R v / (m n)
 * (the Frobenius optimum for fixed signs), and R loses that term.  After the
 * r terms the coefficients are refit together by least squares for the fixed
 * signs (normal equations G alpha = b, G_ij = (u_i . u_j)(v_i . v_j),
 * b_i = u_i^T W v_i), and R = W - U diag(alpha) V^T with the refit ones.
 *   W          [m][n] fp32 (input; finite)
 *   v_init     uint32 [r][ceil(n/32)]: start signs of each term, bit b of word
 *              w is coordinate 32w+b, a set bit meaning -1 (bits >= n ignored).
 *              The caller draws them: the pages start each term from random
 *              signs.
 *   u_packed   uint32 [ceil(r/32)][m] = pack_signs(U^T)  (output; the form
 *   v_packed   uint32 [ceil(r/32)][n] = pack_signs(V^T)   biloco_gemm_lowrank takes)
 *   alpha      fp32 [r]: refit coefficients (output)
 *   alpha_greedy fp32 [r] or NULL: the coefficients found during the peel
 *   R          fp32 [m][n] or NULL: the residual W - U diag(alpha) V^T
 *   workspace  >= biloco_peel_workspace_bytes(m, n, r) bytes; no fill needed.
 * 1 <= m <= 2^18, 4 <= n <= 2^18 with n % 4 == 0, 1 <= r <= 1024, T >= 1.
 * Arithmetic: fp32 sums for R v and R^T u (the terms found so far enter
 * through exact integer sign dot products), fp64 for the refit.  A sign
 * decision can differ from another summation order's where |(R v)_a| or
 * |(R^T u)_k| is within rounding of 0.  If the sign terms are linearly
 * dependent (a Cholesky pivot of G falls below 1e-6 m n, e.g. a term found
 * twice), least squares has many minimisers: each term whose outer product
 * lies in the span of the earlier ones is dropped from the solve (its alpha
 * is 0) and alpha is the least-squares minimiser of the others.
 * About (5 T + 1) r + 4 launches on `stream`; no two of the output and
 * input arrays may overlap. */
biloco_status biloco_peel_decompose(const float *W, int64_t m, int64_t n, int32_t r, int32_t T,
                                    const uint32_t *v_init, uint32_t *u_packed, uint32_t *v_packed,
                                    float *alpha, float *alpha_greedy, float *R, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace biloco_peel_decompose needs.  Same shape rules. */
biloco_status biloco_peel_workspace_bytes(int64_t m, int64_t n, int32_t r, size_t *bytes);

/* Bytes of device workspace biloco_gemm_lowrank needs for this shape, enough
 * for every schedule the shape allows.  May be 0 (then workspace may be
 * NULL).  Same argument rules as biloco_gemm_lowrank. */
biloco_status biloco_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t r,
                                          size_t *bytes);

/* The fused product (BiLoCo "Kernel"):
 *   y[m][n] = bf16( g * sum_k A[m][k] B[n][k]  +  sum_{i<r} z[m][i] U[n][i] )
 *   A[m][k] = e2m1(a_codes) * e4m3(a_scales[m][k/16])   (the FP4 activation)
 *   B[n][k] = e2m1(w_codes) * e4m3(w_scales[n][k/16])   (the NVFP4 residual R)
 *   z[m][i] = alpha_i * sum_k x[m][k] V[k][i]           (bf16 x, not FP4)
 *   U, V in {+-1}: bit 1 of the packed words means -1.
 * Operands:
 *   a_codes  [M][K/2] uint8, a_scales [M][K/16] uint8  (biloco_quant_act_fp4)
 *   x_bf16   [M][K] bf16
 *   w_codes  [N][K/2] uint8, w_scales [N][K/16] uint8, w_global_scale (g)
 *   v_packed [ceil(r/32)][K] uint32  = pack_signs(V^T)
 *   u_packed [ceil(r/32)][N] uint32  = pack_signs(U^T)
 *   alpha_bf16 [r] bf16
 *   y_bf16   [M][N] bf16 (output; exactly M rows; must not alias an input)
 *   workspace: >= biloco_gemm_workspace_bytes(...) bytes of device memory,
 *          ZERO-FILLED by the caller before its first use; afterwards the
 *          library keeps it consistent by itself.  One workspace must not be
 *          used by two calls that can run at the same time (use one per
 *          stream).
 * Limits: 1 <= M <= 32; N >= 1; K >= 32 and K % 32 == 0; r >= 0;
 *   N * K / 2 < 2^31 and 4 * ceil(r/32) * max(N, K) < 2^31 (R's codes and the
 *   sign words are addressed with 32-bit byte offsets).
 * With r == 0, x_bf16, v_packed, u_packed and alpha_bf16 may be NULL.
 * Accuracy: y is within 8e-3*|y_ref| + 1e-3*rms(y_ref) of the exact value
 * (fp32 accumulation, bf16 output rounding).  One to four launches on
 * `stream`, depending on the schedule and the shape. */
biloco_status biloco_gemm_lowrank(const uint8_t *a_codes, const uint8_t *a_scales,
                                  const uint16_t *x_bf16,
                                  const uint8_t *w_codes, const uint8_t *w_scales,
                                  float w_global_scale,
                                  const uint32_t *v_packed, const uint32_t *u_packed,
                                  const uint16_t *alpha_bf16,
                                  int32_t M, int32_t N, int32_t K, int32_t r,
                                  uint16_t *y_bf16, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* As biloco_gemm_lowrank, with an explicit schedule (BILOCO_SCHED_*).  A
 * schedule the shape does not allow returns BILOCO_ERR_UNSUPPORTED. */
biloco_status biloco_gemm_lowrank_sched(const uint8_t *a_codes, const uint8_t *a_scales,
                                        const uint16_t *x_bf16,
                                        const uint8_t *w_codes, const uint8_t *w_scales,
                                        float w_global_scale,
                                        const uint32_t *v_packed, const uint32_t *u_packed,
                                        const uint16_t *alpha_bf16,
                                        int32_t M, int32_t N, int32_t K, int32_t r,
                                        uint16_t *y_bf16, void *workspace, size_t workspace_bytes,
                                        int32_t schedule, hipStream_t stream);

/* The activation quantisation and the product in one call (the per-token
 * hot path of the BiLoCo README's section "Kernel": FP4(x), then the fused
 * product).  Writes a_codes / a_scales exactly as biloco_quant_act_fp4 would
 * (they are OUTPUTS here, and must not overlap any other array), then
 * computes y exactly as biloco_gemm_lowrank_sched.  Where the schedule
 * computes z in a launch of its own (r > 0: BILOCO_SCHED_UNFUSED at M <= 2,
 * BILOCO_SCHED_FUSED_MFMA), that launch also quantises x, so the call takes
 * one launch fewer than the two calls; elsewhere the quantisation is a
 * launch of its own.  x_bf16 is required also when r == 0.  Same limits,
 * workspace and errors as biloco_gemm_lowrank_sched. */
biloco_status biloco_gemm_lowrank_quant(const uint16_t *x_bf16, uint8_t *a_codes, uint8_t *a_scales,
                                        const uint8_t *w_codes, const uint8_t *w_scales,
                                        float w_global_scale, const uint32_t *v_packed,
                                        const uint32_t *u_packed, const uint16_t *alpha_bf16,
                                        int32_t M, int32_t N, int32_t K, int32_t r, uint16_t *y_bf16,
                                        void *workspace, size_t workspace_bytes, int32_t schedule,
                                        hipStream_t stream);

/* For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): biloco_gemm_lowrank_quant without
 * a workspace argument.  The workspace is a device array of
 * BILOCO_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU (each
 * GPU the call runs on holds its copy until the process ends); the call
 * allocates nothing.  The array is used on the current device (hipGetDevice),
 * so `stream` must belong to it.  Every call on one GPU shares that GPU's
 * array: calls that can run at the same time on one GPU (other streams,
 * other threads) race and give wrong results; calls ordered on one stream
 * are safe.  A shape whose workspace (biloco_gemm_workspace_bytes) exceeds
 * the array returns BILOCO_ERR_UNSUPPORTED before any HIP call; otherwise
 * the arguments, results and errors are those of biloco_gemm_lowrank_quant. */
#define BILOCO_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
biloco_status biloco_gemm_lowrank_quant_noalloc(const uint16_t *x_bf16, uint8_t *a_codes,
                                                uint8_t *a_scales, const uint8_t *w_codes,
                                                const uint8_t *w_scales, float w_global_scale,
                                                const uint32_t *v_packed, const uint32_t *u_packed,
                                                const uint16_t *alpha_bf16, int32_t M, int32_t N,
                                                int32_t K, int32_t r, uint16_t *y_bf16,
                                                int32_t schedule, hipStream_t stream);

/* Host-only argument check of biloco_gemm_lowrank_sched: returns the status
 * the call would return for these arguments before launching anything.
 * Makes no HIP call (usable without a GPU). */
biloco_status biloco_gemm_check(const void *a_codes, const void *a_scales, const void *x_bf16,
                                const void *w_codes, const void *w_scales,
                                const void *v_packed, const void *u_packed,
                                const void *alpha_bf16,
                                int32_t M, int32_t N, int32_t K, int32_t r,
                                const void *y_bf16, const void *workspace,
                                size_t workspace_bytes, int32_t schedule);

/* The schedule BILOCO_SCHED_AUTO resolves to for this shape (0 if the shape
 * is invalid).  No HIP call. */
int32_t biloco_default_schedule(int32_t M, int32_t N, int32_t K, int32_t r);

/* Writes up to `cap` schedules this shape allows into `out` and returns how
 * many there are (BiLoCo "Kernel": modes_for(M, r, K)).  No HIP call. */
int32_t biloco_schedules_for(int32_t M, int32_t N, int32_t K, int32_t r,
                             int32_t *out, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* BILOCO_H_ */
