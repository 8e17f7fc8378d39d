/*
 * q4.h -- C ABI of libq4: weight-only 4-bit block-quantised matmul on
 * AMD Instinct MI355X (gfx950).
 *
 *   y[m][n] = sum_k x[m][k] * w[n][k],   w[n][k] = (c[n][k] - 8) * s[n][k / 32]
 *
 * Where the operation comes from.  The spec "spec: specialized model
 * runtimes" puts quant/dequant and GEMM in its T0 kernel tier (section
 * "Architecture"), names a quantised GEMM as the first measured kernel
 * (section "Feasibility gate") and groupwise-int as the first weight profile
 * (section "Target package and artifact"); it wants runtimes loaded
 * in-process behind a C ABI whose version is pinned and whose failures
 * return a clean value the caller handles (sections "Architecture" and
 * "Prototype ABI scope").  The expert-routed call follows the routed top-k
 * expert matmul plus weighted sum of the "Layer Package Repository Spec"
 * (MoE fixture paragraph under "Policy Resolution").  The pages fix no bit
 * layout; the layout below is this library's.
 *
 * Data layout (all tensors contiguous, row-major, in DEVICE memory):
 *   x    bf16  [M][K]      activations (bit patterns, uint16 storage)
 *   w_q  uint8 [N][K/2]    codes: element k = 2j is the LOW nibble of byte
 *                          j of its row, k = 2j+1 the HIGH nibble; a code c
 *                          stands for the integer c - 8 (-8..7)
 *   w_s  fp16  [N][K/32]   one IEEE binary16 scale per 32 consecutive k
 *   y    fp32 or bf16 [M][N]
 * K must be a positive multiple of 32.
 *
 * Numerics.  Products and sums are fp32 and every weight (c-8)*s enters
 * exactly, on every path: each 32-element block's sum of x * (c - 8) is
 * formed first (exact products; on the matrix-core paths the small integers
 * c - 8 are exact bf16 operands) and the block's scale is applied to it once
 * in fp32.  q4_matmul_path tells which kernel a shape takes.  bf16 outputs
 * are rounded nearest-even from the fp32 result.  Results are bit-identical
 * from run to run (no floating-point atomics).
 *
 * Conventions of every call:
 *   - All checks run on the host before anything is enqueued; on any error
 *     nothing is launched and no output is written.
 *   - Check order: dtype, shape, zero-size no-op, NULL, alignment,
 *     workspace, device, pending HIP error, launch.  M == 0 or N == 0 (T == 0 for MoE) returns Q4_OK and touches
 *     nothing (pointers may then be NULL).
 *   - Alignment: every tensor pointer must be 16-byte aligned (the kernels
 *     use 128-bit loads and stores).
 *   - HIP error state: a HIP error already pending when a call is made (from
 *     the caller's own earlier work) is left in place, and the call returns
 *     Q4_ERR_PENDING without launching anything.  An error raised by this
 *     call's own launches is reported as Q4_ERR_LAUNCH and consumed, so no
 *     HIP error state leaves a call.
 *   - Device: the current HIP device must be a gfx950 GPU, else
 *     Q4_ERR_DEVICE.
 *   - The call returns once the work is enqueued on `stream` (a hipStream_t;
 *     NULL is the default stream).  The caller owns and frees every buffer,
 *     synchronises the stream, and keeps the buffers alive until the work
 *     completes.  The library allocates no device memory; where a call can
 *     use scratch memory it takes a caller-owned workspace.
 *   - Calls are thread-safe; calls on one stream execute in order.
 *   - No C++ exception crosses this boundary.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define Q4_API __attribute__((visibility("default")))
#else
#define Q4_API
#endif

#define Q4_ABI_VERSION 10

/* Status codes. */
#define Q4_OK            0
#define Q4_ERR_NULL      1  /* a required pointer is NULL */
#define Q4_ERR_SHAPE     2  /* negative size, K <= 0, K % 32 != 0, or size overflow */
#define Q4_ERR_ALIGN     3  /* a tensor pointer is not 16-byte aligned */
#define Q4_ERR_DTYPE     4  /* unknown output dtype */
#define Q4_ERR_WORKSPACE 5  /* workspace NULL (MoE), misaligned or too small */
#define Q4_ERR_DEVICE    6  /* no current HIP device, or it is not gfx950 */
#define Q4_ERR_LAUNCH    7  /* the HIP runtime reported an error at enqueue */
#define Q4_ERR_PENDING   8  /* a HIP error from before the call was pending: left
                               in place, nothing launched (ABI version 8) */
#define Q4_ERR_SCRATCH   9  /* needs more than Q4_MOE_NOALLOC_MAX_BYTES of the
                               built-in scratch (q4_moe_matmul_noalloc) */
#define Q4_ERR_FLAGS    10  /* unknown bits in a flags argument */

/* Output dtypes. */
#define Q4_F32  0
#define Q4_BF16 1

/* Paths chosen by q4_matmul. */
#define Q4_PATH_GEMV  0     /* fused dequant + matrix-vector, exact weights */
#define Q4_PATH_MFMA  1     /* exact (c - 8) tiles in LDS + bf16 matrix-core
                               tiles, fp32 block scales: exact weights */
#define Q4_PATH_SMALL 2     /* exact (c - 8) on bf16 matrix cores, fp32 block
                               scales: exact weights */

typedef void *q4_stream_t;  /* a hipStream_t */

/* ABI version of the loaded library (== Q4_ABI_VERSION it was built with).
 * A caller built against another version must refuse to use it. */
Q4_API int32_t q4_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL
 * (unknown codes map to "unknown status"). */
Q4_API const char *q4_status_str(int32_t status);

/* Path q4_matmul takes for an [M][K] x [N][K] product; -1 for sizes
 * q4_matmul would reject (M or N negative, K not a positive multiple of 32).
 *   M <= 2                                         Q4_PATH_GEMV
 *   3 <= M <= 32                                   Q4_PATH_SMALL
 *   M <= 128 and ceil(M/128) * ceil(N/128) < 256   Q4_PATH_SMALL
 *   otherwise                                      Q4_PATH_MFMA
 * Host-only: enqueues nothing. */
Q4_API int32_t q4_matmul_path(int64_t M, int64_t N, int64_t K);

/* Path q4_matmul_ex takes (ABI version 7): with_workspace == 0 as
 * q4_matmul_path; otherwise, for a workspace of at least
 * q4_matmul_workspace_bytes(M, N, K) bytes, shapes with 33 <= M <= 128 that
 * q4_matmul_path sends to Q4_PATH_SMALL take Q4_PATH_MFMA (the tiled kernel
 * cut along K) when K is a multiple of 64, N * K is
 * at least 2^24 and the grid of 128 x 128 tiles is small enough to be cut.  q4_mx_matmul_ex follows
 * the same rule (its tiled weights are exact).  Host-only. */
Q4_API int32_t q4_matmul_path_ex(int64_t M, int64_t N, int64_t K, int32_t with_workspace);

/* y = x * dequant(W)^T.
 *   x       bf16  [M][K]    device
 *   w_q     uint8 [N][K/2]  device
 *   w_s     fp16  [N][K/32] device
 *   y       [M][N] device, fp32 (y_dtype = Q4_F32) or bf16 (Q4_BF16);
 *           fully overwritten
 *   M, N, K sizes (K a positive multiple of 32)
 *   stream  hipStream_t or NULL
 * Returns Q4_OK or an error code (see the conventions above). */
Q4_API int32_t q4_matmul(const void *x, const void *w_q, const void *w_s,
                         void *y, int32_t y_dtype,
                         int64_t M, int64_t N, int64_t K, q4_stream_t stream);

/* Device workspace (bytes) that lets q4_matmul_ex cut work along K into
 * slices whose fp32 partial sums are added in order.  Q4_PATH_GEMV shapes:
 * slices * M * N floats, cut when K is above 8192 or the activations are too
 * large for one workgroup's LDS.  Q4_PATH_SMALL: 3..16 rows, slices * M * N
 * floats with one slice per 32 blocks of K when that makes 2..64 slices;
 * otherwise slices * M * N floats for grids of fewer than 1024 workgroups.
 * Tiled shapes
 * (q4_matmul_path_ex(M, N, K, 1) == Q4_PATH_MFMA) with K a multiple of 64:
 * up to 128 rows, tiles of 128 x 128, slices * M * N floats for grids of
 * fewer than 512 tiles (at most 768 / tiles and 64 slices, each of at least
 * 8 steps of 64 k); more rows, tiles of 256 x 128 (one workgroup per CU,
 * 256 a round): slices * M * N floats for grids of fewer than 171 tiles (at
 * most 256 / tiles slices), or, for a grid of whole rounds plus a last round
 * at most half full, the last round's tiles cut into S slices of at least 4
 * steps (S = min(256 / tail tiles, steps / 4)): tail tiles * S * 256 * 128
 * floats.  0 when the call needs none, or for sizes q4_matmul would reject. */
Q4_API size_t q4_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* q4_matmul with an optional workspace.  workspace == NULL: exactly
 * q4_matmul.  Otherwise it must be 16-byte aligned and hold at least
 * q4_matmul_workspace_bytes(M, N, K) bytes (else Q4_ERR_WORKSPACE, checked
 * after the NULL and alignment checks of the tensors); its contents on
 * entry do not matter, and calls that may run concurrently must not share
 * it.  With a workspace, long rows are split into slices whose fp32 partial
 * sums are added in slice order: the result is the same function of the
 * inputs on every run, though its rounding can differ from the unsplit
 * call's in the last bits. */
Q4_API int32_t q4_matmul_ex(const void *x, const void *w_q, const void *w_s,
                            void *y, int32_t y_dtype,
                            int64_t M, int64_t N, int64_t K,
                            void *workspace, size_t workspace_bytes,
                            q4_stream_t stream);

/* Device workspace (bytes) q4_rmsnorm_matmul needs for these sizes (ABI
 * version 8): 0 when the fused matrix-vector form serves the shape (M <= 2,
 * K up to 8192) or a size is invalid; otherwise the normalised activations,
 * M * K bf16 rounded up to 256 bytes, followed by
 * q4_matmul_workspace_bytes(M, N, K) bytes that let the product cut K (a
 * workspace of only the first part is accepted; the product then runs
 * uncut).  Host-only. */
Q4_API size_t q4_rmsnorm_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y = RMSNorm(x) . dequant(W)^T: the quantised matmul behind an RMSNorm
 * prologue, the first measured kernel of "spec: specialized model runtimes"
 * ("Feasibility gate": one quantized GEMM plus fused RMSNorm; "Development
 * sequence", Phase 1).  The pages do not define RMSNorm; this library takes,
 * per activation row m,
 *     x'[m][k] = x[m][k] * gamma[k] / sqrt(mean_k x[m][k]^2 + eps)
 * with the sum of squares in double.
 *   x, w_q, w_s, y, y_dtype, M, N, K   as for q4_matmul
 *   gamma   bf16 [K] device, the norm weights
 *   eps     >= 0 and finite (else Q4_ERR_SHAPE)
 *   workspace, workspace_bytes   device scratch of at least the first part
 *           of q4_rmsnorm_matmul_workspace_bytes(M, N, K) when that is
 *           non-zero (else Q4_ERR_WORKSPACE, after the NULL and alignment
 *           checks); contents on entry do not matter; may be NULL when 0.
 * M <= 2 with K up to 8192: one matrix-vector kernel whose activation
 * staging applies the norm (x' in fp32).  Otherwise the normalised
 * activations are written to the workspace as bf16 (nearest-even; the matrix
 * cores' operand type) and the product takes the q4_matmul_ex path on them;
 * that rounding can move y by at most sum_k hulp(x'[m][k]) * |w[n][k]|,
 * hulp = half a bf16 unit in the last place.  Weights enter exactly.
 * Returns Q4_OK or an error code. */
Q4_API int32_t q4_rmsnorm_matmul(const void *x, const void *gamma, float eps,
                                 const void *w_q, const void *w_s, void *y,
                                 int32_t y_dtype, int64_t M, int64_t N, int64_t K,
                                 void *workspace, size_t workspace_bytes,
                                 q4_stream_t stream);

/* Device workspace (bytes) q4_sb_matmul needs (ABI version 8): the fp32
 * block scales, N * K/32 floats rounded up to 256 bytes, followed by
 * q4_matmul_workspace_bytes(M, N, K) bytes that let the tiled product cut K
 * (optional: a workspace of only the first part is accepted).  0 for an
 * invalid or empty shape.  Host-only. */
Q4_API size_t q4_sb_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y = x . W^T with super-block (two-level) scales (ABI version 8):
 *     w[n][k] = (c[n][k] - 8) * d[n][k/256] * sc[n][k/32]
 * The layer-package spec names K-quant profiles (Q4_K-class, q2_K / q3_K) in
 * "Repository Identity" and "Policy Resolution" without defining them; this
 * is the two-level block-scale structure they share, on this library's codes.
 *   x, w_q, y, y_dtype, M, N   as for q4_matmul
 *   w_d     fp16  [N][K/256] device, one scale per 256-element super-block
 *   w_sc    uint8 [N][K/32]  device, an unsigned multiplier per block
 *   K       a positive multiple of 256 (else Q4_ERR_SHAPE)
 *   workspace  device scratch of at least the first part of
 *           q4_sb_matmul_workspace_bytes (else Q4_ERR_WORKSPACE, after the
 *           NULL and alignment checks); contents on entry do not matter.
 * Every d * sc is exact in fp32 and every weight enters exactly.  Returns
 * Q4_OK or an error code. */
Q4_API int32_t q4_sb_matmul(const void *x, const void *w_q, const void *w_d,
                            const void *w_sc, void *y, int32_t y_dtype, int64_t M,
                            int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                            q4_stream_t stream);

/* Dequantise W to fp32 ((c-8)*s, exact) or bf16 (that value rounded
 * nearest-even): w_out [N][K] device, out_dtype Q4_F32 or Q4_BF16.  Same
 * conventions as q4_matmul (N == 0 is a no-op). */
Q4_API int32_t q4_dequantize(const void *w_q, const void *w_s, void *w_out,
                             int32_t out_dtype, int64_t N, int64_t K,
                             q4_stream_t stream);

/* bf16 weights -> this format (ABI version 8): the convert step of "spec:
 * specialized model runtimes" ("Target package and artifact": weights are
 * converted into the runtime's profile, then qualified).  The pages fix no
 * method; per 32-element block of a row, m = the element of largest |w|
 * (first on ties), s = fp16(m / -8) (nearest-even; |m / 8| clamped to 65504),
 * c = clamp(rint(w / s) + 8, 0, 15) with an IEEE fp32 quotient and
 * round-half-even (s == 0: every code 8).  The block's largest-magnitude
 * weight is reproduced exactly by dequantisation; every other one to within
 * half a step |s| / 2 (one step for a weight of -m, clamped to code 15).
 *   w    bf16  [N][K]     device
 *   w_q  uint8 [N][K/2]   device, fully overwritten
 *   w_s  fp16  [N][K/32]  device, fully overwritten
 * K a positive multiple of 32.  Returns Q4_OK or an error code. */
Q4_API int32_t q4_quantize(const void *w, void *w_q, void *w_s, int64_t N, int64_t K,
                           q4_stream_t stream);

/* Device workspace (bytes) q4_moe_matmul needs for these sizes; 0 if a size
 * is negative or the size overflows. */
Q4_API size_t q4_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t N);

/* Expert-routed rows:
 *   y[t][n] = sum_{j < topk} g[t][j] * sum_k x[t][k] * w_{id[t][j]}[n][k]
 *   x         bf16  [T][K]          device
 *   w_q       uint8 [E][N][K/2]     device (E experts, each laid out as above)
 *   w_s       fp16  [E][N][K/32]    device
 *   topk_ids  int32 [T][topk]       device; an id outside [0, E) selects no
 *                                   expert and contributes nothing; repeated
 *                                   ids of one token are summed
 *   topk_w    fp32  [T][topk]       device gate weights g
 *   y         fp32  [T][N]          device, fully overwritten
 *   workspace device scratch of at least q4_moe_workspace_bytes(T, topk, E, N)
 *             bytes, 16-byte aligned, owned by the caller; its contents on
 *             entry do not matter and it must not be shared by calls that
 *             may run concurrently
 * Every expert's weights are read once per call, whatever the number of
 * tokens routed to it; the per-(token, slot) products are summed in slot
 * order, so results are bit-identical from run to run.  Returns Q4_OK or an
 * error code (Q4_ERR_WORKSPACE for a missing or short workspace). */
Q4_API int32_t q4_moe_matmul(const void *x, const void *w_q, const void *w_s,
                             const int32_t *topk_ids, const float *topk_w,
                             float *y,
                             int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K,
                             void *workspace, size_t workspace_bytes,
                             q4_stream_t stream);

/* q4_moe_matmul without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops or
 * harnesses that forbid allocation).  Same arguments, checks and result as
 * q4_moe_matmul; the workspace is the library's own scratch array, one per
 * GPU, of Q4_MOE_NOALLOC_MAX_BYTES bytes, held from the first call on that
 * GPU until the process ends.  A call whose q4_moe_workspace_bytes(T, topk,
 * E, N) exceeds that returns Q4_ERR_SCRATCH (after the argument checks,
 * before anything is enqueued).  Every call on one GPU shares its array:
 * calls that may overlap on one GPU (different streams, different host
 * threads) race and must be serialised by the caller; calls on one stream
 * are ordered.  Nothing in the array needs to start at zero (each call
 * rebuilds what it reads).  Allocates nothing (no hipMalloc, no library
 * allocation).  ABI version 8. */
#define Q4_MOE_NOALLOC_MAX_BYTES ((size_t)8 << 20)
Q4_API int32_t q4_moe_matmul_noalloc(const void *x, const void *w_q, const void *w_s,
                                     const int32_t *topk_ids, const float *topk_w,
                                     float *y, int64_t T, int64_t topk, int64_t E,
                                     int64_t N, int64_t K, q4_stream_t stream);

/* Device workspace (bytes) q4_moe_ffn needs for these sizes; 0 if a size is
 * negative or the size overflows. */
Q4_API size_t q4_moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H,
                                         int64_t F);

/* Routed expert FFN of one MoE layer (the routed gate/up and down expert
 * matmuls, the fused SwiGLU split and the weighted sum that the "Layer
 * Package Repository Spec" measures on its MoE fixture, paragraph under
 * "Policy Resolution"):
 *   for each slot j of token t, e = id[t][j]:
 *     gate_f = sum_k x[t][k] * w13_e[2f][k],  up_f = sum_k x[t][k] * w13_e[2f+1][k]
 *     a_f    = silu(gate_f) * up_f,   silu(z) = z / (1 + exp(-z))   (fp32, not rounded)
 *     y[t][h] += g[t][j] * sum_f a_f * w2_e[h][f]
 *   x         bf16  [T][H]             device
 *   w13_q     uint8 [E][2F][H/2]       device; row 2f is the gate row and
 *   w13_s     fp16  [E][2F][H/32]      row 2f+1 the up row of unit f
 *   w2_q      uint8 [E][H][F/2]        device; down projection
 *   w2_s      fp16  [E][H][F/32]
 *   topk_ids, topk_w, workspace        as for q4_moe_matmul (workspace of at
 *                                      least q4_moe_ffn_workspace_bytes bytes)
 *   y         fp32  [T][H]             device, fully overwritten
 * H and F must be positive multiples of 32 and at most 8192 (else
 * Q4_ERR_SHAPE).  Weights enter exactly (as on the matrix-vector path).
 * Every touched expert's weights are read once per call; results are
 * bit-identical from run to run.  T == 0 is a no-op. */
Q4_API int32_t q4_moe_ffn(const void *x, const void *w13_q, const void *w13_s,
                          const void *w2_q, const void *w2_s,
                          const int32_t *topk_ids, const float *topk_w, float *y,
                          int64_t T, int64_t topk, int64_t E, int64_t H, int64_t F,
                          void *workspace, size_t workspace_bytes, q4_stream_t stream);

/* q4_moe_ffn with flags (ABI version 9):
 *   Q4_MOE_WEIGHTED_DOWN  the route weights multiply the SwiGLU outputs before
 *                         the down product (g * a_f in fp32), so the down
 *                         products come out weighted and the final sum over a
 *                         token's slots adds them as they are: the
 *                         weighted-down graph shape that "Execution Policy"
 *                         ("Layer Package Repository Spec") lists as an
 *                         evidence-gated experiment.  Same result up to
 *                         rounding (within the same bar).
 * flags == 0 is q4_moe_ffn.  Unknown bits return Q4_ERR_FLAGS (checked
 * first). */
#define Q4_MOE_WEIGHTED_DOWN 1u
Q4_API int32_t q4_moe_ffn_ex(const void *x, const void *w13_q, const void *w13_s,
                             const void *w2_q, const void *w2_s,
                             const int32_t *topk_ids, const float *topk_w, float *y,
                             int64_t T, int64_t topk, int64_t E, int64_t H, int64_t F,
                             uint32_t flags, void *workspace, size_t workspace_bytes,
                             q4_stream_t stream);

/* y = x . dequant(W)^T with 4-bit float block weights (ABI version 5): the
 * 4-bit float block format that "spec: specialized model runtimes" (section
 * "Target package and artifact") plans after groupwise-int weights, read as
 * the public microscaling definition with 32-element blocks:
 *   w[n][k] = e2m1(c[n][k]) * 2^(E[n][k/32] - 127)
 * where an element c is bit 3 sign, bits 2..1 exponent (bias 1; 0 is
 * subnormal: m * 2^-1), bit 0 mantissa, values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6};
 * E is an E8M0 byte, E = 255 is NaN.
 *   x    bf16  [M][K] device
 *   w_q  uint8 [N][K/2] device, elements packed as the int4 codes (k = 2j in
 *        the low nibble of byte j)
 *   w_e  uint8 [N][K/32] device, E8M0 scale bytes
 *   y    [M][N] device, fp32 (Q4_F32) or bf16 (Q4_BF16)
 * M <= 2 takes the matrix-vector kernel.  Where q4_matmul_path(M, N, K) is
 * Q4_PATH_MFMA and K is a multiple of 64, the tiled matrix-core kernel runs,
 * with e2m1 * 2^(E - 129) exact in bf16 and the fp32 sums times 4; otherwise
 * (3 <= M <= 65535 * 32) the few-row matrix-core kernel, in slabs of 32 rows
 * (e2m1 values exact in bf16, scales applied in fp32).
 * M = 0 or N = 0 is a no-op; a larger M is Q4_ERR_SHAPE; K must be a
 * positive multiple of 32.  Every weight enters exactly; sums are fp32.  x,
 * w_q, w_e and y must be 16-byte aligned.  Checks and error behaviour as for
 * q4_matmul. */
Q4_API int32_t q4_mx_matmul(const void *x, const void *w_q, const void *w_e,
                            void *y, int32_t y_dtype,
                            int64_t M, int64_t N, int64_t K, q4_stream_t stream);

/* Device workspace (bytes) that lets q4_mx_matmul_ex cut the tiled path's
 * grid along K (ABI version 6): slices * M * N fp32 partial sums, with the
 * slices q4_matmul_workspace_bytes gives a Q4_PATH_MFMA shape (grids of fewer
 * than 512 tiles, K a multiple of 64).  0 when the call needs none, or for
 * sizes q4_mx_matmul would reject. */
Q4_API size_t q4_mx_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* q4_mx_matmul with an optional workspace (ABI version 6).  workspace ==
 * NULL: exactly q4_mx_matmul.  Otherwise the same contract as q4_matmul_ex's:
 * 16-byte aligned, at least q4_mx_matmul_workspace_bytes(M, N, K) bytes
 * (else Q4_ERR_WORKSPACE, after the tensor NULL and alignment checks),
 * contents on entry do not matter, not shared by calls that may overlap.
 * The slices' fp32 sums are added in slice order: the same result on every
 * run, which can differ from the unsplit call's in the last bits. */
Q4_API int32_t q4_mx_matmul_ex(const void *x, const void *w_q, const void *w_e,
                               void *y, int32_t y_dtype,
                               int64_t M, int64_t N, int64_t K,
                               void *workspace, size_t workspace_bytes,
                               q4_stream_t stream);

/* Measurement helper, not part of the matmul path (ABI version 10): the
 * streaming ceiling a benchmark sets beside the decode kernel's HBM rate.
 * Reads the bytes at src once, 16 bytes per lane and load with
 * non-temporal hints (the decode kernel's width and hint), each wavefront
 * streaming a contiguous stretch with six 1 KB loads in flight, and writes the
 * XOR of what each wavefront read to one word of sink, so that every load
 * is used; the XOR of all of sink is the XOR of every 32-bit word read.
 *   src    device, 16-byte aligned, bytes a positive multiple of 16
 *   sink   uint32 [q4_stream_read_sink_words()] device, fully overwritten
 * Returns Q4_OK or an error code (Q4_ERR_SHAPE for a size that is zero or
 * not a multiple of 16). */
Q4_API int32_t q4_stream_read_sink_words(void);
Q4_API int32_t q4_stream_read(const void *src, size_t bytes, uint32_t *sink,
                              q4_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
