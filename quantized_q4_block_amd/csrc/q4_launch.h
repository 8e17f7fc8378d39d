// q4_launch.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

// bf16 weights [N][K] -> codes [N][K/2] and fp16 scales [N][K/32].
hipError_t launch_quantize(const uint16_t* w, uint8_t* wq, uint16_t* ws, int64_t N, int64_t K,
                           hipStream_t stream);

hipError_t launch_dequant(const uint8_t* wq, const uint16_t* ws, void* out, bool bf16,
                          int64_t N, int64_t K, hipStream_t stream);

// Few rows (the library uses it for M <= 2): fused dequant + matrix-vector
// product, exact weights.
// partial: NULL, or fp32 scratch of gemv_split_slices(M, K) * M * N floats
// that lets long rows be cut into slices.
hipError_t launch_gemv(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream);

// Slices a row of K is cut into on the matrix-vector path when scratch is
// given (0: never cut).
int64_t gemv_split_slices(int64_t M, int64_t K);

// The RMSNorm prologue fused into the matrix-vector kernel: M <= 2, whole
// rows that fit its LDS staging (gemv_norm_fits).
bool gemv_norm_fits(int64_t M, int64_t K);
hipError_t launch_gemv_norm(const uint16_t* x, const uint16_t* gamma, float eps,
                            const uint8_t* wq, const uint16_t* ws, void* y, bool y_bf16,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);

// RMSNorm prologue + product: the fused matrix-vector kernel where it fits,
// else the normalised activations (bf16) into the first rmsnorm_act_bytes
// of the workspace and the q4_matmul_ex paths on them (K slices when the
// rest of the workspace holds q4_matmul_workspace_bytes).
size_t rmsnorm_act_bytes(int64_t M, int64_t K);
hipError_t launch_rmsnorm_matmul(const uint16_t* x, const uint16_t* gamma, float eps,
                                 const uint8_t* wq, const uint16_t* ws, void* y, bool y_bf16,
                                 int64_t M, int64_t N, int64_t K, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

// Few rows (3 <= M, at most 65535 slabs of 32): exact (c - 8) on the bf16
// matrix cores, block scales applied in fp32; exact weights.
// partial: NULL, or fp32 scratch of small_split_slices(M, N, K) * M * N
// floats that lets a grid of few workgroups be cut along K.
hipError_t launch_small(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                        bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                        hipStream_t stream);

// K slices of the few-row kernel when scratch is given (1: never cut).
int64_t small_split_slices(int64_t M, int64_t N, int64_t K);

// y = sum over s < slices, in order, of partial[s][MN] (fp32 or bf16 y).
hipError_t launch_slice_combine(const float* partial, void* y, bool y_bf16, int64_t MN,
                                int64_t slices, hipStream_t stream);

// 4-bit float block weights (e2m1 elements, E8M0 scales), M <= 2: fused
// dequant + matrix-vector product, exact weights.
hipError_t launch_mx_gemv(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// 4-bit float block weights, M >= 3 (at most 65535 slabs of 32): the few-row
// matrix-core kernel with e2m1 elements in bf16 and E8M0 block scales.
hipError_t launch_small_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                           bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// 4-bit float block weights, many rows, K a multiple of 64: e2m1 * 2^(E-129)
// exact in bf16 in LDS + bf16 MFMA tiles, accumulators times 4; exact weights.
// partial: NULL, or fp32 scratch of gemm_split_slices(M, N, K) * M * N floats.
hipError_t launch_gemm_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                          hipStream_t stream);

// Many rows: exact (c - 8) tiles in LDS + bf16 MFMA, fp32 block scales (exact
// weights); any K that is a multiple of 32.
// partial: NULL, or fp32 scratch of gemm_q4_split_slices(M, N, K) * M * N floats
// that lets a grid of few tiles be cut along K (K a multiple of 64).
hipError_t launch_gemm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream);

// K slices of the tiled kernels when scratch is given (1: never cut): the
// 128-row tiles (the 4-bit float product, and int4 codes up to 128 rows or K
// not a multiple of 64) and the int4 product as launch_gemm runs it.
int64_t gemm_split_slices(int64_t M, int64_t N, int64_t K);
int64_t gemm_q4_split_slices(int64_t M, int64_t N, int64_t K);
// Workspace bytes of the int4 tiled product's tail plan (the last, partly
// filled round of wide tiles cut along K; 0: none).  launch_gemm takes the
// larger of this and the K slices' scratch.
size_t gemm_q4_tail_bytes(int64_t M, int64_t N, int64_t K);

// Expert-routed rows; workspace laid out by moe_workspace_layout.
struct MoeLayout {
  size_t counts, fill, offsets, order, active, num_active, items, num_items, partial, total;
};
MoeLayout moe_workspace_layout(int64_t T, int64_t topk, int64_t E, int64_t N);

hipError_t launch_moe(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                      const int32_t* ids, const float* gates, float* y, int64_t T,
                      int64_t topk, int64_t E, int64_t N, int64_t K, void* workspace,
                      hipStream_t stream);

// launch_moe with the workspace in the library's per-device scratch array
// (at most kMoeScratchBytes of it; hipErrorInvalidValue past that).
constexpr size_t kMoeScratchBytes = size_t(8) << 20;
hipError_t launch_moe_noalloc(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                              const int32_t* ids, const float* gates, float* y, int64_t T,
                              int64_t topk, int64_t E, int64_t N, int64_t K, hipStream_t stream);

// Super-block scales read as stored (fp16 d [N][K/256], 8-bit multipliers
// [N][K/32]), M <= 2, whole rows that gemv_norm_fits, K a multiple of 256.
hipError_t launch_gemv_sb(const uint16_t* x, const uint8_t* wq, const uint16_t* wd,
                          const uint8_t* wsc, void* y, bool y_bf16, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream);

// The int4 kernels with exact fp32 block scales [N][K/32] in place of fp16
// ones (super-block scales expanded): few-row and tiled forms.
hipError_t launch_small_f32s(const uint16_t* x, const uint8_t* wq, const float* ws, void* y,
                             bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                             hipStream_t stream);
hipError_t launch_gemm_f32s(const uint16_t* x, const uint8_t* wq, const float* ws, void* y,
                            bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                            hipStream_t stream);

// Super-block scales: the fp32 block scales into the first sb_scale_bytes of
// the workspace, then the product (K slices when the rest of the workspace
// holds q4_matmul_workspace_bytes).  K a multiple of 256.
size_t sb_scale_bytes(int64_t N, int64_t K);
hipError_t launch_sb_matmul(const uint16_t* x, const uint8_t* wq, const uint16_t* wd,
                            const uint8_t* wsc, void* y, bool y_bf16, int64_t M, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

// Grouped matrix-core product over the expert buckets, for routed rows with
// many pairs per expert (moe_use_grouped: at least kMoeMmMinPairsPerExpert
// pairs per touched expert on average).  The prep tables plus the slab list
// (expert, first pair) that launch_moe_items writes.
#ifndef Q4_MOE_MM_MIN_PAIRS
#define Q4_MOE_MM_MIN_PAIRS 4
#endif
constexpr int64_t kMoeMmMinPairsPerExpert = Q4_MOE_MM_MIN_PAIRS;
struct MoeMmTables {
  const int32_t *counts, *offsets, *order, *items, *num_items;
};
bool moe_use_grouped(int64_t P, int64_t E);
// Pairs per slab of the grouped product.
int moe_mm_rows();
// Slab list length bound for P pairs over A touched experts, slabs of tm.
int64_t moe_mm_max_items(int64_t P, int64_t A, int tm);
hipError_t launch_moe_items(const int32_t* counts, const int32_t* active,
                            const int32_t* num_active, int32_t* items, int32_t* num_items,
                            int tm, hipStream_t stream);
// Plain routed rows: fp32 partial [P][N].
hipError_t launch_moe_mm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                         const MoeMmTables& t, float* partial, int64_t max_items, int64_t topk,
                         int64_t N, int64_t K, hipStream_t stream);
// Gate/up rows of the routed FFN with the SwiGLU in the store: act as bf16
// hi / lo [P][F] (times gates[p] when gates is not NULL).
hipError_t launch_moe_mm_glu(const uint16_t* x, const uint8_t* w13q, const uint16_t* w13s,
                             const MoeMmTables& t, const float* gates, uint16_t* act_hi,
                             uint16_t* act_lo, int64_t max_items, int64_t topk, int64_t F,
                             int64_t H, hipStream_t stream);
// Down rows of the routed FFN over the hi / lo activations: fp32 partial [P][H].
hipError_t launch_moe_mm_down(const uint16_t* act_hi, const uint16_t* act_lo,
                              const uint8_t* w2q, const uint16_t* w2s, const MoeMmTables& t,
                              float* partial, int64_t max_items, int64_t H, int64_t F,
                              hipStream_t stream);

// Routed expert FFN; the MoE layout for N = H followed by the SwiGLU
// outputs act [T * topk][F] (fp32).  H and F at most 8192 (4 stages).
struct MoeFfnLayout {
  MoeLayout base;
  size_t act, total;
};
MoeFfnLayout moe_ffn_workspace_layout(int64_t T, int64_t topk, int64_t E, int64_t H,
                                      int64_t F);
constexpr int64_t kMoeFfnMaxWidth = 8192;

hipError_t launch_moe_ffn(const uint16_t* x, const uint8_t* w13q, const uint16_t* w13s,
                          const uint8_t* w2q, const uint16_t* w2s, const int32_t* ids,
                          const float* gates, float* y, int64_t T, int64_t topk, int64_t E,
                          int64_t H, int64_t F, bool weighted_down, void* workspace,
                          hipStream_t stream);

// The benchmark's streaming ceiling: reads bytes (a multiple of 16) at src
// once with 16-byte non-temporal loads over kStreamReadBlocks workgroups of
// 4 wavefronts, each streaming a contiguous stretch; sink receives
// kStreamReadBlocks * 4 words (the XOR of what each wavefront read).
constexpr int kStreamReadBlocks = 2048;
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace q4
