// q4_norm.hip -- the quantised matmul behind an RMSNorm prologue:
//   y = RMSNorm(x) . dequant(W)^T,  RMSNorm(x)[m,k] = x[m,k] * gamma[k] * r_m,
//   r_m = 1 / sqrt(mean_k x[m,k]^2 + eps).
//
// The specialised-runtime spec's first measured kernel is "one quantized GEMM
// plus fused RMSNorm" ("spec: specialized model runtimes", section
// "Feasibility gate"; Phase 1 of "Development sequence").  Two forms:
//  * decode (M <= 2, whole rows that fit the LDS kernel): the norm is fused
//    into the matrix-vector kernel (gemv_lds_kernel with NORM): x * gamma is
//    staged in fp32 and each output is multiplied by r; no extra launch;
//  * otherwise: rmsnorm_rows_kernel writes the normalised activations as bf16
//    (the matrix cores' operand type) into the caller's workspace, and the
//    product runs on them through the same paths as q4_matmul_ex.  Reading
//    the activations once more costs M * K * 4 bytes, under 1 % of a
//    prefill-sized product.
// Sums of squares are taken in double (exact squares, no overflow for any
// bf16 input) and reduced in a fixed order: results are run-to-run identical.
#include <math.h>

#include "../../include/q4.h"
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {
constexpr int kNormThreads = 256;
}

// One workgroup per activation row; 8 elements (16 bytes) per thread step.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_rows_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, float eps,
    uint16_t* __restrict__ out, int64_t K) {
  __shared__ double red[kNormThreads / kWave];
  __shared__ float rs;
  const int64_t m = blockIdx.x;
  const uint16_t* xr = x + m * K;
  uint16_t* orow = out + m * K;
  double ss = 0.0;
  for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += kNormThreads * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const double a = bf16_lo(w[h]), b = bf16_hi(w[h]);
      ss = __builtin_fma(a, a, ss);
      ss = __builtin_fma(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) t += red[w];
    rs = (float)(1.0 / __builtin_sqrt(t / (double)K + (double)eps));
  }
  __syncthreads();
  const float r = rs;
  for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += kNormThreads * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + k);
    const uint4 g = *reinterpret_cast<const uint4*>(gamma + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = pack_bf16x2(bf16_lo(w[h]) * bf16_lo(gw[h]) * r, bf16_hi(w[h]) * bf16_hi(gw[h]) * r);
    *reinterpret_cast<uint4*>(orow + k) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

size_t rmsnorm_act_bytes(int64_t M, int64_t K) {
  return ((size_t)M * (size_t)K * 2 + 255) & ~size_t(255);
}

hipError_t launch_rmsnorm_matmul(const uint16_t* x, const uint16_t* gamma, float eps,
                                 const uint8_t* wq, const uint16_t* ws, void* y, bool y_bf16,
                                 int64_t M, int64_t N, int64_t K, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (gemv_norm_fits(M, K))
    return launch_gemv_norm(x, gamma, eps, wq, ws, y, y_bf16, M, N, K, stream);
  if (M > 0x7FFFFFFF) return hipErrorInvalidValue;
  uint16_t* xn = static_cast<uint16_t*>(workspace);
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3((unsigned)M), dim3(kNormThreads), 0, stream, x,
                     gamma, eps, xn, K);
  const hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  // the rest of the workspace, if large enough, lets the product cut K
  const size_t act = rmsnorm_act_bytes(M, K);
  const size_t need = q4_matmul_workspace_bytes(M, N, K);
  float* partial = need > 0 && workspace_bytes >= act + need
                       ? reinterpret_cast<float*>(static_cast<char*>(workspace) + act)
                       : nullptr;
  switch (q4_matmul_path_ex(M, N, K, partial != nullptr)) {
    case Q4_PATH_GEMV: return launch_gemv(xn, wq, ws, y, y_bf16, M, N, K, partial, stream);
    case Q4_PATH_SMALL: return launch_small(xn, wq, ws, y, y_bf16, M, N, K, partial, stream);
    default: return launch_gemm(xn, wq, ws, y, y_bf16, M, N, K, partial, stream);
  }
}

}  // namespace q4
