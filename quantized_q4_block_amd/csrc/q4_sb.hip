// q4_sb.hip -- weights with super-block (two-level) scales:
//   w[n,k] = (c[n,k] - 8) * d[n, k/256] * sc[n, k/32]
// with fp16 super-block scales d [N][K/256] and unsigned 8-bit block
// multipliers sc [N][K/32]: the two-level block-scale structure of the
// K-quant profiles that the "Layer Package Repository Spec" names ("Repository
// Identity", "Policy Resolution"), on this library's 4-bit codes.
//
// d * sc has at most 19 significant bits, so every block scale is exact in
// fp32.  The matrix-vector kernel (M <= 2, whole rows up to K = 8192) reads
// d and sc as stored and forms each block scale in fp32 as it uses it.  For
// the other shapes a small kernel writes the fp32 scales into the caller's
// workspace (N * K/32 floats, read back once by the product), then the
// few-row matrix-core kernel or the tiled kernel runs with fp32 block scales
// in place of fp16 ones -- weights exact on every path, as for the base
// format.
#include "../../include/q4.h"
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

// One thread per 256-element super-block: one fp16 scale and eight
// multiplier bytes in (one 8-byte load), eight fp32 block scales out (two
// 16-byte stores).
__global__ __launch_bounds__(256) void sb_expand_kernel(const uint16_t* __restrict__ wd,
                                                        const uint2* __restrict__ wsc,
                                                        float4* __restrict__ s,
                                                        uint32_t n_super) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n_super; i += stride) {
    const float d = fp16_to_f32(wd[i]);
    const uint2 m = wsc[i];
    s[2 * i] = make_float4(d * (float)(m.x & 0xFFu), d * (float)((m.x >> 8) & 0xFFu),
                           d * (float)((m.x >> 16) & 0xFFu), d * (float)(m.x >> 24));
    s[2 * i + 1] = make_float4(d * (float)(m.y & 0xFFu), d * (float)((m.y >> 8) & 0xFFu),
                               d * (float)((m.y >> 16) & 0xFFu), d * (float)(m.y >> 24));
  }
}

size_t sb_scale_bytes(int64_t N, int64_t K) {
  return ((size_t)N * (size_t)(K / 32) * 4 + 255) & ~size_t(255);
}

hipError_t launch_sb_matmul(const uint16_t* x, const uint8_t* wq, const uint16_t* wd,
                            const uint8_t* wsc, void* y, bool y_bf16, int64_t M, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  // matrix-vector shapes whose rows fit the decode kernel read the scales as
  // stored (1.25 instead of 4 bytes per 32 weights, and no expansion)
  if (gemv_norm_fits(M, K)) return launch_gemv_sb(x, wq, wd, wsc, y, y_bf16, M, N, K, stream);
  float* s = static_cast<float*>(workspace);
  // the super-blocks of all rows are consecutive: d [N][K/256] and sc
  // [N][K/32] share the index n * K/256 + j (eight multipliers per j)
  const int64_t n_super = N * (K / 256);
  if (n_super > 0xFFFFFFFFll) return hipErrorInvalidValue;
  int64_t grid = (n_super + 255) / 256;
  if (grid > 65536) grid = 65536;
  sb_expand_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
      wd, reinterpret_cast<const uint2*>(wsc), reinterpret_cast<float4*>(s), (uint32_t)n_super);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the rest of the workspace, if large enough, lets the tiled product cut K
  const size_t sb = sb_scale_bytes(N, K);
  const size_t need = q4_matmul_workspace_bytes(M, N, K);
  float* partial = need > 0 && workspace_bytes >= sb + need
                       ? reinterpret_cast<float*>(static_cast<char*>(workspace) + sb)
                       : nullptr;
  const int32_t path = q4_matmul_path_ex(M, N, K, partial != nullptr);
  if (path == Q4_PATH_MFMA)
    return launch_gemm_f32s(x, wq, s, y, y_bf16, M, N, K, partial, stream);
  // matrix-vector shapes past the LDS kernel's rows (no K slices: the
  // workspace was sized for the matrix-vector path's), and the few-row ones
  return launch_small_f32s(x, wq, s, y, y_bf16, M, N, K,
                           path == Q4_PATH_SMALL ? partial : nullptr, stream);
}

}  // namespace q4
