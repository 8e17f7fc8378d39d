// q4_gemv.hip -- decode path (M <= 8): fused dequant + matrix-vector product.
//
// The quantised GEMM of the T0 kernel tier ("spec: specialized model
// runtimes", sections "Architecture" and "Feasibility gate") at decode
// shapes, where every weight byte is used by at most 8 activation rows and
// the op is bound by streaming W from HBM.  The layer-package spec's
// expert-matmul fixtures ("Layer Package Repository Spec", MoE paragraph
// under "Policy Resolution") measure the same lesson on another GPU: the
// matrix-vector kernel beat the matrix-matrix one about 5x for one token,
// and taking several rows per thread group mattered more than other knobs.
//
// Mapping.  A wavefront owns R consecutive weight rows at a time (grid-stride
// over row groups); lane l owns the 32-element blocks l, l+64, l+128, ... of
// every row, so each row read is one coalesced run of 128-bit loads (one
// block = 16 code bytes = one load per lane).  The activation block a lane
// needs is loaded once per block index and reused for all R rows.
//
// Arithmetic.  Codes become exact fp16 (c - 8) pairs in registers (two
// bitwise ops and one packed fp16 subtract per 4 codes); v_fma_mix_f32
// multiplies each fp16 weight with the fp32 activation and accumulates in
// fp32, so every product x * (c - 8) is exact.  Each 32-element block is
// summed on its own, then scaled by its fp16 scale into the row total; the
// 64 lane totals are combined by a fixed butterfly.  A row of zero weights
// (all codes 8) gives exactly zero.
#include "q4_device.h"
#include "q4_gemv.h"
#include "q4_launch.h"

namespace q4 {

template <int M, int R>
__global__ __launch_bounds__(256) void gemv_kernel(const uint16_t* __restrict__ x,
                                                   const uint8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ ws,
                                                   void* __restrict__ y, int y_bf16,
                                                   int64_t N, int64_t K) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t groups = (N + R - 1) / R;
  const uint16_t* xrow[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xrow[m] = x + m * K;

  for (int64_t g = (int64_t)blockIdx.x * 4 + wave; g < groups; g += (int64_t)gridDim.x * 4) {
    const int64_t n0 = g * R;
    float out[R][M];
    gemv_tile<M, R>(xrow, wq, ws, n0, N - 1, K, out);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (lane == r * M + m && n0 + r < N) {
          if (y_bf16)
            static_cast<uint16_t*>(y)[m * N + n0 + r] = to_bf16(out[r][m]);
          else
            static_cast<float*>(y)[m * N + n0 + r] = out[r][m];
        }
      }
    }
  }
}

template <int M, int R>
static hipError_t launch_m(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                           bool y_bf16, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t groups = (N + R - 1) / R;
  int64_t grid = (groups + 3) / 4;
  if (grid > (1 << 20)) grid = 1 << 20;
  gemv_kernel<M, R><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(x, wq, ws, y, y_bf16 ? 1 : 0,
                                                                   N, K);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1, GemvRows<1>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 2: return launch_m<2, GemvRows<2>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 3: return launch_m<3, GemvRows<3>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 4: return launch_m<4, GemvRows<4>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 5: return launch_m<5, GemvRows<5>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 6: return launch_m<6, GemvRows<6>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 7: return launch_m<7, GemvRows<7>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    case 8: return launch_m<8, GemvRows<8>::R>(x, wq, ws, y, y_bf16, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4
