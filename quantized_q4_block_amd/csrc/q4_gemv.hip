// q4_gemv.hip -- decode path (M <= 2): fused dequant + matrix-vector product.
//
// The quantised GEMM of the T0 kernel tier ("spec: specialized model
// runtimes", sections "Architecture" and "Feasibility gate") at decode
// shapes, where every weight byte is used by one or two activation rows and
// the op is bound by streaming W from HBM (from 3 rows the few-row
// matrix-core kernel is faster).  The layer-package spec's
// expert-matmul fixtures ("Layer Package Repository Spec", MoE paragraph
// under "Policy Resolution") measure the same lesson on another GPU: the
// matrix-vector kernel beat the matrix-matrix one about 5x for one token,
// and taking several rows per thread group mattered more than other knobs.
//
// Two kernels (see q4_gemv.h for the per-wavefront work):
//  * gemv_lds_kernel (rows of at most 4 x 64 blocks, activations within
//    64 KB as fp32) -- one task of 2 rows per wavefront, 8
//    wavefronts per workgroup, compiled per row geometry.  Each wavefront
//    first issues every code and scale load of its task, then the
//    workgroup converts the activations to fp32 in LDS (one conversion per
//    workgroup instead of one per task), so the staging and its barrier run
//    while the weights are in flight.
//  * gemv_glb_kernel -- one task per wavefront, activations read as bf16
//    from global memory (L1/L2 hits); for longer rows.
// Every product x * (c - 8) is exact and each 32-element block is summed on
// its own before its scale is applied, so a row of zero weights (all codes
// 8) gives exactly zero.
#include <type_traits>

#include "q4_device.h"
#include "q4_gemv.h"
#include "q4_launch.h"

namespace q4 {

constexpr int64_t kLdsLimit = 64 * 1024;

template <int M, int R>
__device__ __forceinline__ void store_rows(void* __restrict__ y, int y_bf16, int64_t N,
                                           int64_t n0, const float (&out)[R][M]) {
  if ((threadIdx.x & 63) != 0) return;
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (n0 + r >= N) break;
      if (y_bf16)
        static_cast<uint16_t*>(y)[m * N + n0 + r] = to_bf16(out[r][m]);
      else
        static_cast<float*>(y)[m * N + n0 + r] = out[r][m];
    }
}

// Rows of FULL whole stages plus a leftover stage of kind TAIL (so the row
// geometry, and with it the register budget, is fixed at compile time).
//
// The kernel works on a piece of each row: blocks blk0 .. blk0 + K/32 - 1
// with blk0 = (slice0 + blockIdx.y) * slice_blocks, rows ld_blocks blocks
// apart.  A whole-row call has one slice (blk0 = 0, ld_blocks = K/32) and
// writes y; a split call (long rows, rem < 0) cuts the rows into slices of
// slice_blocks blocks (the last one shorter) that are FULL whole stages
// plus a partial one (TAIL = kWideTail; lanes past the slice's end add
// zero) and writes the fp32 partial sums of slice s to partial[s][M][N],
// which gemv_combine_kernel then adds in slice order.
//
// NORM: the RMSNorm prologue fused into the staging (whole rows only): the
// workgroup also loads the norm weights gamma at its activations' positions
// and stages x * gamma (exact in fp32) instead of x; each wavefront sums the
// squares of its chunks of every activation row in double and leaves the sum
// in LDS before the staging barrier; after it every wavefront adds the eight
// sums in the same fixed order, forms r = 1 / sqrt(sum / K + eps) and
// multiplies its outputs by r, since y = r * sum_k (x gamma)_k w_k.  Every
// workgroup computes the same r; the prologue adds no barrier.
//
// SP: the block scales' storage -- uint16_t (fp16, the format's own) or float
// (exact fp32 scales, e.g. expanded from super-block scales).
template <int M, int FULL, int TAIL, bool NORM = false, typename SP = uint16_t>
__global__ __launch_bounds__(kLdsWaves * 64) void gemv_lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const SP* __restrict__ ws, void* __restrict__ y, int y_bf16, int64_t N, int64_t K,
    int rem, int64_t ld_blocks, int slice0, int slice_blocks, float* __restrict__ partial,
    const uint16_t* __restrict__ gamma = nullptr, float eps = 0.0f,
    const uint16_t* __restrict__ sb_d = nullptr) {
  // SP: the block scales' storage -- uint16_t (fp16), float (exact fp32) or
  // uint8_t (super-block multipliers, with the fp16 super-block scales in
  // sb_d; whole rows only)
  using SC = typename std::conditional<
      std::is_same<SP, float>::value, float,
      typename std::conditional<std::is_same<SP, uint8_t>::value, SbScale, _Float16>::type>::type;
  constexpr int R = kLdsRows;
  constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
  __shared__ float4 xs[M * S * 8 * kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = ((int64_t)blockIdx.x * kLdsWaves + wave) * R;
  const bool live = n0 < N;
  const int64_t nl = live ? n0 : N - 1;
  const int room = (int)((N - 1 - nl) < R ? (N - 1 - nl) : R);
  const int slice = slice0 + (int)blockIdx.y;
  const int64_t blk0 = (int64_t)slice * slice_blocks;
  if (rem < 0) {   // slices of FULL whole stages plus a partial one
    const int64_t left = ld_blocks - blk0;
    const int len = (int)(left < slice_blocks ? left : slice_blocks);
    rem = len - FULL * kWave;
    K = (int64_t)len * kBlock;
  }
  const uint32_t row_bytes = (uint32_t)(ld_blocks * 16), row_sc = (uint32_t)ld_blocks;
  // activation loads, then weight loads; the activations are converted
  // into LDS while the weights are in flight
  XStager<M, S, kLdsWaves * 64> xst;
  xst.load(x + blk0 * kBlock, K, ld_blocks * kBlock);
  XStager<1, S, kLdsWaves * 64> gst;
  if constexpr (NORM) gst.load(gamma, K, 0);
  UpfrontLoads<R, FULL, TAIL, SC> b;
  if constexpr (std::is_same<SC, SbScale>::value)
    upfront_load_sb<R, FULL, TAIL>(b, wq + nl * (int64_t)row_bytes,
                                   sb_d + nl * (int64_t)(row_sc / 8), ws + nl * (int64_t)row_sc,
                                   row_bytes, row_sc, room, rem, lane);
  else
    upfront_load<R, FULL, TAIL>(b, wq + nl * (int64_t)row_bytes + blk0 * 16,
                                ws + nl * (int64_t)row_sc + blk0, row_bytes, row_sc, room, rem,
                                lane, (uint32_t)(ld_blocks - blk0));
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the staging
  xst.pin();
  __shared__ double red[NORM ? M : 1][kLdsWaves];
  if constexpr (NORM) {
    gst.pin();
    double ss[M];
    xst.sum_squares(ss);
    float one[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ss[m] += __shfl_xor(ss[m], off, kWave);
      if (lane == 0) red[m][wave] = ss[m];
      one[m] = 1.0f;
    }
    xst.store_f32_scaled(xs, gst, one);
  } else {
    xst.store_f32(xs);
  }
  __syncthreads();
  // a wavefront past the last row computes on clamped rows and stores
  // nothing (an early exit would let the compiler sink its loads past the
  // barrier)
  float out[R][M];
  upfront_compute<M, R, FULL, TAIL, SC>(b, xs, rem, lane, out);
  if constexpr (NORM) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < kLdsWaves; ++w) t += red[m][w];
      const float r = (float)(1.0 / __builtin_sqrt(t / (double)K + (double)eps));
#pragma unroll
      for (int rr = 0; rr < R; ++rr) out[rr][m] *= r;
    }
  }
  if (!live) return;
  if (partial)
    store_rows<M, R>(partial + (int64_t)slice * M * N, 0, N, n0, out);
  else
    store_rows<M, R>(y, y_bf16, N, n0, out);
}

// y[i] = sum over slices s = 0 .. slices-1, in order, of partial[s][i].
__global__ __launch_bounds__(256) void gemv_combine_kernel(const float* __restrict__ partial,
                                                           void* __restrict__ y, int y_bf16,
                                                           int64_t MN, int slices) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
    const float acc = sum_slices<32>(partial + i, MN, slices);
    if (y_bf16)
      static_cast<uint16_t*>(y)[i] = to_bf16(acc);
    else
      static_cast<float*>(y)[i] = acc;
  }
}

template <int M, int FULL, int TAIL>
static hipError_t launch_lds(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                             int yb, int64_t N, int64_t K, int rem, int64_t ld_blocks,
                             int slice0, int slices, int slice_blocks, float* partial,
                             hipStream_t stream) {
  constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
  if constexpr ((int64_t)M * S * 8 * kWave * 16 > kLdsLimit) {
    return hipErrorInvalidValue;   // never chosen (the caller checks the size)
  } else {
    const int64_t tasks = (N + kLdsRows - 1) / kLdsRows;
    const int64_t grid = (tasks + kLdsWaves - 1) / kLdsWaves;
    if (grid > 0x7FFFFFFF || slices > 65535) return hipErrorInvalidValue;
    gemv_lds_kernel<M, FULL, TAIL>
        <<<dim3((unsigned)grid, (unsigned)slices), dim3(kLdsWaves * 64), 0, stream>>>(
            x, wq, ws, y, yb, N, K, rem, ld_blocks, slice0, slice_blocks, partial);
    return hipGetLastError();
  }
}

// Rows longer than the LDS kernel takes in one piece are cut into slices
// when the caller gives a workspace for the fp32 partial sums: as few
// slices of 65 .. 128 blocks (two stages, the second partial) as cover the
// row, when the last one also gets more than 64 blocks; otherwise slices of
// up to 64 blocks (one stage).
struct SplitPlan {
  int64_t slices = 0;
  int slice_blocks = 0;
  int full = 0;          // whole stages per slice before the partial one
};

static SplitPlan split_plan(int64_t M, int64_t K) {
  SplitPlan p;
  if (M < 1 || M > 2) return p;
  if (x_stages(K) <= kLdsMaxStages && xlds_bytes(M, K) <= kLdsLimit) return p;
  const int64_t bpr = K / kBlock;
  const int64_t ns = (bpr + 2 * kWave - 1) / (2 * kWave);
  const int64_t sb = (bpr + ns - 1) / ns;
  if (sb > kWave && bpr - (ns - 1) * sb > kWave) {
    p.slices = ns;
    p.slice_blocks = (int)sb;
    p.full = 1;
  } else {
    p.slices = (bpr + kWave - 1) / kWave;
    p.slice_blocks = kWave;
    p.full = 0;
  }
  return p;
}

int64_t gemv_split_slices(int64_t M, int64_t K) { return split_plan(M, K).slices; }

// One task of R rows per wavefront, starting at row `row0`; activations
// read from global memory.
template <int M, int R>
__global__ __launch_bounds__(256) void gemv_glb_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ ws,
                                                       void* __restrict__ y, int y_bf16,
                                                       int64_t N, int64_t K, int64_t row0) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = row0 + ((int64_t)blockIdx.x * 4 + wave) * R;
  if (n0 >= N) return;
  const uint16_t* xrow[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xrow[m] = x + m * K;
  float out[R][M];
  gemv_task<M, R>(xrow, wq, ws, n0, N - 1, K, out);
  store_rows<M, R>(y, y_bf16, N, n0, out);
}

template <int M, int R>
static hipError_t launch_m(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                           bool y_bf16, int64_t N, int64_t K, float* partial,
                           hipStream_t stream) {
  static_assert(M >= 1 && M <= 2, "the matrix-vector path takes one or two rows");
  const int yb = y_bf16 ? 1 : 0;
  {
    const int64_t bpr = K / kBlock;
    if (x_stages(K) <= kLdsMaxStages && xlds_bytes(M, K) <= kLdsLimit) {
      const int rem = row_leftover(K);
      return dispatch_row_geometry(K, [&](auto full, auto tail) {
        return launch_lds<M, decltype(full)::value, decltype(tail)::value>(
            x, wq, ws, y, yb, N, K, rem, bpr, 0, 1, 0, nullptr, stream);
      });
    }
    if (partial) {
      const SplitPlan sp = split_plan(M, K);
      const int64_t slices = sp.slices;
      hipError_t e =
          sp.full == 1
              ? launch_lds<M, 1, kWideTail>(x, wq, ws, y, yb, N, 0, -1, bpr, 0, (int)slices,
                                            sp.slice_blocks, partial, stream)
              : launch_lds<M, 0, kWideTail>(x, wq, ws, y, yb, N, 0, -1, bpr, 0, (int)slices,
                                            sp.slice_blocks, partial, stream);
      if (e != hipSuccess) return e;
      const int64_t MN = (int64_t)M * N;
      int64_t grid = (MN + 255) / 256;
      if (grid > 65536) grid = 65536;
      gemv_combine_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(partial, y, yb, MN,
                                                                          (int)slices);
      return hipGetLastError();
    }
  }
  {
    const int64_t tasks = (N + R - 1) / R;
    const int64_t grid = (tasks + 3) / 4;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemv_glb_kernel<M, R><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
        x, wq, ws, y, yb, N, K, 0);
  }
  return hipGetLastError();
}

// RMSNorm fused into the LDS kernel (M <= 2, whole rows of at most
// kLdsMaxStages stages whose activations fit the LDS).
bool gemv_norm_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= 2 && x_stages(K) <= kLdsMaxStages && xlds_bytes(M, K) <= kLdsLimit;
}

template <int M>
static hipError_t launch_norm_m(const uint16_t* x, const uint16_t* gamma, float eps,
                                const uint8_t* wq, const uint16_t* ws, void* y, bool y_bf16,
                                int64_t N, int64_t K, hipStream_t stream) {
  const int rem = row_leftover(K);
  const int64_t bpr = K / kBlock;
  return dispatch_row_geometry(K, [&](auto full, auto tail) {
    constexpr int FULL = decltype(full)::value, TAIL = decltype(tail)::value;
    const int64_t tasks = (N + kLdsRows - 1) / kLdsRows;
    const int64_t grid = (tasks + kLdsWaves - 1) / kLdsWaves;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemv_lds_kernel<M, FULL, TAIL, true><<<dim3((unsigned)grid), dim3(kLdsWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, N, K, rem, bpr, 0, 0, nullptr, gamma, eps);
    return hipGetLastError();
  });
}

hipError_t launch_gemv_norm(const uint16_t* x, const uint16_t* gamma, float eps,
                            const uint8_t* wq, const uint16_t* ws, void* y, bool y_bf16,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (!gemv_norm_fits(M, K)) return hipErrorInvalidValue;
  if (M == 1) return launch_norm_m<1>(x, gamma, eps, wq, ws, y, y_bf16, N, K, stream);
  return launch_norm_m<2>(x, gamma, eps, wq, ws, y, y_bf16, N, K, stream);
}

// The matrix-vector kernel with super-block scales read as stored (fp16 d
// per 256 k, 8-bit multipliers per 32 k; M <= 2, whole rows that fit its LDS
// staging: gemv_norm_fits, K a multiple of 256).
template <int M>
static hipError_t launch_sb_m(const uint16_t* x, const uint8_t* wq, const uint16_t* wd,
                              const uint8_t* wsc, void* y, bool y_bf16, int64_t N, int64_t K,
                              hipStream_t stream) {
  const int rem = row_leftover(K);
  const int64_t bpr = K / kBlock;
  return dispatch_row_geometry(K, [&](auto full, auto tail) {
    constexpr int FULL = decltype(full)::value, TAIL = decltype(tail)::value;
    const int64_t tasks = (N + kLdsRows - 1) / kLdsRows;
    const int64_t grid = (tasks + kLdsWaves - 1) / kLdsWaves;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemv_lds_kernel<M, FULL, TAIL, false, uint8_t>
        <<<dim3((unsigned)grid), dim3(kLdsWaves * 64), 0, stream>>>(
            x, wq, wsc, y, y_bf16 ? 1 : 0, N, K, rem, bpr, 0, 0, nullptr, nullptr, 0.0f, wd);
    return hipGetLastError();
  });
}

hipError_t launch_gemv_sb(const uint16_t* x, const uint8_t* wq, const uint16_t* wd,
                          const uint8_t* wsc, void* y, bool y_bf16, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
  if (!gemv_norm_fits(M, K) || K % 256 != 0) return hipErrorInvalidValue;
  if (M == 1) return launch_sb_m<1>(x, wq, wd, wsc, y, y_bf16, N, K, stream);
  return launch_sb_m<2>(x, wq, wd, wsc, y, y_bf16, N, K, stream);
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream) {
  // one or two rows; more take the few-row matrix-core kernel
  switch (M) {
    case 1: return launch_m<1, GemvRows<1>::R>(x, wq, ws, y, y_bf16, N, K, partial, stream);
    case 2: return launch_m<2, GemvRows<2>::R>(x, wq, ws, y, y_bf16, N, K, partial, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4
