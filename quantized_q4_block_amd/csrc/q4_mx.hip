// q4_mx.hip -- 4-bit float block weights (e2m1 elements, one E8M0 scale per
// 32 k): fused dequant + matrix-vector product for decode (M <= 2; from 3
// rows on q4_small.hip's matrix-core kernel takes the format).
//
// The specialised-runtime spec ("spec: specialized model runtimes", section
// "Target package and artifact") plans a 4-bit float block format after the
// groupwise-int weights.  The format here is the public microscaling reading
// with 32-element blocks: element bits s e e m (bit 3 sign, exponent bias 1,
// exponent 0 subnormal), value e2m1(c) * 2^(E - 127), E = 255 NaN.  Elements
// are packed like the int4 codes: k = 2j in the low nibble of byte j.
//
// Work split as in the int4 matrix-vector kernel (q4_gemv.h): a task is R
// rows per wavefront, lane l owns the blocks l, l+64, ... of every row, and a
// leftover stage of at most 32 blocks is split between the half-waves.  Two
// kernels, as for the int4 codes:
//  * mx_lds_kernel (M <= 4, rows of at most 4 stages): 2 rows per wavefront,
//    8 wavefronts per workgroup; every code and scale load of a task is
//    issued up front and the workgroup stages the activations as fp32 in LDS
//    while they are in flight;
//  * mx_gemv_kernel (longer rows): activations read as bf16 through L1/L2,
//    one stage ahead of the math.
//
// Arithmetic per byte of elements: one v_cvt_scalef32_pk_f32_fp4 (scale 1)
// gives the two elements as exact fp32 values (at most 2 significant bits),
// two fmas multiply them by fp32 activations (exact products, fp32 sums); the
// block's power of two is applied to its 32-term partial with one fma.
#include "q4_device.h"
#include "q4_gemv.h"
#include "q4_launch.h"

namespace q4 {

namespace {

// acc[r][m] += 2^(E_r - 127) * sum over one block of x[m] * e2m1(c[r]).
template <int M, int RR>
__device__ __forceinline__ void mx_block_rows(const uint4 (&c)[RR], const uint32_t (&e)[RR],
                                              const uint4 (&xd)[M][4], float (&acc)[RR][M]) {
  float part[RR][M];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) part[r][m] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {       // dword i: elements 8i .. 8i+7
    float xv[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 d = xd[m][i];
      xv[m][0] = bf16_lo(d.x); xv[m][1] = bf16_hi(d.x);
      xv[m][2] = bf16_lo(d.y); xv[m][3] = bf16_hi(d.y);
      xv[m][4] = bf16_lo(d.z); xv[m][5] = bf16_hi(d.z);
      xv[m][6] = bf16_lo(d.w); xv[m][7] = bf16_hi(d.w);
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const uint32_t d = i == 0 ? c[r].x : i == 1 ? c[r].y : i == 2 ? c[r].z : c[r].w;
      // byte b holds elements 8i + 2b (low nibble) and 8i + 2b + 1
      f32x2v w[4];
      w[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
      w[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
      w[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
      w[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = part[r][m];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          a = __builtin_fmaf(w[b][0], xv[m][2 * b], a);
          a = __builtin_fmaf(w[b][1], xv[m][2 * b + 1], a);
        }
        part[r][m] = a;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    const float s = e8m0_to_f32(e[r]);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(s, part[r][m], acc[r][m]);
  }
}

template <int M> struct MxRows {
  static constexpr int R = M <= 2 ? 4 : 2;
};

constexpr int kMxWaves = 4;

// One task of R rows per wavefront (rows n0 .. n0+R-1); loads one stage ahead.
template <int M, int R>
__global__ __launch_bounds__(kMxWaves * 64) void mx_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ we, void* __restrict__ y, int y_bf16, int64_t N, int64_t K) {
  static_assert(R % 2 == 0, "rows per task must be even");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = ((int64_t)blockIdx.x * kMxWaves + wave) * R;
  if (n0 >= N) return;
  const int64_t n_last = N - 1;
  const StagePlan sp(K, lane);
  const int64_t row_bytes = K / 2;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  struct Buf {
    uint4 c[R];
    uint32_t e[R];
    uint4 xd[M][4];
  };
  // codes, scale bytes and activations of stage st (rows past n_last read
  // row n_last; their results are not stored)
  auto load = [&](int64_t st, Buf& b) {
    const int64_t blk = sp.block(st, lane);
    const bool last = st >= sp.full;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = last ? tail_row<R>(sp, r) : r;
      const int64_t n = n0 + row < n_last ? n0 + row : n_last;
      b.c[r] = *reinterpret_cast<const uint4*>(wq + n * row_bytes + blk * 16);
      b.e[r] = we[n * sp.bpr + blk];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* p = reinterpret_cast<const uint4*>(x + m * K + blk * kBlock);
#pragma unroll
      for (int q = 0; q < 4; ++q) b.xd[m][q] = p[q];
    }
  };
  auto compute = [&](int64_t st, const Buf& b) {
    if (st < sp.full) {
      mx_block_rows<M, R>(b.c, b.e, b.xd, acc);
    } else if (sp.split) {
      constexpr int H = R / 2;
      uint4 c[H];
      uint32_t e[H];
      float t[H][M];
#pragma unroll
      for (int r = 0; r < H; ++r) {
        c[r] = b.c[r];
        e[r] = b.e[r];
#pragma unroll
        for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
      }
      mx_block_rows<M, H>(c, e, b.xd, t);
      add_tail_split<M, R>(sp, t, acc);
    } else {
      float t[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
      mx_block_rows<M, R>(b.c, b.e, b.xd, t);
      add_tail<M, R>(sp, t, acc);
    }
  };

  Buf A, B;
  if (sp.S > 0) load(0, A);
  for (int64_t st = 0; st < sp.S; st += 2) {
    if (st + 1 < sp.S) load(st + 1, B);
    compute(st, A);
    if (st + 1 < sp.S) {
      if (st + 2 < sp.S) load(st + 2, A);
      compute(st + 1, B);
    }
  }
  float out[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) out[r][m] = wave_total(acc[r][m]);
  if (lane != 0) return;
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

// Rows of FULL whole stages plus a leftover stage of kind TAIL, activations
// staged in LDS (the int4 decode kernel's scheme with E8M0 scale bytes).
template <int M, int FULL, int TAIL>
__global__ __launch_bounds__(kLdsWaves * 64) void mx_lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ we, void* __restrict__ y, int y_bf16, int64_t N, int64_t K,
    int rem) {
  constexpr int R = kLdsRows;
  constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
  __shared__ float4 xs[M * S * 8 * kWave];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = ((int64_t)blockIdx.x * kLdsWaves + wave) * R;
  const bool live = n0 < N;
  const int64_t nl = live ? n0 : N - 1;
  const int room = (int)((N - 1 - nl) < R ? (N - 1 - nl) : R);
  const uint32_t row_bytes = (uint32_t)(K / 2), row_sc = (uint32_t)(K / kBlock);
  XStager<M, S, kLdsWaves * 64> xst;
  xst.load(x, K, K);
  UpfrontLoads<R, FULL, TAIL, uint8_t> b;
  upfront_load<R, FULL, TAIL>(b, wq + nl * (int64_t)row_bytes, we + nl * (int64_t)row_sc,
                              row_bytes, row_sc, room, rem, lane, row_sc);
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the staging
  xst.pin();
  xst.store_f32(xs);
  __syncthreads();
  // a wavefront past the last row computes on clamped rows and stores nothing
  float out[R][M];
  upfront_compute<M, R, FULL, TAIL, uint8_t>(b, xs, rem, lane, out);
  if (!live || lane != 0) return;
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

template <int M>
hipError_t launch_mx_m(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                       bool y_bf16, int64_t N, int64_t K, hipStream_t stream) {
  if constexpr (M <= 4) {
    if (x_stages(K) <= kLdsMaxStages && xlds_bytes(M, K) <= 64 * 1024) {
      const int rem = row_leftover(K);
      const int64_t tasks = (N + kLdsRows - 1) / kLdsRows;
      const int64_t grid = (tasks + kLdsWaves - 1) / kLdsWaves;
      if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
      return dispatch_row_geometry(K, [&](auto full, auto tail) {
        constexpr int FULL = decltype(full)::value, TAIL = decltype(tail)::value;
        constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
        if constexpr ((int64_t)M * S * 8 * kWave * 16 > 64 * 1024) {
          return hipErrorInvalidValue;   // never chosen (checked above)
        } else {
          mx_lds_kernel<M, FULL, TAIL><<<dim3((unsigned)grid), dim3(kLdsWaves * 64), 0, stream>>>(
              x, wq, we, y, y_bf16 ? 1 : 0, N, K, rem);
          return hipGetLastError();
        }
      });
    }
  }
  constexpr int R = MxRows<M>::R;
  const int64_t tasks = (N + R - 1) / R;
  const int64_t grid = (tasks + kMxWaves - 1) / kMxWaves;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  mx_gemv_kernel<M, R><<<dim3((unsigned)grid), dim3(kMxWaves * 64), 0, stream>>>(
      x, wq, we, y, y_bf16 ? 1 : 0, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemv(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (M) {
    case 1: return launch_mx_m<1>(x, wq, we, y, y_bf16, N, K, stream);
    case 2: return launch_mx_m<2>(x, wq, we, y, y_bf16, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4
