// q4_gemv.h -- the wavefront matrix-vector tile shared by the dense decode
// kernel and the expert-routed kernel.
#pragma once

#include "q4_device.h"

namespace q4 {

// Rows per wavefront task for M activation rows: enough rows that one
// activation load feeds several weight rows, few enough that R * M
// accumulators (and R * M <= 64 storing lanes) fit.
template <int M> struct GemvRows { static constexpr int R = M == 1 ? 8 : (M <= 4 ? 4 : 2); };

// Dot products of M activation rows with R consecutive weight rows
// n0 .. n0+R-1 of one weight matrix.  Rows past n_last are read as row
// n_last (in bounds) and their results must be discarded by the caller.
// Returns the totals in every lane.  Must be called by all 64 lanes of the
// wavefront with the same arguments.
//
// Per lane and block: one 128-bit code load and one fp16 scale per row, one
// 128-bit activation load per 8 elements per activation row (shared by the
// R rows), then for each dword of codes 9 integer/fp16 ops and 8 fp32 fused
// multiply-adds per activation row.
template <int M, int R>
__device__ __forceinline__ void gemv_tile(const uint16_t* const (&xrow)[M],
                                          const uint8_t* __restrict__ wq,
                                          const uint16_t* __restrict__ ws, int64_t n0,
                                          int64_t n_last, int64_t K, float (&out)[R][M]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t bpr = K / kBlock;   // blocks per row
  const int64_t row_bytes = K / 2;
  const uint8_t* wrow[R];
  const uint16_t* srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t n = (n0 + r < n_last) ? n0 + r : n_last;
    wrow[r] = wq + n * row_bytes;
    srow[r] = ws + n * bpr;
  }
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  for (int64_t b = lane; b < bpr; b += kWave) {
    uint4 codes[R];
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      codes[r] = *reinterpret_cast<const uint4*>(wrow[r] + b * 16);
      s[r] = fp16_to_f32(srow[r][b]);
    }
    float part[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) part[r][m] = 0.0f;

#pragma unroll
    for (int i = 0; i < 4; ++i) {       // dword i: elements 8i .. 8i+7
      float xv[M][8];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 xd = *reinterpret_cast<const uint4*>(xrow[m] + b * kBlock + 8 * i);
        xv[m][0] = bf16_lo(xd.x); xv[m][1] = bf16_hi(xd.x);
        xv[m][2] = bf16_lo(xd.y); xv[m][3] = bf16_hi(xd.y);
        xv[m][4] = bf16_lo(xd.z); xv[m][5] = bf16_hi(xd.z);
        xv[m][6] = bf16_lo(xd.w); xv[m][7] = bf16_hi(xd.w);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t d = i == 0 ? codes[r].x : i == 1 ? codes[r].y : i == 2 ? codes[r].z : codes[r].w;
        half2v p[4];
        codes_to_half_pairs(d, p);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = part[r][m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a = __builtin_fmaf((float)p[j][0], xv[m][j], a);      // element 8i + j
            a = __builtin_fmaf((float)p[j][1], xv[m][j + 4], a);  // element 8i + j + 4
          }
          part[r][m] = a;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(s[r], part[r][m], acc[r][m]);
  }

#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) out[r][m] = wave_sum(acc[r][m]);
}

}  // namespace q4
