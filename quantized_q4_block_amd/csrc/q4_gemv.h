// q4_gemv.h -- wavefront matrix-vector kernels shared by the dense decode
// kernel and the expert-routed kernel.
//
// A task is R consecutive weight rows n0 .. n0+R-1 against M activation rows.
// Lane l owns the 32-element blocks l, l+64, l+128, ... of every row of the
// task ("stages"), so each row read is one coalesced run of 128-bit loads
// (one block = 16 code bytes).  When K/32 is not a multiple of 64 and the
// leftover r <= 32 blocks would leave half the lanes idle, the two
// half-waves split the task's rows for that last stage instead: lanes 0..31
// take the leftover blocks of the first R/2 rows, lanes 32..63 those of the
// last R/2 rows, so every lane does the same work.
//
// Arithmetic per block and row: 4 dwords of codes -> 16 exact fp16 (c - 8)
// pairs (one shift, four v_and_or_b32, four v_pk_add_f16 per dword), one
// v_fma_mix_f32 per element and activation row (fp16 weight x fp32
// activation, fp32 accumulate: every product exact), then one fma with the
// block's fp16 scale into the row total.  The 64 lane totals are summed with
// DPP row operations in a fixed order.  Lanes or slots outside the leftover
// blocks add exactly nothing (their contribution is selected away, so even a
// non-finite activation cannot leak in).
#pragma once

#include <type_traits>

#include "q4_device.h"

namespace q4 {

// Rows per wavefront task for M activation rows.
#ifndef Q4_GEMV_R_SMALL
#define Q4_GEMV_R_SMALL 4
#endif
#ifndef Q4_GEMV_R_LARGE
#define Q4_GEMV_R_LARGE 2
#endif
template <int M> struct GemvRows {
  static constexpr int R = M <= 2 ? Q4_GEMV_R_SMALL : Q4_GEMV_R_LARGE;
};

// One DPP move of a float: lanes in ROW_MASK rows read the lane CTRL picks;
// other rows read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float a) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), CTRL,
                                                               ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wavefront with DPP row ops; the total lands in
// lanes 48..63.  Fixed order, so the result is deterministic.
__device__ __forceinline__ float dpp_wave_sum(float v) {
  v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp_f<0x141, 0xF>(v);  // row_half_mirror: 8 lanes
  v += dpp_f<0x140, 0xF>(v);  // row_mirror: 16 lanes (a row)
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Wave-uniform total of a per-lane value.
__device__ __forceinline__ float wave_total(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dpp_wave_sum(v)), 63));
}

// Stage geometry of a row of K elements (see the file comment).
struct StagePlan {
  int64_t bpr, full, S;  // blocks per row, full stages, stages
  int rem;               // leftover blocks per row
  bool split;            // leftover stage split between the half-waves
  int sub;               // this lane's leftover block (within the last stage)
  bool tail_ok;          // this lane has a leftover block
  int half;              // 0: lanes 0..31, 1: lanes 32..63 (split only)
  int64_t tail_b;        // block index this lane reads in the leftover stage
  __device__ __forceinline__ StagePlan(int64_t K, int lane) {
    bpr = K / kBlock;
    full = bpr / kWave;
    rem = (int)(bpr % kWave);
    split = rem > 0 && rem <= kWave / 2;
    S = full + (rem > 0 ? 1 : 0);
    sub = split ? (lane & 31) : lane;
    tail_ok = sub < rem;
    half = split ? (lane >> 5) : 0;
    tail_b = full * kWave + (tail_ok ? sub : 0);
  }
  __device__ __forceinline__ int64_t block(int64_t st, int lane) const {
    return st < full ? st * kWave + lane : tail_b;
  }
};

// ---------------------------------------------------------------------------
// Block arithmetic.

// acc[r][m] += s[r] * sum over one block of x[m] * (c[r] - 8), activations
// given as bf16 (8 per uint4, converted here).
template <int M, int RR>
__device__ __forceinline__ void block_rows_bf16(const CodeUnpacker& unpack, const uint4 (&c)[RR],
                                                const _Float16 (&s)[RR], const uint4 (&xd)[M][4],
                                                float (&acc)[RR][M]) {
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
      half2v p[4];
      unpack(d, p);
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
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf((float)s[r], part[r][m], acc[r][m]);
}

// The same with fp32 activations xv[m][k], k = 0..31 within the block.
template <int M, int RR, typename SC>
__device__ __forceinline__ void block_rows_f32(const CodeUnpacker& unpack, const uint4 (&c)[RR],
                                               const SC (&s)[RR], const float (&xv)[M][32],
                                               float (&acc)[RR][M]) {
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = i == 0 ? c[r].x : i == 1 ? c[r].y : i == 2 ? c[r].z : c[r].w;
      half2v p[4];
      unpack(d, p);
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          part[m] = __builtin_fmaf((float)p[j][0], xv[m][8 * i + j], part[m]);
          part[m] = __builtin_fmaf((float)p[j][1], xv[m][8 * i + j + 4], part[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf((float)s[r], part[m], acc[r][m]);
  }
}

// 4-bit float blocks: acc[r][m] += s[r] * sum over one block of
// x[m] * e2m1(c[r]), fp32 activations xv[m][k], k = 0..31 within the block,
// s[r] the block's power of two as fp32.  Each byte of elements becomes two
// exact fp32 values with one v_cvt_scalef32_pk_f32_fp4 (scale 1; the low
// nibble is the first value).
template <int M, int RR>
__device__ __forceinline__ void mx_block_rows_f32(const uint4 (&c)[RR], const float (&s)[RR],
                                                  const float (&xv)[M][32], float (&acc)[RR][M]) {
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = i == 0 ? c[r].x : i == 1 ? c[r].y : i == 2 ? c[r].z : c[r].w;
      f32x2v w[4];
      w[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
      w[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
      w[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
      w[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          part[m] = __builtin_fmaf(w[b][0], xv[m][8 * i + 2 * b], part[m]);
          part[m] = __builtin_fmaf(w[b][1], xv[m][8 * i + 2 * b + 1], part[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(s[r], part[m], acc[r][m]);
  }
}

// Leftover-stage epilogue (not split): contributions t, computed from raw
// loads, are added only by lanes that own a leftover block.
template <int M, int R>
__device__ __forceinline__ void add_tail(const StagePlan& sp, const float (&t)[R][M],
                                         float (&acc)[R][M]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] += sp.tail_ok ? t[r][m] : 0.0f;
}

// Split leftover stage: slot j of half h is row h*H + j, so row r takes
// slot r % H of the half that owns it, and only from lanes with a block.
template <int M, int R>
__device__ __forceinline__ void add_tail_split(const StagePlan& sp, const float (&t)[R / 2][M],
                                               float (&acc)[R][M]) {
  constexpr int H = R / 2;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const bool owns = r < H ? sp.half == 0 : sp.half == 1;
      acc[r][m] += (sp.tail_ok && owns) ? t[r % H][m] : 0.0f;
    }
}

// Row (relative to the task) that slot r of this lane reads in the
// leftover stage.  Split: slots 0..H-1 hold this half's rows; the other
// slots repeat a valid row and are never used.
template <int R>
__device__ __forceinline__ int64_t tail_row(const StagePlan& sp, int r) {
  constexpr int H = R / 2;
  return sp.split ? sp.half * H + (r % H) : r;
}

// ---------------------------------------------------------------------------
// Code and scale loads through buffer descriptors (buffer_rsrc).
// aux = 2: the non-temporal hint (each weight byte is used once)
__device__ __forceinline__ uint4 buffer_codes(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                              uint32_t soff) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v =
      __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buffer_scale(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                             uint32_t soff, _Float16& s) {
  s = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 2));
}
__device__ __forceinline__ void buffer_scale(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                             uint32_t soff, uint8_t& s) {
  s = __builtin_amdgcn_raw_buffer_load_b8(rs, voff, soff, 2);
}
__device__ __forceinline__ void buffer_scale(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                             uint32_t soff, float& s) {
  s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 2));
}

// ---------------------------------------------------------------------------
// Activations in LDS as fp32 (exact from bf16), laid out [m][stage][chunk q]
// [lane] in 16-byte units, chunk q = elements 4q .. 4q+3 of the block, so
// that in a stage consecutive lanes read consecutive 16 bytes (no bank
// conflicts).  Positions past K hold 0.
__host__ __device__ __forceinline__ int64_t x_stages(int64_t K) {
  return (K / kBlock + kWave - 1) / kWave;
}
__host__ __device__ __forceinline__ int64_t xlds_bytes(int64_t M, int64_t K) {
  return M * x_stages(K) * 8 * kWave * 16;
}

// Copies the M activation rows into that layout (whole workgroup
// of THREADS threads, S stages per row), in two steps so that a kernel can
// issue the activation loads before its weight loads and convert them
// while the weights are in flight: the memory counter waits for loads in
// issue order, so data loaded first can be used without waiting for the
// rest.  Each thread holds whole 8-element chunks.
template <int M, int S, int THREADS>
struct XStager {
  static constexpr int kRowChunks = S * 4 * kWave;   // 8-element chunks per row
  static constexpr int kPer = (kRowChunks + THREADS - 1) / THREADS;
  uint4 d[M][kPer];

  // x: row 0 of the activations at the first element of the row piece; K:
  // length of the piece; ldx: distance between rows (elements).  Raw buffer
  // loads whose extent is the row piece: a chunk past K (or a thread past
  // the row's chunks) reads zero, with no address clamp or mask.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ x, int64_t K, int64_t ldx) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(x + m * ldx, (uint32_t)K * 2u);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = i * THREADS + (int)threadIdx.x;
        const int st = c >> 8, q = (c >> 6) & 3, l = c & 63;
        const uint32_t k = (uint32_t)((st * kWave + l) * kBlock + q * 8);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t v =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, k * 2u, 0, 0));
        d[m][i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  // Marks the loaded activations as used here, so that the compiler cannot
  // sink a load into the conditional store of a thread's last chunk (that
  // load would then be issued after, and wait for, the weight loads).
  __device__ __forceinline__ void pin() const {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        asm volatile("" ::"v"(d[m][i].x), "v"(d[m][i].y), "v"(d[m][i].z), "v"(d[m][i].w));
  }
  __device__ __forceinline__ void store_f32(float4* __restrict__ xs) const {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = i * THREADS + (int)threadIdx.x;
        if (kRowChunks % THREADS != 0 && c >= kRowChunks) break;
        const int st = c >> 8, q = (c >> 6) & 3, l = c & 63;
        float4* row = xs + m * (2 * kRowChunks) + st * 8 * kWave + l;
        row[(2 * q) * kWave] = make_float4(bf16_lo(d[m][i].x), bf16_hi(d[m][i].x),
                                           bf16_lo(d[m][i].y), bf16_hi(d[m][i].y));
        row[(2 * q + 1) * kWave] = make_float4(bf16_lo(d[m][i].z), bf16_hi(d[m][i].z),
                                               bf16_lo(d[m][i].w), bf16_hi(d[m][i].w));
      }
  }
  // This thread's share of sum_k x[m][k]^2, in double (each square is exact
  // there, and the sum cannot overflow for any bf16 input).
  __device__ __forceinline__ void sum_squares(double (&ss)[M]) const {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      ss[m] = 0.0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t w[4] = {d[m][i].x, d[m][i].y, d[m][i].z, d[m][i].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const double a = bf16_lo(w[h]), b = bf16_hi(w[h]);
          ss[m] = __builtin_fma(a, a, ss[m]);
          ss[m] = __builtin_fma(b, b, ss[m]);
        }
      }
    }
  }
  // store_f32 of x[m][k] * g[k] * r[m] (g: a one-row stager loaded at the
  // same positions), each product in fp32.
  __device__ __forceinline__ void store_f32_scaled(float4* __restrict__ xs,
                                                   const XStager<1, S, THREADS>& g,
                                                   const float (&r)[M]) const {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = i * THREADS + (int)threadIdx.x;
        if (kRowChunks % THREADS != 0 && c >= kRowChunks) break;
        const int st = c >> 8, q = (c >> 6) & 3, l = c & 63;
        float4* row = xs + m * (2 * kRowChunks) + st * 8 * kWave + l;
        const uint4 v = d[m][i], gv = g.d[0][i];
        const float rm = r[m];
        row[(2 * q) * kWave] =
            make_float4(bf16_lo(v.x) * bf16_lo(gv.x) * rm, bf16_hi(v.x) * bf16_hi(gv.x) * rm,
                        bf16_lo(v.y) * bf16_lo(gv.y) * rm, bf16_hi(v.y) * bf16_hi(gv.y) * rm);
        row[(2 * q + 1) * kWave] =
            make_float4(bf16_lo(v.z) * bf16_lo(gv.z) * rm, bf16_hi(v.z) * bf16_hi(gv.z) * rm,
                        bf16_lo(v.w) * bf16_lo(gv.w) * rm, bf16_hi(v.w) * bf16_hi(gv.w) * rm);
      }
  }
};

// The same staging for one activation row that is already fp32 (the routed
// FFN's SwiGLU output): two 16-byte loads per 8-element chunk, stored as is.
template <int S, int THREADS>
struct XStagerF32 {
  static constexpr int kRowChunks = S * 4 * kWave;
  static constexpr int kPer = (kRowChunks + THREADS - 1) / THREADS;
  uint4 d[kPer][2];

  // raw buffer loads over the row (chunks past K read zero)
  __device__ __forceinline__ void load(const float* __restrict__ x, int64_t K) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(x, (uint32_t)K * 4u);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * THREADS + (int)threadIdx.x;
      const int st = c >> 8, q = (c >> 6) & 3, l = c & 63;
      const uint32_t k = (uint32_t)((st * kWave + l) * kBlock + q * 8);
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t v0 =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, k * 4u, 0, 0));
      const u32x4_t v1 =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, k * 4u + 16u, 0, 0));
      d[i][0] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
      d[i][1] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
    }
  }
  __device__ __forceinline__ void pin() const {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        asm volatile("" ::"v"(d[i][h].x), "v"(d[i][h].y), "v"(d[i][h].z), "v"(d[i][h].w));
  }
  __device__ __forceinline__ void store_f32(float4* __restrict__ xs) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = i * THREADS + (int)threadIdx.x;
      if (kRowChunks % THREADS != 0 && c >= kRowChunks) break;
      const int st = c >> 8, q = (c >> 6) & 3, l = c & 63;
      float4* row = xs + st * 8 * kWave + l;
      row[(2 * q) * kWave] = __builtin_bit_cast(float4, d[i][0]);
      row[(2 * q + 1) * kWave] = __builtin_bit_cast(float4, d[i][1]);
    }
  }
};

// ---------------------------------------------------------------------------
// One task of R rows with the activations in LDS and every code and scale
// load issued up front, for rows of FULL whole stages plus a leftover stage
// of kind TAIL (none, split between the half-waves, one block per lane, or
// -- rows of a single leftover stage of at most 48 blocks, a multiple of 4
// rows a task -- the rows' blocks laid end to end over the lanes, 3 passes
// per 4 rows, so no lane idles when a row has 48 blocks).
//
// Split in two so a kernel can issue the loads before it stages the
// activations: the LDS staging and its barrier then overlap the loads'
// HBM latency.  Rows past the last one are read as the last row (in
// bounds); the caller discards their results.
enum TailKind { kNoTail = 0, kSplitTail = 1, kWideTail = 2, kFlatTail = 3 };
constexpr int kFlatMaxBlocks = 48;
template <int R>
constexpr int flat_passes() { return R * kFlatMaxBlocks / kWave; }

// Slot t of lane l in the flat layout of R rows of rem blocks: block
// j = l + 64 t of the rows laid end to end, i.e. block blk of task row row
// (row = R, blk = 0 past the last slot).  recip = ceil(65536 / rem):
// (j * recip) >> 16 is j / rem exactly for j < 2^16 / rem (here j < 8 * 48).
template <int R>
__device__ __forceinline__ void flat_slot(int lane, int t, int rem, uint32_t recip, int& row,
                                          int& blk) {
  const uint32_t j = (uint32_t)(lane + kWave * t);
  const uint32_t q = (j * recip) >> 16;
  row = q < (uint32_t)R ? (int)q : R;
  blk = q < (uint32_t)R ? (int)(j - q * (uint32_t)rem) : 0;
}
__host__ __device__ __forceinline__ uint32_t flat_recip(int rem) {
  return (65536u + (uint32_t)rem - 1u) / (uint32_t)rem;
}

// SC: how a block scale is held -- _Float16 (the int4 codes' fp16 scales),
// float (exact fp32 block scales, e.g. expanded from super-block scales) or
// uint8_t (the E8M0 bytes of 4-bit float blocks).
// Super-block scales held as loaded: the fp16 scale d of the block's
// 256-element super-block and the block's 8-bit multiplier; the block scale
// d * m has at most 19 significant bits and is formed exactly in fp32.
struct SbScale {
  _Float16 d;
  uint8_t m;
  __device__ __forceinline__ SbScale() : d((_Float16)0.0f), m(0) {}
  __device__ __forceinline__ explicit SbScale(float) : d((_Float16)0.0f), m(0) {}
  __device__ __forceinline__ operator float() const { return (float)d * (float)m; }
};

template <int R, int FULL, int TAIL, typename SC = _Float16>
struct UpfrontLoads {
  static_assert(TAIL != kFlatTail || (FULL == 0 && R % 4 == 0),
                "the flat layout covers a multiple of 4 rows of one leftover stage");
  static constexpr int TR = TAIL == kSplitTail ? R / 2
                            : TAIL == kWideTail ? R
                            : TAIL == kFlatTail ? flat_passes<R>() : 0;
  uint4 c[FULL > 0 ? FULL : 1][R];
  SC s[FULL > 0 ? FULL : 1][R];
  uint4 ct[TR > 0 ? TR : 1];
  SC st[TR > 0 ? TR : 1];
};

// Weights and scales are read once per call: the loads are non-temporal, so
// they do not displace reusable lines from the caches (a loads-only stream
// of 100 MB from a cold 1.3 GB rotation measured 76% of HBM peak this way
// against 69-71% with ordinary loads).
__device__ __forceinline__ void load_scale(const uint16_t* p, _Float16& s) {
  s = __builtin_bit_cast(_Float16, __builtin_nontemporal_load(p));
}
__device__ __forceinline__ void load_scale(const uint8_t* p, uint8_t& s) {
  s = __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void load_scale(const float* p, float& s) {
  s = __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint4 load_codes(const uint8_t* p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// cbase / sbase: codes and scales of the task's first row at the first
// block of the row piece; row_bytes / row_sc: distance between rows (bytes,
// scales); room = rows that exist past the first (>= 0); rem = leftover
// blocks of the piece; bpr = blocks from the piece's first block to the end
// of its rows (bounds the loads).
//
// Raw buffer loads (above): descriptors over the task's rows exactly, a
// row's offset in the scalar part, the lane's block in the vector part.
template <int R, int FULL, int TAIL, typename SC, typename SP>
__device__ __forceinline__ void upfront_load(UpfrontLoads<R, FULL, TAIL, SC>& b,
                                             const uint8_t* __restrict__ cbase,
                                             const SP* __restrict__ sbase,
                                             uint32_t row_bytes, uint32_t row_sc, int room,
                                             int rem, int lane, uint32_t bpr) {
  constexpr uint32_t SZ = (uint32_t)sizeof(SP);
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(cbase, (uint32_t)room * row_bytes + bpr * 16u);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sbase, ((uint32_t)room * row_sc + bpr) * SZ);
  auto load = [&](int row, uint32_t blk, uint32_t lane_blk, uint4& c, SC& s) {
    row = row < room ? row : room;
    c = buffer_codes(rc, lane_blk * 16u, (uint32_t)row * row_bytes + blk * 16u);
    buffer_scale(rs, lane_blk * SZ, ((uint32_t)row * row_sc + blk) * SZ, s);
  };
#pragma unroll
  for (int st = 0; st < FULL; ++st)
#pragma unroll
    for (int r = 0; r < R; ++r)
      load(r, (uint32_t)(st * kWave), (uint32_t)lane, b.c[st][r], b.s[st][r]);
  if constexpr (TAIL == kSplitTail) {
    constexpr int H = R / 2;
    const int sub = lane & 31, half = lane >> 5;
    const uint32_t t = (uint32_t)(sub < rem ? sub : 0);
    // the two half-waves read different rows: the row offset is per lane
#pragma unroll
    for (int j = 0; j < H; ++j) {
      int row = half * H + j;
      row = row < room ? row : room;
      const uint32_t blk = (uint32_t)(FULL * kWave);
      b.ct[j] = buffer_codes(rc, (uint32_t)row * row_bytes + t * 16u, blk * 16u);
      buffer_scale(rs, ((uint32_t)row * row_sc + t) * SZ, blk * SZ, b.st[j]);
    }
  } else if constexpr (TAIL == kWideTail) {
    const uint32_t t = (uint32_t)(lane < rem ? lane : 0);
#pragma unroll
    for (int r = 0; r < R; ++r) load(r, (uint32_t)(FULL * kWave), t, b.ct[r], b.st[r]);
  } else if constexpr (TAIL == kFlatTail) {
    // slots past the rows read row 0's block 0 (in bounds; not added)
    const uint32_t recip = flat_recip(rem);
#pragma unroll
    for (int t = 0; t < flat_passes<R>(); ++t) {
      int row, blk;
      flat_slot<R>(lane, t, rem, recip, row, blk);
      row = row < R ? (row < room ? row : room) : 0;
      const uint32_t off = (uint32_t)row * row_bytes + (uint32_t)blk * 16u;
      b.ct[t] = buffer_codes(rc, off, 0u);
      buffer_scale(rs, ((uint32_t)row * row_sc + (uint32_t)blk) * SZ, 0u, b.st[t]);
    }
  }
}

// The same for super-block scales, whole rows only (the piece starts at
// block 0, so lane l's block st * 64 + l lies in super-block st * 8 + l / 8):
// dbase and mbase are the task's first row's super-block scales and block
// multipliers; row_d = K/256 scales per row.
template <int R, int FULL, int TAIL>
__device__ __forceinline__ void upfront_load_sb(UpfrontLoads<R, FULL, TAIL, SbScale>& b,
                                                const uint8_t* __restrict__ cbase,
                                                const uint16_t* __restrict__ dbase,
                                                const uint8_t* __restrict__ mbase,
                                                uint32_t row_bytes, uint32_t row_sc, int room,
                                                int rem, int lane) {
  const uint32_t row_d = row_sc / 8;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(cbase, ((uint32_t)room + 1) * row_bytes);
  const __amdgpu_buffer_rsrc_t rm = buffer_rsrc(mbase, ((uint32_t)room + 1) * row_sc);
  const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dbase, ((uint32_t)room + 1) * row_d * 2u);
  auto load = [&](uint32_t row, uint32_t blk, uint32_t lane_blk, uint4& c, SbScale& s) {
    c = buffer_codes(rc, lane_blk * 16u, row * row_bytes + blk * 16u);
    s.m = __builtin_amdgcn_raw_buffer_load_b8(rm, lane_blk, row * row_sc + blk, 2);
    s.d = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(
                                           rd, (lane_blk >> 3) * 2u, (row * row_d + blk / 8) * 2u, 2));
  };
#pragma unroll
  for (int st = 0; st < FULL; ++st)
#pragma unroll
    for (int r = 0; r < R; ++r)
      load((uint32_t)(r < room ? r : room), (uint32_t)(st * kWave), (uint32_t)lane, b.c[st][r],
           b.s[st][r]);
  if constexpr (TAIL == kSplitTail) {
    constexpr int H = R / 2;
    const int sub = lane & 31, half = lane >> 5;
    const uint32_t t = (uint32_t)(sub < rem ? sub : 0);
    const uint32_t blk = (uint32_t)(FULL * kWave);
    // the two half-waves read different rows: the row offset is per lane
#pragma unroll
    for (int j = 0; j < H; ++j) {
      int row = half * H + j;
      row = row < room ? row : room;
      b.ct[j] = buffer_codes(rc, (uint32_t)row * row_bytes + t * 16u, blk * 16u);
      b.st[j].m = __builtin_amdgcn_raw_buffer_load_b8(rm, (uint32_t)row * row_sc + t, blk, 2);
      b.st[j].d = __builtin_bit_cast(
          _Float16, __builtin_amdgcn_raw_buffer_load_b16(
                        rd, ((uint32_t)row * row_d + (t >> 3)) * 2u, (blk / 8) * 2u, 2));
    }
  } else if constexpr (TAIL == kWideTail) {
    const uint32_t t = (uint32_t)(lane < rem ? lane : 0);
#pragma unroll
    for (int r = 0; r < R; ++r)
      load((uint32_t)(r < room ? r : room), (uint32_t)(FULL * kWave), t, b.ct[r], b.st[r]);
  }
}

// Rows per task and wavefronts per workgroup of the kernels built on the
// up-front loads; rows of at most kLdsMaxStages stages (K <= 8192).
constexpr int kLdsRows = 2;
constexpr int kLdsWaves = 4;
constexpr int kLdsMaxStages = 4;

// Calls f(FULL, TAIL) -- both std::integral_constant -- with the row
// geometry of K when it has at most kLdsMaxStages stages; otherwise returns
// hipErrorInvalidValue without calling f.
template <class F>
hipError_t dispatch_row_geometry(int64_t K, F&& f) {
  using std::integral_constant;
  const int64_t bpr = K / kBlock;
  const int64_t full = bpr / kWave;
  const int rem = (int)(bpr % kWave);
  const int tail = rem == 0 ? kNoTail : (rem <= kWave / 2 ? kSplitTail : kWideTail);
  switch (full * 3 + tail) {
    case 0 * 3 + kSplitTail: return f(integral_constant<int, 0>{}, integral_constant<int, kSplitTail>{});
    case 0 * 3 + kWideTail: return f(integral_constant<int, 0>{}, integral_constant<int, kWideTail>{});
    case 1 * 3 + kNoTail: return f(integral_constant<int, 1>{}, integral_constant<int, kNoTail>{});
    case 1 * 3 + kSplitTail: return f(integral_constant<int, 1>{}, integral_constant<int, kSplitTail>{});
    case 1 * 3 + kWideTail: return f(integral_constant<int, 1>{}, integral_constant<int, kWideTail>{});
    case 2 * 3 + kNoTail: return f(integral_constant<int, 2>{}, integral_constant<int, kNoTail>{});
    case 2 * 3 + kSplitTail: return f(integral_constant<int, 2>{}, integral_constant<int, kSplitTail>{});
    case 2 * 3 + kWideTail: return f(integral_constant<int, 2>{}, integral_constant<int, kWideTail>{});
    case 3 * 3 + kNoTail: return f(integral_constant<int, 3>{}, integral_constant<int, kNoTail>{});
    case 3 * 3 + kSplitTail: return f(integral_constant<int, 3>{}, integral_constant<int, kSplitTail>{});
    case 3 * 3 + kWideTail: return f(integral_constant<int, 3>{}, integral_constant<int, kWideTail>{});
    case 4 * 3 + kNoTail: return f(integral_constant<int, 4>{}, integral_constant<int, kNoTail>{});
    default: return hipErrorInvalidValue;
  }
}

// Leftover blocks per row (0 .. 63).
__host__ __device__ __forceinline__ int row_leftover(int64_t K) {
  return (int)((K / kBlock) % kWave);
}

// Totals (wave-uniform) of the task loaded into b; xs is the LDS activation
// table (fp32 layout above).  SC = uint8_t: 4-bit float blocks (e2m1
// elements, E8M0 scales); else the int4 codes with fp16 scales.
template <int M, int R, int FULL, int TAIL, typename SC = _Float16>
__device__ __forceinline__ void upfront_compute(const UpfrontLoads<R, FULL, TAIL, SC>& b,
                                                const float4* xs, int rem, int lane,
                                                float (&out)[R][M]) {
  constexpr bool kMx = std::is_same<SC, uint8_t>::value;
  constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
  const CodeUnpacker unpack;
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  // acc += block products of stage st for rows c/s, activations of lane l
  auto rows = [&](int st, int l, const auto& c, const auto& s, auto& a) __attribute__((always_inline)) {
    constexpr int RR = sizeof(c) / sizeof(c[0]);
    float xv[M][32];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = xs[((m * S + st) * 8 + q) * kWave + l];
        xv[m][4 * q + 0] = v.x;
        xv[m][4 * q + 1] = v.y;
        xv[m][4 * q + 2] = v.z;
        xv[m][4 * q + 3] = v.w;
      }
    if constexpr (kMx) {
      float sf[RR];
#pragma unroll
      for (int r = 0; r < RR; ++r) sf[r] = e8m0_to_f32(s[r]);
      mx_block_rows_f32<M, RR>(c, sf, xv, a);
    } else {
      block_rows_f32<M, RR>(unpack, c, s, xv, a);
    }
  };
#pragma unroll
  for (int st = 0; st < FULL; ++st) rows(st, lane, b.c[st], b.s[st], acc);
  if constexpr (TAIL == kSplitTail) {
    constexpr int H = R / 2;
    const int sub = lane & 31, half = lane >> 5;
    float t[H][M];
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m) t[j][m] = 0.0f;
    rows(FULL, sub, b.ct, b.st, t);
    // slot j of half h is row h*H + j; only lanes with a leftover block add
    const bool ok = sub < rem;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const bool owns = r < H ? half == 0 : half == 1;
        acc[r][m] += (ok && owns) ? t[r % H][m] : 0.0f;
      }
  } else if constexpr (TAIL == kWideTail) {
    // A lane past the leftover blocks reads zero activations (LDS holds 0
    // past K) and gets scale 0, so it adds exactly zero whatever its
    // (clamped, real) codes and scale are.
    const bool ok = lane < rem;
    if constexpr (kMx) {
      // E8M0 has no zero: take the lane's contribution away by selection
      // (its clamped real scale may be NaN)
      float t[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
      rows(FULL, lane, b.ct, b.st, t);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] += ok ? t[r][m] : 0.0f;
    } else {
      SC sc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r] = ok ? b.st[r] : (SC)0.0f;
      rows(FULL, lane, b.ct, sc, acc);
    }
  } else if constexpr (TAIL == kFlatTail) {
    static_assert(!kMx, "the flat layout is built for int4 codes");
    // each slot's block product goes to its own row (slots past the rows to
    // none); LDS holds the activations of block blk at position blk
    const uint32_t recip = flat_recip(rem);
#pragma unroll
    for (int t = 0; t < flat_passes<R>(); ++t) {
      int row, blk;
      flat_slot<R>(lane, t, rem, recip, row, blk);
      float part[1][M];
#pragma unroll
      for (int m = 0; m < M; ++m) part[0][m] = 0.0f;
      const uint4 c1[1] = {b.ct[t]};
      const SC s1[1] = {b.st[t]};
      rows(FULL, blk, c1, s1, part);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] += row == r ? part[0][m] : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) out[r][m] = wave_total(acc[r][m]);
}

// ---------------------------------------------------------------------------
// One task of R rows with activations read from global memory (bf16),
// loads one stage ahead.  Used by the expert-routed kernel, whose tokens are
// gathered rows of x, and by the decode kernel when the activations do not
// fit in LDS.  Rows past n_last are read as row n_last (in bounds); the
// caller discards their results.  Totals are returned wave-uniform.
template <int M, int R>
__device__ __forceinline__ void gemv_task(const uint16_t* const (&xrow)[M],
                                          const uint8_t* __restrict__ wq,
                                          const uint16_t* __restrict__ ws, int64_t n0,
                                          int64_t n_last, int64_t K, float (&out)[R][M]) {
  static_assert(R % 2 == 0, "rows per task must be even");
  const int lane = threadIdx.x & (kWave - 1);
  const StagePlan sp(K, lane);
  const int64_t row_bytes = K / 2;
  const CodeUnpacker unpack;

  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  struct Buf {
    uint4 c[R];
    _Float16 s[R];
  };
  auto load = [&](int64_t st, Buf& b) {
    const int64_t blk = sp.block(st, lane);
    const bool last = st >= sp.full;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = last ? tail_row<R>(sp, r) : r;
      const int64_t n = n0 + row < n_last ? n0 + row : n_last;
      b.c[r] = load_codes(wq + n * row_bytes + blk * 16);
      load_scale(ws + n * sp.bpr + blk, b.s[r]);
    }
  };
  auto compute = [&](int64_t st, const Buf& b) {
    uint4 xd[M][4];
    const int64_t blk = sp.block(st, lane);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4* p = reinterpret_cast<const uint4*>(xrow[m] + blk * kBlock);
#pragma unroll
      for (int q = 0; q < 4; ++q) xd[m][q] = p[q];
    }
    if (st < sp.full) {
      block_rows_bf16<M, R>(unpack, b.c, b.s, xd, acc);
    } else if (sp.split) {
      constexpr int H = R / 2;
      uint4 c[H];
      _Float16 sc[H];
      float t[H][M];
#pragma unroll
      for (int r = 0; r < H; ++r) {
        c[r] = b.c[r];
        sc[r] = b.s[r];
#pragma unroll
        for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
      }
      block_rows_bf16<M, H>(unpack, c, sc, xd, t);
      add_tail_split<M, R>(sp, t, acc);
    } else {
      float t[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
      block_rows_bf16<M, R>(unpack, b.c, b.s, xd, t);
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
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) out[r][m] = wave_total(acc[r][m]);
}

}  // namespace q4
