// q4_small.hip -- few activation rows (3 <= M <= 32, or up to 128 when the
// tiled path would have too few tiles): exact-weight matrix-core kernel.
//
// The quantised GEMM of the T0 kernel tier ("spec: specialized model
// runtimes", sections "Architecture" and "Feasibility gate") between the
// decode and the prefill shapes.  The matrix-vector kernel spends one fma per
// weight per activation row, so from about 3 rows on it is bound by vector
// ALU issue; the tiled bf16 kernel rounds the weights to bf16 and needs
// hundreds of 128 x 128 tiles to fill the chip.  This kernel keeps the
// weights exact and puts the products on the matrix cores:
//
//  * (c - 8) is a small integer, exact in bf16, so each 32-element block's
//    partial sum sum_k x[m][k] * (c[n][k] - 8) is one
//    v_mfma_f32_16x16x32_bf16 (16 activation rows x 16 weight rows x the
//    block's 32 k): products exact, fp32 sums;
//  * the block's fp16 scale is applied to that 16 x 16 partial in fp32 (one
//    fma per output per block), which is the groupwise definition
//    y = sum_blocks s * sum_k x * (c - 8) and needs no rounding of weights.
//    A block of all-8 codes contributes exactly zero.
//
// Operand layout (wave64, lane = 16 * g + r):
//  * A (activations): lane holds x[m = r][32 b + 8 g .. + 7] (16 bytes);
//  * B (weights):     lane holds the 8 codes k = 32 b + 8 g .. + 7 of weight
//                     row n = r, i.e. dword g of block b;
//  * D:               lane holds rows m = 4 g .. 4 g + 3 of column n = r, so
//                     a lane needs the one scale s[n][b].
// Codes are read as 16 bytes per lane -- lane (r, g) takes block b0 + g of
// row r, so the 4 lane groups read 64 consecutive bytes of each row -- and a
// 4 x 4 transpose across the lane groups (v_permlane16_swap and
// v_permlane32_swap) then gives lane (r, g) dword g of blocks b0 .. b0 + 3.
//
// 4-bit float blocks (MX = true: e2m1 elements, E8M0 scale bytes) take the
// same kernel: e2m1 values are exact in bf16 too (at most 2 significant bits),
// so each byte of elements becomes two exact fp32 values with
// v_cvt_scalef32_pk_f32_fp4 (scale 1) and one v_cvt_pk_bf16_f32, and the
// block's 2^(E-127) is applied in fp32 where the int4 path applies its fp16
// scale.
//
// Work split: a workgroup of kWaves wavefronts owns kNg * 16 weight rows and
// one slab of 16 * MG activation rows; its wavefronts take consecutive
// stretches of the row's 4-block groups, each keeping two groups of loads in
// flight, and their partial sums are added in wavefront order through LDS
// (deterministic).
#include <type_traits>

#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {

constexpr int kNg = 2;      // 16-row weight groups per workgroup
constexpr int kWaves = 4;   // wavefronts per workgroup (split of K)
constexpr int kDepth = 2;   // 4-block groups in flight per wavefront

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 (c - 8) of the 8 codes of d, in k order (exact: small integers).
__device__ __forceinline__ bf16x8v codes_to_bf16(uint32_t d, const ExactBf16Unpacker& unpack) {
  uint32_t o[4];
  unpack(d, o);
  const u32x4 v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8v, v);
}

// bf16 elements of the 8 e2m1 values of d, in k order (exact).
__device__ __forceinline__ bf16x8v fp4_to_bf16(uint32_t d) {
  const f32x2v w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
  const f32x2v w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
  const f32x2v w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
  const f32x2v w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
  u32x4 o;
  o[0] = pack_bf16x2(w0[0], w0[1]);
  o[1] = pack_bf16x2(w1[0], w1[1]);
  o[2] = pack_bf16x2(w2[0], w2[1]);
  o[3] = pack_bf16x2(w3[0], w3[1]);
  return __builtin_bit_cast(bf16x8v, o);
}

// Before: register j of lane group g (16 lanes) holds E[g][j].
// After:  register j of lane group g holds E[j][g].
__device__ __forceinline__ void transpose_groups(uint32_t r[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap(r[0], r[1], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(r[2], r[3], false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  r[0] = c[0];
  r[2] = c[1];
  r[1] = d[0];
  r[3] = d[1];
}

}  // namespace

// SCALE4: K/32 is a multiple of 4, so a row's 4 scales of a group are one
// aligned load (8 bytes of fp16, 4 E8M0 bytes or 16 bytes of fp32).
// MX: 4-bit float blocks (scales are E8M0 bytes); else int4 codes with fp16
// scales.
// F32S: int4 codes with exact fp32 block scales [N][K/32] (e.g. expanded from
// super-block scales) instead of fp16 ones.
template <int MG, bool SCALE4, bool MX, bool F32S>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(MG == 1 ? 4 : 2))) void small_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const void* __restrict__ wsv, void* __restrict__ y, int y_bf16, int64_t M, int64_t N,
    int64_t K, int64_t groups_per_wave, int64_t groups_per_slice, float* __restrict__ partial) {
  using ScaleT = typename std::conditional<
      MX, uint8_t, typename std::conditional<F32S, float, uint16_t>::type>::type;
  // scales of a group as loaded: 4 fp16 in 2 dwords, 4 E8M0 bytes in 1, or
  // 4 fp32
  constexpr int SW = F32S ? 4 : (MX ? 1 : 2);
  const ScaleT* ws = static_cast<const ScaleT*>(wsv);
  __shared__ f32x4v red[kWaves][kNg][MG][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t bpr = K / 32;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * kNg);
  const int64_t m0 = (int64_t)blockIdx.y * (16 * MG);
  // Rows past N (M) read the workgroup's last row; their outputs are not
  // stored.
  const int64_t rows_w = N - n0 < 16 * kNg ? N - n0 : 16 * kNg;
  const int64_t rows_x = M - m0 < 16 * MG ? M - m0 : 16 * MG;
  int wl[kNg], xl[MG];   // this lane's weight and activation rows in the workgroup
#pragma unroll
  for (int ng = 0; ng < kNg; ++ng) wl[ng] = ng * 16 + r < rows_w ? ng * 16 + r : (int)rows_w - 1;
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) xl[mg] = mg * 16 + r < rows_x ? mg * 16 + r : (int)rows_x - 1;
  const uint8_t* wq_g = wq + n0 * (K / 2);
  const ScaleT* ws_g = ws + n0 * bpr;
  const uint16_t* x_g = x + m0 * K;
  // K slice blockIdx.z: 4-block groups [q_beg, q_end) of the row
  const int64_t q_beg = (int64_t)blockIdx.z * groups_per_slice;
  const int64_t q_end = q_beg + groups_per_slice;
  const ExactBf16Unpacker unpack;
  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};
  f32x4v acc[kNg][MG];
#pragma unroll
  for (int ng = 0; ng < kNg; ++ng)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) acc[ng][mg] = zero;

  // Ring of kDepth groups.  Slot loads are unconditional: a group index past
  // the row's end reads the row's last group again (never out of bounds) and
  // is skipped when computed.
  uint32_t codes[kDepth][kNg][4];
  uint32_t sraw[kDepth][kNg][SW];
  bf16x8v xf[kDepth][4][MG];
  auto load = [&](int64_t q, auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    int64_t b0 = q * 4;   // wave-uniform
    if (b0 >= bpr) b0 = (bpr - 1) & ~int64_t(3);
    // lane (r, g) takes block b0 + g of its row (the row's last block past
    // its end, which only a group that is cut short reaches)
    const int64_t bl = SCALE4 ? b0 + g : (b0 + g < bpr ? b0 + g : bpr - 1);
#pragma unroll
    for (int ng = 0; ng < kNg; ++ng) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wq_g + (int64_t)wl[ng] * (K / 2) + bl * 16);
      codes[d][ng][0] = v[0];
      codes[d][ng][1] = v[1];
      codes[d][ng][2] = v[2];
      codes[d][ng][3] = v[3];
      if constexpr (SCALE4) {
        // the row's 4 scales of the group, as stored
        const ScaleT* sp = ws_g + (int64_t)wl[ng] * bpr + b0;
#pragma unroll
        for (int j = 0; j < SW; ++j) sraw[d][ng][j] = reinterpret_cast<const uint32_t*>(sp)[j];
      } else {
        // one scale at a time, clamped to the row
        ScaleT sv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t bj = b0 + j < bpr ? b0 + j : bpr - 1;
          sv[j] = ws_g[(int64_t)wl[ng] * bpr + bj];
        }
        if constexpr (SW == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) sraw[d][ng][j] = __builtin_bit_cast(uint32_t, sv[j]);
        } else if constexpr (SW == 2) {
          sraw[d][ng][0] = (uint32_t)sv[0] | ((uint32_t)sv[1] << 16);
          sraw[d][ng][1] = (uint32_t)sv[2] | ((uint32_t)sv[3] << 16);
        } else {
          sraw[d][ng][0] = (uint32_t)sv[0] | ((uint32_t)sv[1] << 8) | ((uint32_t)sv[2] << 16) |
                           ((uint32_t)sv[3] << 24);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t bj = b0 + j < bpr ? b0 + j : bpr - 1;   // wave-uniform
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
        xf[d][j][mg] = *reinterpret_cast<const bf16x8v*>(x_g + (int64_t)xl[mg] * K + 8 * g + bj * 32);
    }
  };
  // block j's scale of 16-row weight group ng, from slot d
  auto scale_of = [&](int d, int ng, int j) __attribute__((always_inline)) -> float {
    if constexpr (SW == 4) return __builtin_bit_cast(float, sraw[d][ng][j]);
    else if constexpr (SW == 2)
      return (float)__builtin_bit_cast(half2v, sraw[d][ng][j >> 1])[j & 1];
    else return e8m0_to_f32((sraw[d][ng][0] >> (8 * j)) & 0xFFu);
  };
  auto block = [&](int j, auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
#pragma unroll
    for (int ng = 0; ng < kNg; ++ng) {
      const bf16x8v w = MX ? fp4_to_bf16(codes[d][ng][j]) : codes_to_bf16(codes[d][ng][j], unpack);
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const f32x4v p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[d][j][mg], w, zero, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[ng][mg][e] = __builtin_fmaf(scale_of(d, ng, j), p[e], acc[ng][mg][e]);
      }
    }
  };
  auto compute = [&](int64_t q, auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
#pragma unroll
    for (int ng = 0; ng < kNg; ++ng) transpose_groups(codes[d][ng]);
    // blocks of this group inside the row (none past the slice's end)
    const int64_t left = q < q_end ? bpr - q * 4 : 0;
    if (left >= 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) block(j, slot);
    } else if (left > 0) {
      block(0, slot);
      if (left > 1) block(1, slot);
      if (left > 2) block(2, slot);
    }
  };
  static_assert(kDepth == 2, "the ring below is written for two slots");
  const std::integral_constant<int, 0> s0;
  const std::integral_constant<int, 1> s1;
  const int64_t q0 = q_beg + (int64_t)wave * groups_per_wave;
  load(q0, s0);
  load(q0 + 1, s1);
  for (int64_t i = 0; i < groups_per_wave; i += kDepth) {
    const int64_t q = q0 + i;
    compute(q, s0);
    load(q + kDepth, s0);
    compute(q + 1, s1);
    load(q + 1 + kDepth, s1);
  }

#pragma unroll
  for (int ng = 0; ng < kNg; ++ng)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) red[wave][ng][mg][lane] = acc[ng][mg];
  __syncthreads();
  // Output (m, n) of the workgroup, n fastest: lane 16 * (m / 4) + n of each
  // wavefront's tile holds it in element m % 4.
  constexpr int kOut = kNg * 16 * MG * 16;
  for (int o = threadIdx.x; o < kOut; o += kWaves * 64) {
    const int nl = o % (kNg * 16), ml = o / (kNg * 16);
    const int ng = nl / 16, mg = ml / 16, mi = ml % 16;
    const int src = (mi / 4) * 16 + nl % 16;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w][ng][mg][src][mi % 4];
    const int64_t m = m0 + ml, n = n0 + nl;
    if (m < M && n < N) {
      if (partial) partial[(int64_t)blockIdx.z * M * N + m * N + n] = s;
      else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(s);
      else static_cast<float*>(y)[m * N + n] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 operands for the few-row kernels.  A bf16 value has an 8-bit
// significand, so it is an fp16 normal number exactly when its exponent lies
// in -14 .. 15.  When the nonzero activations of a workgroup's slice span at
// most 30 binary exponents (largest minus smallest <= 29), none of them
// subnormal, infinite or NaN, one power-of-two scaling x' = x * 2^-e puts
// all of them in that window; (c - 8) is exact in fp16 too, so
// v_mfma_f32_16x16x32_f16 forms the same exact products as the bf16 one,
// and the unpack of 8 codes takes 9 instructions instead of 17.  The
// results are multiplied back by 2^e (exact).  The range of a set of bf16
// values is kept as a "range key": the largest magnitude (bits without the
// sign) in the low 16 bits and 0x8000 minus the smallest nonzero magnitude
// in the high 16 bits (0 when all are zero), both maxima, so keys combine
// with one packed 16-bit maximum.
namespace {

typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2v, a),
                                                                __builtin_bit_cast(u16x2v, b)));
}

// range key of the 8 bf16 values of a 16-byte unit
__device__ __forceinline__ uint32_t unit_range_key(uint4 v) {
  const u16x2v one = {1, 1}, top = {0x7FFF, 0x7FFF};
  u16x2v mag = {0, 0}, inv = {0, 0};
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u16x2v m = __builtin_bit_cast(u16x2v, w[q] & 0x7FFF7FFFu);
    mag = __builtin_elementwise_max(mag, m);
    // zero wraps to 0xFFFF and saturates to 0; a magnitude v >= 1 gives 0x8000 - v
    inv = __builtin_elementwise_max(inv, __builtin_elementwise_sub_sat(top, m - one));
  }
  const uint32_t lo = mag[0] > mag[1] ? mag[0] : mag[1];
  const uint32_t hi = inv[0] > inv[1] ? inv[0] : inv[1];
  return lo | hi << 16;
}

// wave-uniform packed maximum over the 64 lanes
__device__ __forceinline__ uint32_t wave_pk_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    v = pk_max_u16(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// The scaling exponent e for a range key, and whether the values fit.  Of
// the exponents that work the one nearest 0 is taken; e lies in -112 .. 112,
// so 2^e and 2^-e are normal fp32.
__device__ __forceinline__ bool h16_scale(uint32_t key, int& e) {
  const uint32_t inv = key >> 16;
  e = 0;
  if (inv == 0) return true;   // all zero
  const int emax = (int)((key & 0xFFFFu) >> 7), emin = (int)((0x8000u - inv) >> 7);
  const int lo = emax - 127 - 15, hi = emin - 127 + 14;   // need lo <= e <= hi
  const int near0 = hi < 0 ? hi : 0;
  e = lo > near0 ? lo : near0;
  return emax <= 254 && emin >= 1 && emax - emin <= 29;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// The unit as fp16 x * sc in CodeUnpacker's element order (e0, e4, e1, e5,
// e2, e6, e3, e7), so that it pairs with the unpacked codes of one dword.
__device__ __forceinline__ uint4 unit_to_f16(uint4 v, float sc) {
  auto pair = [](float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  };
  return make_uint4(pair(bf16_lo(v.x) * sc, bf16_lo(v.z) * sc),
                    pair(bf16_hi(v.x) * sc, bf16_hi(v.z) * sc),
                    pair(bf16_lo(v.y) * sc, bf16_lo(v.w) * sc),
                    pair(bf16_hi(v.y) * sc, bf16_hi(v.w) * sc));
}

}  // namespace

// ---------------------------------------------------------------------------
// Few rows with a K-slice workspace (M <= 16): the matrix-vector kernel's
// streaming structure on the matrix cores.  A workgroup of kBatchWaves
// wavefronts owns 16 * kBatchWaves weight rows and one K slice of
// kBatchBlocks blocks; each wavefront takes 16 rows of the slice and issues
// every code and scale load of them up front (kBatchGroups 4-block groups,
// the few-row kernel's lane layout and transpose), after the loads of the
// slice's activations, which the workgroup then writes once to LDS as MFMA A
// operands while the weights are in flight.  Products are the few-row
// kernel's: one v_mfma_f32_16x16x32_bf16 per block with exact bf16 (c - 8),
// the block's scale applied to the 16 x 16 partial in fp32.  Every
// workgroup of the grid is resident at once for the shapes this kernel is
// chosen for, so the whole weight stream is in flight from the start.  The
// fp32 partial sums of the slices are added in slice order afterwards.
constexpr int kBatchWaves = 8;
constexpr int kBatchGroups = 8;
constexpr int kBatchBlocks = 4 * kBatchGroups;
constexpr int64_t kBatchMaxSlices = 64;

// LDS unit (b, g, r), 16 bytes: x[r][32 b + 8 g .. + 7] of the slice's block b
// (the A operand of lane 16 g + r), rows r >= M zero.  The 16 units of one
// (b, g) sit together, 17 apart from the next (b, g): the MFMA reads (16 lanes
// on consecutive units) and the staging writes (16 lanes on consecutive
// (b, g) of one row, 272 bytes apart) both meet 16 distinct bank groups.
constexpr int kBatchUnitStride = 17;
__device__ __forceinline__ int batch_unit(int b, int g, int r) {
  return (b * 4 + g) * kBatchUnitStride + r;
}

// STAGED: the workgroup's scales of the slice (128 rows x kBatchBlocks) go
// through LDS too, one 16-byte load per thread (rows whose slice scales are
// 16-byte aligned: K/32 a multiple of 8 for fp16, of 4 for fp32 scales);
// otherwise each lane loads its row's scales group by group (16 rows per
// load instruction, a few bytes each: far slower on HBM).
template <bool SCALE4, bool STAGED, typename SP>
__global__ __launch_bounds__(kBatchWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void batch_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const SP* __restrict__ ws,
    void* __restrict__ y, int y_bf16, int64_t M, int64_t N, int64_t K, float* __restrict__ partial) {
  static_assert(!STAGED || SCALE4, "staged scales come in whole groups");
  constexpr int kThreads = kBatchWaves * 64;
  constexpr int kUnits = kBatchBlocks * 4 * 16;
  constexpr int kPer = kUnits / kThreads;
  constexpr bool kF32 = std::is_same<SP, float>::value;
  // scales of a group as loaded: 4 fp16 in 2 dwords or 4 fp32
  constexpr int SW = kF32 ? 4 : 2;
  // staged scales: row stride in bytes (a row's slice plus 8 or 16 bytes of
  // padding, so that the 16 rows a load instruction reads fall in distinct
  // banks) and 16-byte chunks per row
  constexpr int kSRow = kF32 ? kBatchBlocks * 4 + 16 : kBatchBlocks * 2 + 8;
  constexpr int kSChunks = kBatchBlocks * (int)sizeof(SP) / 16;
  constexpr int kSPer = STAGED ? 16 * kBatchWaves * kSChunks / kThreads : 0;
  __shared__ uint4 xa[kBatchBlocks * 4 * kBatchUnitStride];
  __shared__ __attribute__((aligned(16))) uint8_t ss[STAGED ? 16 * kBatchWaves * kSRow : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t bpr = K / kBlock;
  const int64_t kb0 = (int64_t)blockIdx.y * kBatchBlocks;
  const int nb = (int)(bpr - kb0 < kBatchBlocks ? bpr - kb0 : kBatchBlocks);   // >= 1
  const int64_t n = (int64_t)blockIdx.x * (16 * kBatchWaves) + wave * 16 + r;
  const int64_t nl = n < N ? n : N - 1;

  // activation loads first (the memory counter waits in issue order, so
  // they can be used while the weight loads are still in flight).  Unit
  // number v = 128 m + 4 b + g (row m, block b, 8-element group g) so that
  // the real rows come first: with M <= 4 every thread holds one real unit
  // in xv[0].  Units of rows past M or blocks past the slice read the
  // slice's first unit and are masked to zero.
  uint4 xv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = i * kThreads + (int)threadIdx.x;
    const int m = v >> 7, b = (v >> 2) & 31, gg = v & 3;
    const bool ok = m < M && b < nb;
    const uint16_t* src = x + (ok ? (int64_t)m * K + (kb0 + b) * kBlock + gg * 8 : kb0 * kBlock);
    const uint4 xw = *reinterpret_cast<const uint4*>(src);
    const uint32_t keep = opaque_vgpr(ok ? 0xFFFFFFFFu : 0u);
    xv[i] = make_uint4(xw.x & keep, xw.y & keep, xw.z & keep, xw.w & keep);
  }
  // staged scales: thread t loads chunk t % kSChunks of workgroup row
  // t / kSChunks (clamped to the last row); chunks past the slice are not
  // loaded (the slice's blocks come in whole chunks)
  const int64_t wg_n0 = (int64_t)blockIdx.x * (16 * kBatchWaves);
  uint4 sv4[kSPer > 0 ? kSPer : 1];
  if constexpr (STAGED) {
#pragma unroll
    for (int i = 0; i < kSPer; ++i) {
      const int c = i * kThreads + (int)threadIdx.x;
      const int row = c / kSChunks, ch = c % kSChunks;
      const int64_t sn = wg_n0 + row < N ? wg_n0 + row : N - 1;
      const int chunk_blocks = 16 / (int)sizeof(SP);
      const int cb = ch * chunk_blocks < nb ? ch * chunk_blocks : 0;
      typedef uint32_t u32x4nt __attribute__((ext_vector_type(4)));
      const u32x4nt t =
          __builtin_nontemporal_load(reinterpret_cast<const u32x4nt*>(ws + sn * bpr + kb0 + cb));
      sv4[i] = make_uint4(t[0], t[1], t[2], t[3]);
    }
  }
  // every code load of the wavefront's 16 rows (and, not staged, every
  // scale load): group j, lane (r, g) takes block 4 j + g of its row
  // (clamped to the slice)
  const uint8_t* wrow = wq + nl * (K / 2) + kb0 * 16;
  const SP* srow = ws + nl * bpr + kb0;
  uint32_t codes[kBatchGroups][4];
  uint32_t sraw[STAGED ? 1 : kBatchGroups][SW];
#pragma unroll
  for (int j = 0; j < kBatchGroups; ++j) {
    const int bj = 4 * j + g < nb ? 4 * j + g : nb - 1;
    // ordinary loads: with the non-temporal hint this pattern (16 rows x 64
    // bytes per instruction) streams about 15% slower from HBM
    const u32x4 v = *reinterpret_cast<const u32x4*>(wrow + bj * 16);
    codes[j][0] = v[0];
    codes[j][1] = v[1];
    codes[j][2] = v[2];
    codes[j][3] = v[3];
    if constexpr (STAGED) {
    } else if constexpr (SCALE4) {
      // whole groups (bpr and the slice start are multiples of 4); a group
      // past the slice reads the slice's first group
      const int b0 = 4 * j < nb ? 4 * j : 0;
      if constexpr (SW == 4) {
        typedef float f32x4nt __attribute__((ext_vector_type(4)));
        const f32x4nt t = __builtin_nontemporal_load(reinterpret_cast<const f32x4nt*>(srow + b0));
#pragma unroll
        for (int q = 0; q < 4; ++q) sraw[j][q] = __builtin_bit_cast(uint32_t, t[q]);
      } else {
        typedef uint32_t u32x2nt __attribute__((ext_vector_type(2)));
        const u32x2nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x2nt*>(srow + b0));
        sraw[j][0] = t[0];
        sraw[j][1] = t[1];
      }
    } else {
      SP sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 4 * j + q < nb ? 4 * j + q : nb - 1;
        sv[q] = __builtin_nontemporal_load(srow + b);
      }
      if constexpr (SW == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sraw[j][q] = __builtin_bit_cast(uint32_t, sv[q]);
      } else {
        sraw[j][0] = (uint32_t)sv[0] | ((uint32_t)sv[1] << 16);
        sraw[j][1] = (uint32_t)sv[2] | ((uint32_t)sv[3] << 16);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // every load ahead of the staging
  // the slice's activation range (units past the real rows hold zeros and
  // are skipped; the condition is uniform)
  __shared__ uint32_t rng[kBatchWaves];
  uint32_t key = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (i * kThreads < M * 128) key = pk_max_u16(key, unit_range_key(xv[i]));
  key = wave_pk_max(key);
  if (lane == 0) rng[wave] = key;
  lds_barrier();
  uint32_t all = rng[0];
#pragma unroll
  for (int w = 1; w < kBatchWaves; ++w) all = pk_max_u16(all, rng[w]);
  int e16;
  const bool h16 = h16_scale(__builtin_amdgcn_readfirstlane((int)all), e16);
  const float sc16 = pow2f(-e16);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = i * kThreads + (int)threadIdx.x;
    const int m = v >> 7, b = (v >> 2) & 31, gg = v & 3;
    if (b >= nb) continue;
    uint4 u = xv[i];
    if (h16 && i * kThreads < M * 128) u = unit_to_f16(u, sc16);   // zeros stay zero
    xa[batch_unit(b, gg, m)] = u;
  }
  if constexpr (STAGED) {
#pragma unroll
    for (int i = 0; i < kSPer; ++i) {
      const int c = i * kThreads + (int)threadIdx.x;
      const int row = c / kSChunks, ch = c % kSChunks;
      uint8_t* dst = ss + row * kSRow + ch * 16;
      if constexpr (kF32) {
        *reinterpret_cast<uint4*>(dst) = sv4[i];
      } else {   // 8-byte aligned rows: two 8-byte stores
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(sv4[i].x, sv4[i].y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(sv4[i].z, sv4[i].w);
      }
    }
  }
  lds_barrier();   // the code loads stay in flight

  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};
  f32x4v acc = zero;
  // one 4-block group: the lane's row scales, the transpose, then each block
  // inside the slice as one MFMA (fp16 or bf16 operands) and four fmas
  auto groups = [&](auto fp16) __attribute__((always_inline)) {
    constexpr bool kH = decltype(fp16)::value;
    const ExactBf16Unpacker unpack;
    const CodeUnpacker unpack16;
#pragma unroll
    for (int j = 0; j < kBatchGroups; ++j) {
      if (4 * j >= nb) break;   // wave-uniform
      uint32_t sg[SW];          // the group's 4 scales of this lane's row
      if constexpr (STAGED) {
        const uint8_t* src = ss + (wave * 16 + r) * kSRow + j * 4 * (int)sizeof(SP);
        if constexpr (kF32) {
          const uint4 t = *reinterpret_cast<const uint4*>(src);
          sg[0] = t.x; sg[1] = t.y; sg[2] = t.z; sg[3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(src);
          sg[0] = t.x; sg[1] = t.y;
        }
      } else {
#pragma unroll
        for (int q = 0; q < SW; ++q) sg[q] = sraw[j][q];
      }
      transpose_groups(codes[j]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 4 * j + q;
        if (b >= nb) break;
        const uint4 au = xa[batch_unit(b, g, r)];
        f32x4v p;
        if constexpr (kH) {
          half2v hp[4];
          unpack16(codes[j][q], hp);
          p = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8v, au),
                                                     __builtin_bit_cast(f16x8v, hp), zero, 0, 0, 0);
        } else {
          const bf16x8v w = codes_to_bf16(codes[j][q], unpack);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, au), w, zero, 0,
                                                      0, 0);
        }
        float sc;
        if constexpr (SW == 4) sc = __builtin_bit_cast(float, sg[q]);
        else sc = (float)__builtin_bit_cast(half2v, sg[q >> 1])[q & 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sc, p[e], acc[e]);
      }
    }
  };
  if (h16) {
    groups(std::true_type{});
    const float back = pow2f(e16);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= back;
  } else {
    groups(std::false_type{});
  }
  // lane (r, g) holds rows 4 g .. 4 g + 3 of column n
  if (n >= N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t m = 4 * g + e;
    if (m >= M) break;
    if (gridDim.y > 1) partial[((int64_t)blockIdx.y * M + m) * N + n] = acc[e];
    else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[e]);
    else static_cast<float*>(y)[m * N + n] = acc[e];
  }
}

namespace {

// K slices of the workspace kernel (0: not taken): one per kBatchBlocks
// blocks, for 3 <= M <= 16 and rows of 2 .. kBatchMaxSlices slices.
int64_t batch_slices(int64_t M, int64_t K) {
  if (M < 3 || M > 16 || K % kBlock != 0) return 0;
  const int64_t s = (K / kBlock + kBatchBlocks - 1) / kBatchBlocks;
  return s >= 2 && s <= kBatchMaxSlices ? s : 0;
}

template <typename SP>
hipError_t launch_batch(const uint16_t* x, const uint8_t* wq, const SP* ws, void* y, bool y_bf16,
                        int64_t M, int64_t N, int64_t K, float* partial, hipStream_t stream) {
  const int64_t slices = batch_slices(M, K);
  const int64_t gx = (N + 16 * kBatchWaves - 1) / (16 * kBatchWaves);
  if (slices == 0 || gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)slices);
  const int64_t bpr = K / kBlock;
  constexpr int64_t kStagedAlign = 16 / sizeof(SP);   // scales per 16 bytes
  if (bpr % kStagedAlign == 0 && bpr % 4 == 0)
    batch_kernel<true, true, SP><<<grid, dim3(kBatchWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, partial);
  else if (bpr % 4 == 0)
    batch_kernel<true, false, SP><<<grid, dim3(kBatchWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, partial);
  else
    batch_kernel<false, false, SP><<<grid, dim3(kBatchWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, partial);
  const hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  return launch_slice_combine(partial, y, y_bf16, M * N, slices, stream);
}

}  // namespace

namespace {

#ifndef Q4_SMALL_SPLIT_WGS
#define Q4_SMALL_SPLIT_WGS 1024
#endif
// Workgroups a cut call aims for (four per CU).
constexpr int64_t kSmallSplitWgs = Q4_SMALL_SPLIT_WGS;

int64_t small_groups(int64_t M) { return M <= 16 ? 1 : 2; }

// Slice plan: slices * per >= groups, per a multiple of kWaves * kDepth.
void small_plan(int64_t M, int64_t N, int64_t K, bool cut, int64_t* slices, int64_t* per) {
  const int64_t groups = (K / 32 + 3) / 4;
  *slices = 1;
  *per = groups;
  if (!cut || M <= 0 || N <= 0 || K % 32 != 0) return;
  const int64_t mg = small_groups(M);
  const int64_t wgs = ((N + 16 * kNg - 1) / (16 * kNg)) * ((M + 16 * mg - 1) / (16 * mg));
  if (wgs >= kSmallSplitWgs) return;
  constexpr int64_t unit = kWaves * kDepth;
  const int64_t target = (kSmallSplitWgs + wgs - 1) / wgs;
  int64_t p = (groups + target - 1) / target;
  p = (p + unit - 1) / unit * unit;
  const int64_t s = (groups + p - 1) / p;
  if (s < 2) return;
  *slices = s;
  *per = p;
}

template <int MG, bool MX, bool F32S = false>
hipError_t launch_mg(const uint16_t* x, const uint8_t* wq, const void* ws, void* y,
                     bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                     hipStream_t stream) {
  int64_t slices, per;
  small_plan(M, N, K, partial != nullptr, &slices, &per);
  int64_t gpw = (per + kWaves - 1) / kWaves;
  gpw = (gpw + kDepth - 1) / kDepth * kDepth;
  const int64_t gx = (N + 16 * kNg - 1) / (16 * kNg), gy = (M + 16 * MG - 1) / (16 * MG);
  if (gx > 0x7FFFFFFF || gy > 65535 || slices > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)slices);
  float* part = slices > 1 ? partial : nullptr;
  if ((K / 32) % 4 == 0)
    small_kernel<MG, true, MX, F32S><<<grid, dim3(kWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, gpw, per, part);
  else
    small_kernel<MG, false, MX, F32S><<<grid, dim3(kWaves * 64), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, gpw, per, part);
  if (slices == 1) return hipGetLastError();
  const hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  return launch_slice_combine(partial, y, y_bf16, M * N, slices, stream);
}

}  // namespace

int64_t small_split_slices(int64_t M, int64_t N, int64_t K) {
  if (const int64_t b = batch_slices(M, K)) return b;
  int64_t slices, per;
  small_plan(M, N, K, true, &slices, &per);
  return slices;
}

hipError_t launch_small(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                        bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                        hipStream_t stream) {
  if (partial && batch_slices(M, K))
    return launch_batch(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
  if (M <= 16) return launch_mg<1, false>(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
  return launch_mg<2, false>(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_small_f32s(const uint16_t* x, const uint8_t* wq, const float* ws, void* y,
                             bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                             hipStream_t stream) {
  if (partial && batch_slices(M, K))
    return launch_batch(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
  if (M <= 16) return launch_mg<1, false, true>(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
  return launch_mg<2, false, true>(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_small_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                           bool y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M <= 16) return launch_mg<1, true>(x, wq, we, y, y_bf16, M, N, K, nullptr, stream);
  return launch_mg<2, true>(x, wq, we, y, y_bf16, M, N, K, nullptr, stream);
}

}  // namespace q4
