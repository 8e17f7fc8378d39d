// q4_gemm.hip -- many activation rows: weights expanded into LDS + bf16 MFMA.
//
// At prefill shapes every weight is used by hundreds of activation rows, so
// the quantised GEMM of the T0 kernel tier ("spec: specialized model
// runtimes", sections "Architecture", "Feasibility gate" and "Phase 3"'s
// tensor-core GEMM rung) is a dense contraction and belongs on the matrix
// cores.  The pages' own design targets another vendor's block-scaled MMA;
// here the gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16) does the products with
// fp32 accumulation, and the weights enter exactly:
//
//  * int4 codes (gemm_q4_kernel): (c - 8) is a small integer, exact in bf16.
//    The tile holds those integers, each 32-element block's partial sum
//    sum_k x * (c - 8) is two chained MFMAs into a scratch accumulator, and
//    the block's fp16 scale is applied to that partial in fp32 (one fma per
//    output and block) -- the groupwise definition y = sum_b s_b sum_k x (c-8)
//    with no rounding of any weight.  A block of all-8 codes adds exactly 0.
//  * 4-bit float blocks (gemm_mx_kernel): e2m1 * 2^(E-129) is exact in bf16
//    for every E < 255, so the scale is folded into the tile and the sums are
//    multiplied by 4 at the end (an exact power-of-two step).
//
// Tile: 128 (activation rows) x 128 (weight rows) per workgroup of 4
// wavefronts (2 x 2, each 64 x 64 = 2 x 2 MFMA tiles of 32 x 32), K step 64
// (two blocks).  The activation tile goes from global memory straight into
// LDS (global_load_lds_dwordx4: no registers, no LDS store instructions).
// Each thread stages one 32-element weight block per K step (one 128-bit code
// load and one scale).  LDS rows are 128 bytes with an XOR swizzle: 16-byte
// chunk c of row r sits at chunk r*8 + (c ^ ((r >> 1) & 7)), which keeps the
// fragment reads (32 rows at one k offset) free of bank conflicts and lets
// every wavefront's load instruction fill 1 KB of consecutive LDS.
// Workgroups sharing one weight tile are numbered onto the same XCD (same L2).
#include <type_traits>

#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// An empty statement that reads and writes v in VGPRs: the compiler keeps the
// instructions producing v before it and those reading it after, and keeps
// volatile statements in program order, so a chain of these fixes the order
// of otherwise independent register work.  It emits no instruction.
template <typename T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// Workgroup b of a grid of slices x tiles: K slice b / tiles of tile b % tiles,
// with the tiles renumbered so that consecutive ids (which the dispatcher
// sends round robin over the 8 XCDs) give each XCD a contiguous range in which
// the activation-row tiles of one weight tile are adjacent.
struct TileOf {
  int slice, tile_m, tile_n;
  __device__ TileOf(int tiles_m, int tiles_n) {
    const int total = tiles_m * tiles_n;
    slice = (int)(blockIdx.x / (unsigned)total);
    int c = (int)blockIdx.x - slice * total;
    if (total % 8 == 0) c = (c % 8) * (total / 8) + c / 8;
    tile_n = c / tiles_m;
    tile_m = c % tiles_m;
  }
};

// Activation tile staging: wavefront w issues 4 loads j; lane l fills
// physical chunk p = (w*4 + j)*64 + l, i.e. row p/8, logical chunk
// (p%8) ^ swizzle.  Rows past M read row M-1 (their outputs are discarded).
// A half K step (the last 32 k of a row whose K is an odd number of blocks)
// points the chunks of the missing block at the present one: their LDS copy
// is never read.
struct ATile {
  const uint16_t* src[4];
  bool upper[4];
  __device__ ATile(const uint16_t* x, int64_t m0, int64_t M, int64_t K, int64_t kbeg, int wave,
                   int lane) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = (wave * 4 + j) * 64 + lane;
      const int r = p >> 3, cl = (p & 7) ^ ((r >> 1) & 7);
      const int64_t m = m0 + r < M ? m0 + r : M - 1;
      src[j] = x + m * K + kbeg + cl * 8;
      upper[j] = cl >= 4;
    }
  }
  __device__ __forceinline__ void dma(uint16_t* dst, int wave, int64_t k0, bool half) const {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[j] + k0 - (half && upper[j] ? 32 : 0)),
          (__attribute__((address_space(3))) void*)(dst + (wave * 4 + j) * 64 * 8), 16, 0, 0);
  }
};

// Weight staging: thread -> (row srow, block shalf of the K step).  The 128-bit
// LDS stores go out 8 lanes at a time, so every 8 consecutive lanes take rows
// 2q + b (q = 0..3, b fixed) of an 8-row group, both halves: with the XOR
// swizzle their 16-byte chunks fall in 8 distinct bank groups.
__device__ __forceinline__ int stage_row(int tid) {
  const int sl = tid & 63;
  return (tid >> 6) * 32 + ((sl >> 4) << 3) + (((sl >> 1) & 3) << 1) + ((sl >> 3) & 1);
}

// Output store of a 64 x 64 wavefront tile: lane l holds column l % 32 of
// MFMA tile (i, j), rows 8 * (v / 4) + 4 * (l / 32) + (v % 4) for v = 0..15.
__device__ __forceinline__ void store_tile(const f32x16v (&acc)[2][2], void* y, int y_bf16,
                                           float* part, int64_t M, int64_t N, int64_t mw,
                                           int64_t nw, int lane) {
  const int col = lane & 31, rbase = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = nw + j * 32 + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = mw + i * 32 + 8 * (v / 4) + rbase + (v % 4);
        if (m < M) {
          if (part) part[m * N + n] = acc[i][j][v];
          else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[i][j][v]);
          else static_cast<float*>(y)[m * N + n] = acc[i][j][v];
        }
      }
    }
}
}  // namespace

// int4 codes with fp16 block scales, any K that is a multiple of 32 (a row
// of an odd number of blocks ends on a half K step).  LDS: activation and
// weight tiles double-buffered, plus the K step's scales as fp32 [row][2], so
// one barrier per K step: the tiles of step t + 1 are written while step t's
// MFMAs read the other buffers.  kt_slice K steps per slice; partial != NULL
// writes the slice's fp32 sums to partial[slice][M][N].
//
// SP: the block scales' storage -- uint16_t (fp16, the format's own) or float
// (exact fp32 scales, e.g. expanded from super-block scales).
template <typename SP>
__global__ __launch_bounds__(kThreads) void gemm_q4_kernel(const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ wq,
                                                          const SP* __restrict__ ws,
                                                          void* __restrict__ y, int y_bf16,
                                                          int64_t M, int64_t N, int64_t K,
                                                          int tiles_m, int tiles_n, int kt_slice,
                                                          float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
  __shared__ __attribute__((aligned(16))) float Ss[2][BN * 2];
  const TileOf t(tiles_m, tiles_n);
  const int64_t steps = (K + BK - 1) / BK;   // the last one may be a half step
  const int64_t kt0 = (int64_t)t.slice * kt_slice;
  const int64_t nk = steps - kt0 < kt_slice ? steps - kt0 : kt_slice;
  if (nk <= 0) return;   // the launcher makes no empty slice
  const bool odd = (K % BK) != 0;          // the row's last step holds one block
  const int64_t kbeg = kt0 * BK;
  const int64_t m0 = (int64_t)t.tile_m * BM, n0 = (int64_t)t.tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bpr = K / 32;

  const ATile a(x, m0, M, K, kbeg, wave, lane);

  const int srow = stage_row(tid), shalf = tid & 1;
  const int64_t bn = n0 + srow;
  const bool b_ok = bn < N;
  const uint8_t* b_src = wq + (b_ok ? bn : 0) * (K / 2);
  const SP* s_src = ws + (b_ok ? bn : 0) * bpr;
  const ExactBf16Unpacker unpack;
  uint4 b_codes;
  SP b_scale;
  // Unconditional loads (rows past N read row 0, the missing block of a half
  // step reads the row's last block): a load under a branch makes the
  // compiler wait for it inside the branch.
  auto load_b = [&](int64_t kt) __attribute__((always_inline)) {
    int64_t blk = (kbeg / 32) + kt * 2 + shalf;
    if (blk >= bpr) blk = bpr - 1;
    b_codes = *reinterpret_cast<const uint4*>(b_src + blk * 16);
    b_scale = s_src[blk];
  };
  auto store_b = [&](int buf) __attribute__((always_inline)) {
    const uint32_t dw[4] = {b_codes.x, b_codes.y, b_codes.z, b_codes.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o[4];
      unpack(dw[i], o);
      const u32x4 v = {o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4*>(&Bs[buf][swz(srow, shalf * 4 + i) * 8]) = v;
    }
    float sv;
    if constexpr (std::is_same<SP, float>::value) sv = b_scale;
    else sv = fp16_to_f32(b_scale);
    Ss[buf][srow * 2 + shalf] = b_ok ? sv : 0.0f;   // rows past N add zero
  };

  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const f32x16v zero = acc[0][0];

  a.dma(As[0], wave, 0, odd && kt0 + 1 == steps);
  load_b(0);
  store_b(0);
  __builtin_amdgcn_s_waitcnt(0);   // the tile loads are not tied to registers
  __syncthreads();

  // Per-lane fragment addresses: lane l reads row (tile row + l % 32), 16-byte
  // chunk kc = 2 * s + l / 32 for MFMA k step s; the swizzle of those rows
  // depends on l only, so the 4 chunk offsets are fixed for the kernel and the
  // tile rows and buffers add constants.
  const int frow = lane & 31, fh = lane >> 5, col = lane & 31;
  const int sw = (frow >> 1) & 7;
  int a_off[4], b_off[4];   // in bf16 elements
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kc = (2 * s + fh) ^ sw;
    a_off[s] = (wm * 64 + frow) * 64 + kc * 8;
    b_off[s] = (wn * 64 + frow) * 64 + kc * 8;
  }
  const int s_off = (wn * 64 + col) * 2;

  // One K step on buffer CUR (HALF: only its first block).  The step's work
  // is 8 units (block b, MFMA tile (i, j)): two chained MFMAs form the
  // block's partial sum, then 16 fmas add it times the block's scale.  The
  // units are software-pipelined -- unit u + 1's MFMAs are issued before unit
  // u's fmas -- so the wavefront's VALU work runs while its MFMAs execute.
  // The loop below is unrolled by two so that every buffer address is a
  // constant offset.
  auto step = [&](int64_t kt, auto cur_c, auto half_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool half = decltype(half_c)::value;
    constexpr int units = half ? 4 : 8;
    const bool more = kt + 1 < nk;
    f32x2 sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sc[j] = *reinterpret_cast<const f32x2*>(&Ss[cur][s_off + j * 64]);
    bf16x8v af[2][2][2], bfr[2][2][2];   // [block][tile][k step of the block]
#pragma unroll
    for (int b = 0; b < (half ? 1 : 2); ++b)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[b][i][s] = __builtin_bit_cast(
              bf16x8v, *reinterpret_cast<const u32x4*>(&As[cur][a_off[b * 2 + s] + i * 32 * 64]));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[b][j][s] = __builtin_bit_cast(
              bf16x8v, *reinterpret_cast<const u32x4*>(&Bs[cur][b_off[b * 2 + s] + j * 32 * 64]));
      }
    // The next step's loads go out after this step's LDS reads: the compiler
    // orders LDS reads after every earlier LDS-bound DMA load (it cannot tell
    // the buffers apart), so issued first they would be waited for here.
    if (more) {
      a.dma(As[cur ^ 1], wave, (kt + 1) * BK, odd && kt0 + kt + 2 == steps);
      load_b(kt + 1);
    }
    // unit u: block u / 4, tile i = (u / 2) % 2, j = u % 2.  The empty asm
    // statements fix the order (left alone the compiler issues every MFMA of
    // the step first, which keeps 8 partials live and spills, and sinks the
    // fmas past the next tile's staging): a unit's fragments are pinned just
    // before its MFMAs, a tile's accumulators right after its fmas.
    auto mm = [&](int u) __attribute__((always_inline)) {
      const int b = u >> 2, i = (u >> 1) & 1, j = u & 1;
      pin(af[b][i][0]);
      pin(af[b][i][1]);
      pin(bfr[b][j][0]);
      pin(bfr[b][j][1]);
      f32x16v p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][i][0], bfr[b][j][0], zero, 0, 0, 0);
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][i][1], bfr[b][j][1], p, 0, 0, 0);
    };
    auto fm = [&](int u, const f32x16v& p) __attribute__((always_inline)) {
      const int b = u >> 2, i = (u >> 1) & 1, j = u & 1;
      const float sv = sc[j][b];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(sv, p[v], acc[i][j][v]);
      pin(acc[i][j]);
    };
    f32x16v p0 = mm(0), p1;
#pragma unroll
    for (int u = 1; u < units; ++u) {
      if (u & 1) {
        p1 = mm(u);
        fm(u - 1, p0);
      } else {
        p0 = mm(u);
        fm(u - 1, p1);
      }
    }
    fm(units - 1, (units - 1) & 1 ? p1 : p0);
    if (more) store_b(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);   // next activation tile landed in LDS
    __syncthreads();
  };
  const std::integral_constant<int, 0> buf0;
  const std::integral_constant<int, 1> buf1;
  const std::false_type full;
  const std::true_type half;
  // the row's half step, if this slice ends the row, comes last
  const int64_t nfull = odd && kt0 + nk == steps ? nk - 1 : nk;
  int64_t kt = 0;
  for (; kt + 1 < nfull; kt += 2) {
    step(kt, buf0, full);
    step(kt + 1, buf1, full);
  }
  if (kt < nfull) {
    step(kt, buf0, full);
    ++kt;
  }
  if (kt < nk) {
    if (kt & 1) step(kt, buf1, half);
    else step(kt, buf0, half);
  }
  float* const part = partial ? partial + (int64_t)t.slice * M * N : nullptr;
  store_tile(acc, y, y_bf16, part, M, N, m0 + wm * 64, n0 + wn * 64, lane);
}

// 4-bit float blocks (e2m1 elements, one E8M0 byte E per 32 k), K a multiple
// of 64.  The tile holds e2m1 * 2^(E-129) in bf16, exact for every E < 255 (at
// most 1.5*2^127, at least 2^-130, a bf16 subnormal), and the accumulators
// are multiplied by 4 before the store.  For E >= 2 the scaled fp4 -> bf16
// conversion does it in one instruction; that instruction reads its scale as
// a power of two from the fp32 exponent field, so 2^-129 and 2^-128 (fp32
// subnormals) would come out as 2^-127, and those two E take an fp32 multiply
// instead.  The activation tile is double-buffered, the weight tile has one
// buffer (two barriers per K step); the light staging lets the wavefront
// raise its priority for the MFMA stretch of each step.
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ wq,
                                                          const uint8_t* __restrict__ we,
                                                          void* __restrict__ y, int y_bf16,
                                                          int64_t M, int64_t N, int64_t K,
                                                          int tiles_m, int tiles_n, int kt_slice,
                                                          float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * BK];
  const TileOf t(tiles_m, tiles_n);
  const int64_t kbeg = (int64_t)t.slice * kt_slice * BK;
  const int64_t nk = K / BK - kbeg / BK < kt_slice ? K / BK - kbeg / BK : kt_slice;
  if (nk <= 0) return;
  const uint8_t* __restrict__ wsc = we + kbeg / 32;
  const int64_t m0 = (int64_t)t.tile_m * BM, n0 = (int64_t)t.tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bpr = K / 32;
  const ATile a(x, m0, M, K, kbeg, wave, lane);
  const int srow = stage_row(tid), shalf = tid & 1;
  const int64_t bn = n0 + srow;
  const bool b_ok = bn < N;
  const uint8_t* b_src = wq + (b_ok ? bn : 0) * (K / 2) + kbeg / 2;
  const uint8_t* s_src = wsc + (b_ok ? bn : 0) * bpr;
  uint4 b_codes;
  uint32_t b_e;
  auto load_b = [&](int64_t k0) __attribute__((always_inline)) {
    const int64_t blk = k0 / 32 + shalf;
    b_codes = *reinterpret_cast<const uint4*>(b_src + blk * 16);
    b_e = s_src[blk];   // columns past N are never stored
  };
  auto store_b = [&]() __attribute__((always_inline)) {
    const uint32_t dw[4] = {b_codes.x, b_codes.y, b_codes.z, b_codes.w};
    // byte j of a dword holds elements 2j (low nibble) and 2j + 1
    if (b_e >= 2) {
      const float s = __uint_as_float(b_e == 255 ? 0x7FC00000u : (b_e - 2) << 23);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 o;
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw[i], s, 0));
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw[i], s, 1));
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw[i], s, 2));
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw[i], s, 3));
        *reinterpret_cast<u32x4*>(&Bs[swz(srow, shalf * 4 + i) * 8]) = o;
      }
    } else {
      const float s = __uint_as_float(0x00100000u << b_e);   // 2^-129 or 2^-128
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2v v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw[i], 1.0f, 0);
        const f32x2v v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw[i], 1.0f, 1);
        const f32x2v v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw[i], 1.0f, 2);
        const f32x2v v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dw[i], 1.0f, 3);
        u32x4 o;
        o[0] = pack_bf16x2(v0[0] * s, v0[1] * s);
        o[1] = pack_bf16x2(v1[0] * s, v1[1] * s);
        o[2] = pack_bf16x2(v2[0] * s, v2[1] * s);
        o[3] = pack_bf16x2(v3[0] * s, v3[1] * s);
        *reinterpret_cast<u32x4*>(&Bs[swz(srow, shalf * 4 + i) * 8]) = o;
      }
    }
  };
  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  a.dma(As[0], wave, 0, false);
  load_b(0);
  store_b();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int frow = lane & 31, fh = lane >> 5;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const int64_t kn = (kt + 1 < nk ? kt + 1 : kt) * BK;
    a.dma(As[cur ^ 1], wave, kn, false);
    load_b(kn);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8v af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&As[cur][swz(wm * 64 + i * 32 + frow, kk * 2 + fh) * 8]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&Bs[swz(wn * 64 + j * 32 + frow, kk * 2 + fh) * 8]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    store_b();
    __builtin_amdgcn_s_waitcnt(0);   // next activation tile landed in LDS
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] *= 4.0f;
  float* const part = partial ? partial + (int64_t)t.slice * M * N : nullptr;
  store_tile(acc, y, y_bf16, part, M, N, m0 + wm * 64, n0 + wn * 64, lane);
}

// y[i] = sum over slices s = 0 .. slices-1, in order, of partial[s][i]; four
// consecutive outputs per thread (16-byte loads when MN is a multiple of 4).
__global__ __launch_bounds__(256) void gemm_combine_kernel(const float* __restrict__ partial,
                                                           void* __restrict__ y, int y_bf16,
                                                           int64_t MN, int slices) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  if (MN % 4 == 0) {
    f32x4v acc = *reinterpret_cast<const f32x4v*>(partial + i);
    for (int s = 1; s < slices; ++s) acc += *reinterpret_cast<const f32x4v*>(partial + s * MN + i);
    if (y_bf16) {
      uint2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + i) = o;
    } else {
      *reinterpret_cast<f32x4v*>(static_cast<float*>(y) + i) = acc;
    }
    return;
  }
  for (int64_t e = i; e < i + 4 && e < MN; ++e) {
    float acc = partial[e];
    for (int s = 1; s < slices; ++s) acc += partial[s * MN + e];
    if (y_bf16) static_cast<uint16_t*>(y)[e] = to_bf16(acc);
    else static_cast<float*>(y)[e] = acc;
  }
}

// The fp32 slice sums of a cut call into y, enqueued after the product on
// the same stream.
hipError_t launch_slice_combine(const float* partial, void* y, bool y_bf16, int64_t MN,
                                 int64_t slices, hipStream_t stream) {
  const int64_t grid = (MN + 1023) / 1024;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partial, y,
                     y_bf16 ? 1 : 0, MN, (int)slices);
  return hipPeekAtLastError();
}

// Workgroup slots the tiled kernels have on the chip (256 CUs, about 3
// workgroups each); a grid with fewer tiles than 2/3 of that is cut along K
// into slices (at least 8 K steps each) when the caller gives a workspace.
#ifndef Q4_GEMM_SPLIT_SLOTS
#define Q4_GEMM_SPLIT_SLOTS 768
#endif

int64_t gemm_split_slices(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K % BK != 0) return 1;
  const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  if (tm >= 512 || tn >= 512) return 1;   // never cut; keeps the product in range
  const int64_t tiles = tm * tn;
  if (tiles * 3 >= int64_t(Q4_GEMM_SPLIT_SLOTS) * 2) return 1;
  int64_t s = int64_t(Q4_GEMM_SPLIT_SLOTS) / tiles;
  const int64_t by_k = K / BK / 8;
  if (s > by_k) s = by_k;
  if (s > 64) s = 64;
  if (s < 2) return 1;
  // ceil(kt / s) K steps per slice; as many slices as that needs, so that
  // none is empty
  const int64_t kt = K / BK, per = (kt + s - 1) / s;
  return (kt + per - 1) / per;
}

namespace {
template <typename Kernel, typename ScaleT>
hipError_t launch_tiled(Kernel kernel, const uint16_t* x, const uint8_t* wq, const ScaleT* ws,
                        void* y, bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                        hipStream_t stream) {
  const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int64_t slices = partial ? gemm_split_slices(M, N, K) : 1;
  const int64_t steps = (K + BK - 1) / BK;
  const int64_t kt_slice = (steps + slices - 1) / slices;
  // every slice has at least one K step: (slices - 1) * kt_slice < steps
  if (tm * tn > 0x7FFFFFFF || tm * tn * slices > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(tm * tn * slices)), dim3(kThreads), 0, stream, x, wq,
                     ws, y, y_bf16 ? 1 : 0, M, N, K, (int)tm, (int)tn, (int)kt_slice,
                     slices > 1 ? partial : nullptr);
  if (slices > 1) {
    const hipError_t e = hipPeekAtLastError();
    if (e != hipSuccess) return e;
    return launch_slice_combine(partial, y, y_bf16, M * N, slices, stream);
  }
  return hipPeekAtLastError();
}
}  // namespace

hipError_t launch_gemm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream) {
  return launch_tiled(gemm_q4_kernel<uint16_t>, x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_gemm_f32s(const uint16_t* x, const uint8_t* wq, const float* ws, void* y,
                            bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                            hipStream_t stream) {
  return launch_tiled(gemm_q4_kernel<float>, x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_gemm_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                          hipStream_t stream) {
  if (K % BK != 0) return hipErrorInvalidValue;
  return launch_tiled(gemm_mx_kernel, x, wq, we, y, y_bf16, M, N, K, partial, stream);
}

}  // namespace q4
