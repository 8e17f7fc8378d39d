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
// of an odd number of blocks ends on a half K step; EVEN: K is a multiple of
// 64, so there is none and no load is clamped).  LDS: activation and weight
// tiles double-buffered, plus the K step's scales as fp32 [row][2], so one
// barrier per K step: the tiles of step t + 1 are written while step t's
// MFMAs read the other buffers.  kt_slice K steps per slice; partial != NULL
// writes the slice's fp32 sums to partial[slice][M][N].
//
// Each wavefront's 64 x 64 outputs are 4 x 4 tiles of 16 x 16, and one
// v_mfma_f32_16x16x32_bf16 forms a tile's partial sum over one 32-element
// block (lane (r, g) = (l % 16, l / 16) gives row r of the A and B operands
// at k = 8 g .. 8 g + 7 and gets rows 4 g .. 4 g + 3, column r of the
// result).  The block's scale is then applied with 4 fmas, two units later:
// the MFMAs of units u + 1 and u + 2 run on the matrix core while unit u's
// fmas run on the vector ALU, and no fma waits for the MFMA it reads.
//
// SP: the block scales' storage -- uint16_t (fp16, the format's own) or float
// (exact fp32 scales, e.g. expanded from super-block scales).
template <typename SP, bool EVEN>
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
  const bool odd = !EVEN && (K % BK) != 0;   // the row's last step holds one block
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
    if (!EVEN && blk >= bpr) blk = bpr - 1;
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

  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};
  f32x4v acc[4][4];   // [16-row group of activations][16-row group of weights]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero;

  a.dma(As[0], wave, 0, odd && kt0 + 1 == steps);
  load_b(0);
  store_b(0);
  __builtin_amdgcn_s_waitcnt(0);   // the tile loads are not tied to registers
  __syncthreads();

  // Per-lane fragment addresses: lane (r, g) reads tile row (16-row group
  // base + r), 16-byte chunk 4 b + g for block b of the step; the swizzle of
  // those rows depends on r only, so the offsets are fixed for the kernel
  // and the row groups and buffers add constants.
  const int r = lane & 15, g = lane >> 4;
  const int sw = (r >> 1) & 7;
  int a_off[2], b_off[2];   // in bf16 elements
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int kc = (4 * b + g) ^ sw;
    a_off[b] = (wm * 64 + r) * 64 + kc * 8;
    b_off[b] = (wn * 64 + r) * 64 + kc * 8;
  }
  const int s_off = (wn * 64 + r) * 2;

  // One K step on buffer CUR (HALF: only its first block): 2 blocks x 16
  // tiles, unit u = (block u / 16, activation group (u / 4) % 4, weight
  // group u % 4).  The loop below is unrolled by two so that every buffer
  // address is a constant offset.
  auto step = [&](int64_t kt, auto cur_c, auto half_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    constexpr bool half = decltype(half_c)::value;
    constexpr int nb = half ? 1 : 2;
    constexpr int units = nb * 16;
    const bool more = kt + 1 < nk;
    f32x2v sc[4];   // [weight group] (block 0, block 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = *reinterpret_cast<const f32x2v*>(&Ss[cur][s_off + j * 32]);
    bf16x8v af[2][4], bfr[2][4];   // [block][16-row group]
#pragma unroll
    for (int b = 0; b < nb; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[b][i] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&As[cur][a_off[b] + i * 16 * 64]));
        bfr[b][i] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&Bs[cur][b_off[b] + i * 16 * 64]));
      }
    // The next step's loads go out after this step's LDS reads: the compiler
    // orders LDS reads after every earlier LDS-bound DMA load (it cannot tell
    // the buffers apart), so issued first they would be waited for here.
    if (more) {
      a.dma(As[cur ^ 1], wave, (kt + 1) * BK, odd && kt0 + kt + 2 == steps);
      load_b(kt + 1);
    }
    // The empty asm statements fix the order (left alone the compiler issues
    // the MFMAs in a burst and the fmas after them, each waiting for its
    // MFMA): a unit's fragments are pinned just before its MFMA, a tile's
    // accumulator right after its fmas.
    auto mm = [&](int u) __attribute__((always_inline)) {
      const int b = u >> 4, i = (u >> 2) & 3, j = u & 3;
      pin(af[b][i]);
      pin(bfr[b][j]);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[b][i], bfr[b][j], zero, 0, 0, 0);
    };
    auto fm = [&](int u, const f32x4v& p) __attribute__((always_inline)) {
      const int b = u >> 4, i = (u >> 2) & 3, j = u & 3;
      const float sv = sc[j][b];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(sv, p[v], acc[i][j][v]);
      pin(acc[i][j]);
    };
    f32x4v p[3];
    p[0] = mm(0);
    p[1] = mm(1);
#pragma unroll
    for (int u = 2; u < units; ++u) {
      p[u % 3] = mm(u);
      fm(u - 2, p[(u - 2) % 3]);
    }
    fm(units - 2, p[(units - 2) % 3]);
    fm(units - 1, p[(units - 1) % 3]);
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
  if constexpr (!EVEN) {
    if (kt < nk) {
      if (kt & 1) step(kt, buf1, half);
      else step(kt, buf0, half);
    }
  }
  // acc[i][j][v]: activation row 16 i + 4 g + v, weight row 16 j + r of the
  // wavefront's 64 x 64
  float* const part = partial ? partial + (int64_t)t.slice * M * N : nullptr;
  const int64_t mw = m0 + wm * 64, nw = n0 + wn * 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = nw + j * 16 + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = mw + i * 16 + 4 * g + v;
        if (m < M) {
          if (part) part[m * N + n] = acc[i][j][v];
          else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[i][j][v]);
          else static_cast<float*>(y)[m * N + n] = acc[i][j][v];
        }
      }
  }
}

// The wide form for more than 128 activation rows, K a multiple of 64: 256
// activation rows x 128 weight rows per workgroup of 16 wavefronts.  Every
// thread converts one dword of codes (8 weights) per K step, so each weight
// is converted once per 256 activation rows; each wavefront owns 32 x 64
// outputs (2 x 4 tiles of 16 x 16), which keeps it within 128 VGPRs: four
// wavefronts per SIMD, where the vector ALU issues from two of them in one
// cycle more often than from two.  The K step is the narrow kernel's (block
// partials by 16 x 16 x 32 MFMAs, scales applied two units later, one
// barrier per step).  All tile loads go through registers -- the compiler
// waits for an LDS-bound load before any later LDS access, so such loads
// could not stay in flight across a step -- the activations one step ahead,
// codes and scales two steps ahead; at the end of each step both tiles of
// the next one are written to the other of two LDS buffers.  LDS: 2 x (32 KB
// + 16 KB) + scales, one workgroup per CU.
constexpr int WM = 256, kWideThreads = 1024;

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4,
// lgkmcnt 11:8): every LDS access done and at most 2 vector loads in flight.
constexpr int kWaitVm2Lgkm0 = 0x72;

// A workgroup barrier without the memory fence of __syncthreads (which
// waits for every load in flight, the prefetches of later steps included):
// the caller has waited for what the other wavefronts must see.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The grid of the wide kernel.  Without a tail plan (full == 0): slices x
// tiles as TileOf numbers them.  With one: the first `full` workgroups (whole
// rounds of the chip, a multiple of 8) take whole tiles, numbered as TileOf
// numbers a grid of `full` tiles, and write y; the remaining tiles of the
// last, partly filled round are cut into `tail_slices` K slices of `tail_kt`
// steps each, one workgroup per (slice, tile), and write their fp32 sums as
// 256 x 128 blocks to tail_part[slice][tile - full].
struct WideTile {
  int tile_m, tile_n;
  int64_t kt0, nk;
  float* tail;   // this workgroup's block of tail_part, or NULL
  __device__ WideTile(int tiles_m, int tiles_n, int64_t steps, int kt_slice, int full,
                      int tail_slices, int tail_kt, float* tail_part) {
    int c, slice = 0;
    int64_t per = kt_slice;
    tail = nullptr;
    if (full > 0 && (int)blockIdx.x >= full) {
      const int tail_tiles = tiles_m * tiles_n - full;
      const int b = (int)blockIdx.x - full;
      slice = b / tail_tiles;
      c = full + (b - slice * tail_tiles);
      per = tail_kt;
      tail = tail_part + ((int64_t)slice * tail_tiles + (c - full)) * (WM * BN);
    } else {
      const int total = full > 0 ? full : tiles_m * tiles_n;
      if (full == 0) slice = (int)(blockIdx.x / (unsigned)total);
      else per = steps;   // whole tiles
      c = (int)blockIdx.x - slice * total;
      if (total % 8 == 0) c = (c % 8) * (total / 8) + c / 8;
    }
    tile_n = c / tiles_m;
    tile_m = c % tiles_m;
    kt0 = (int64_t)slice * per;
    nk = steps - kt0 < per ? steps - kt0 : per;
  }
};

template <typename SP>
__global__ __launch_bounds__(kWideThreads) void gemm_q4_wide_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq, const SP* __restrict__ ws,
    void* __restrict__ y, int y_bf16, int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n,
    int kt_slice, float* __restrict__ partial, int full, int tail_slices, int tail_kt,
    float* __restrict__ tail_part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][WM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
  __shared__ __attribute__((aligned(16))) float Ss[2][BN * 2];
  const int64_t steps = K / BK;
  const WideTile t(tiles_m, tiles_n, steps, kt_slice, full, tail_slices, tail_kt, tail_part);
  const int64_t kt0 = t.kt0, nk = t.nk;
  if (nk <= 0) return;   // the launcher makes no empty slice
  const int64_t kbeg = kt0 * BK;
  const int64_t m0 = (int64_t)t.tile_m * WM, n0 = (int64_t)t.tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bpr = K / 32;
  const int64_t last = nk - 1;

  // Activation staging: thread t moves 16-byte chunk t % 8 of tile rows
  // t / 8 and t / 8 + 128 (rows past M read row M - 1, not stored); the LDS
  // copy is swizzled as in the narrow kernel.
  const int arow = tid >> 3, ach = tid & 7;
  const uint16_t* a_src[2];
  int a_pos[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = arow + 128 * j;
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    a_src[j] = x + m * K + kbeg + ach * 8;
    a_pos[j] = swz(r, ach) * 8;
  }
  u32x4 a_reg[2];

  // Weight staging: thread t takes dword t % 8 (8 codes) of tile row t / 8;
  // threads 0..255 also the scale of block t % 2 of row t / 2 (every thread
  // loads one, so that all wavefronts have the same loads in flight).  Rows
  // past N read row 0 and get scale 0.
  const int brow = tid >> 3, bdw = tid & 7;
  const int64_t bn = n0 + brow;
  const uint8_t* b_src = wq + (bn < N ? bn : 0) * (K / 2) + kbeg / 2 + bdw * 4;
  const int srow = (tid & 255) >> 1, sblk = tid & 1;
  const bool s_ok = n0 + srow < N;
  const SP* s_src = ws + (s_ok ? n0 + srow : 0) * bpr + kbeg / 32 + sblk;
  const bool stages_scale = tid < 256;   // wavefronts 0..3
  const ExactBf16Unpacker unpack;
  uint32_t b_codes[2];
  SP b_scale[2];

  // Loads in issue order: activations of step ka (1 step ahead), then codes
  // and scale of step kb (2 steps ahead, register slot kb % 2).  Past the
  // slice's last step the requests repeat that step (in bounds, unused).
  auto load_a = [&](int64_t ka) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) a_reg[j] = *reinterpret_cast<const u32x4*>(a_src[j] + ka * BK);
  };
  auto load_b = [&](int64_t kb, int slot) __attribute__((always_inline)) {
    b_scale[slot] = s_src[kb * 2];
    b_codes[slot] = *reinterpret_cast<const uint32_t*>(b_src + kb * (BK / 2));
  };
  auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&As[buf][a_pos[j]]) = a_reg[j];
  };
  auto store_b = [&](int buf, int slot) __attribute__((always_inline)) {
    uint32_t o[4];
    unpack(b_codes[slot], o);
    const u32x4 v = {o[0], o[1], o[2], o[3]};
    *reinterpret_cast<u32x4*>(&Bs[buf][swz(brow, bdw) * 8]) = v;
    if (stages_scale) {
      float sv;
      if constexpr (std::is_same<SP, float>::value) sv = b_scale[slot];
      else sv = fp16_to_f32(b_scale[slot]);
      Ss[buf][srow * 2 + sblk] = s_ok ? sv : 0.0f;
    }
  };

  const f32x4v zero = {0.f, 0.f, 0.f, 0.f};
  f32x4v acc[2][4];   // [16-row group of activations][16-row group of weights]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero;

  // step 0 staged; step 1's activations, codes and scales requested
  load_a(0);
  load_b(0, 0);
  load_b(last < 1 ? last : 1, 1);
  store_a(0);
  store_b(0, 0);
  load_a(last < 1 ? last : 1);
  __syncthreads();

  const int r = lane & 15, g = lane >> 4;
  const int sw = (r >> 1) & 7;
  int a_off[2], b_off[2];   // in bf16 elements
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int kc = (4 * b + g) ^ sw;
    a_off[b] = (wm * 32 + r) * 64 + kc * 8;
    b_off[b] = (wn * 64 + r) * 64 + kc * 8;
  }
  const int s_off = (wn * 64 + r) * 2;

  // Step kt computes from buffer kt % 2, requests the codes of step kt + 2
  // (slot kt % 2), writes step kt + 1's activations (requested in step
  // kt - 1) and converted weights to the other buffer (last read in step
  // kt - 1), then requests the activations of step kt + 2.  unit u = (block
  // u / 8, activation group (u / 4) % 2, weight group u % 4); a block's
  // fragments are read from LDS when its first unit comes up.
  auto step = [&](int64_t kt, auto cur_c) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    f32x2v sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = *reinterpret_cast<const f32x2v*>(&Ss[cur][s_off + j * 32]);
    bf16x8v af[2][2], bfr[2][4];
    auto frags = [&](int b) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[b][i] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&As[cur][a_off[b] + i * 16 * 64]));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[b][j] = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const u32x4*>(&Bs[cur][b_off[b] + j * 16 * 64]));
    };
    frags(0);
    const int64_t k2 = kt + 2 < last ? kt + 2 : last;
    load_b(k2, cur);
    auto mm = [&](int u) __attribute__((always_inline)) {
      const int b = u >> 3, i = (u >> 2) & 1, j = u & 3;
      pin(af[b][i]);
      pin(bfr[b][j]);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[b][i], bfr[b][j], zero, 0, 0, 0);
    };
    auto fm = [&](int u, const f32x4v& p) __attribute__((always_inline)) {
      const int b = u >> 3, i = (u >> 2) & 1, j = u & 3;
      const float sv = sc[j][b];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(sv, p[v], acc[i][j][v]);
      pin(acc[i][j]);
    };
    constexpr int units = 16;
    f32x4v p[3];
    p[0] = mm(0);
    p[1] = mm(1);
#pragma unroll
    for (int u = 2; u < units; ++u) {
      if (u == 8) frags(1);
      p[u % 3] = mm(u);
      fm(u - 2, p[(u - 2) % 3]);
    }
    fm(units - 2, p[(units - 2) % 3]);
    fm(units - 1, p[(units - 1) % 3]);
    store_a(cur ^ 1);
    store_b(cur ^ 1, cur ^ 1);
    load_a(k2);
    // this step's LDS writes done; the loads just issued stay in flight
    __builtin_amdgcn_s_waitcnt(kWaitVm2Lgkm0);
    barrier_only();
  };
  const std::integral_constant<int, 0> buf0;
  const std::integral_constant<int, 1> buf1;
  int64_t kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, buf0);
    step(kt + 1, buf1);
  }
  if (kt < nk) step(kt, buf0);

  // acc[i][j][v]: activation row 32 wm + 16 i + 4 g + v, weight row
  // 64 wn + 16 j + r of the tile
  if (t.tail) {
    // the whole 256 x 128 block (rows and columns past M and N hold sums of
    // repeated rows; the combine skips them)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          t.tail[(wm * 32 + i * 16 + 4 * g + v) * BN + wn * 64 + j * 16 + r] = acc[i][j][v];
    return;
  }
  const int64_t slice = kt_slice > 0 ? kt0 / kt_slice : 0;
  float* const part = partial ? partial + slice * M * N : nullptr;
  const int64_t mw = m0 + wm * 32, nw = n0 + wn * 64;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = nw + j * 16 + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = mw + i * 16 + 4 * g + v;
        if (m < M) {
          if (part) part[m * N + n] = acc[i][j][v];
          else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[i][j][v]);
          else static_cast<float*>(y)[m * N + n] = acc[i][j][v];
        }
      }
  }
}

// The tail tiles' slices summed in order into y: one workgroup per 1024
// entries of a 256 x 128 block, four consecutive entries (one row) a thread.
__global__ __launch_bounds__(256) void wide_tail_combine_kernel(const float* __restrict__ part,
                                                                void* __restrict__ y, int y_bf16,
                                                                int64_t M, int64_t N, int tiles_m,
                                                                int full, int tail_tiles,
                                                                int slices) {
  constexpr int kChunks = WM * BN / 1024;
  const int ti = (int)blockIdx.x / kChunks, chunk = (int)blockIdx.x % kChunks;
  const int c = full + ti;
  const int64_t m0 = (int64_t)(c % tiles_m) * WM, n0 = (int64_t)(c / tiles_m) * BN;
  const int e = chunk * 1024 + (int)threadIdx.x * 4;
  const int64_t m = m0 + e / BN, n = n0 + e % BN;
  if (m >= M) return;
  const int64_t block = (int64_t)WM * BN;
  const f32x4v acc = sum_slices<16>(reinterpret_cast<const f32x4v*>(part + ti * block + e),
                                    tail_tiles * block / 4, slices);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (n + q >= N) break;
    if (y_bf16) static_cast<uint16_t*>(y)[m * N + n + q] = to_bf16(acc[q]);
    else static_cast<float*>(y)[m * N + n + q] = acc[q];
  }
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

// y[i] = sum over slices s = 0 .. slices-1, in order, of partial[s][i].
__global__ __launch_bounds__(256) void gemm_combine_kernel(const float* __restrict__ partial,
                                                           void* __restrict__ y, int y_bf16,
                                                           int64_t MN, int slices) {
  // one output per thread, so that every slice's load is in flight at once
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  const float acc = sum_slices<32>(partial + i, MN, slices);
  if (y_bf16) static_cast<uint16_t*>(y)[i] = to_bf16(acc);
  else static_cast<float*>(y)[i] = acc;
}

hipError_t launch_slice_combine(const float* partial, void* y, bool y_bf16, int64_t MN,
                                 int64_t slices, hipStream_t stream) {
  const int64_t grid = (MN + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, partial, y,
                     y_bf16 ? 1 : 0, MN, (int)slices);
  return hipPeekAtLastError();
}

// Workgroup slots the tiled kernels have on the chip: the narrow kernels
// (128 activation rows) about 3 per CU, the wide one 1 per CU; a grid with
// fewer tiles than 2/3 of its slots is cut along K into slices (at least 8 K
// steps each) when the caller gives a workspace.
#ifndef Q4_GEMM_SPLIT_SLOTS
#define Q4_GEMM_SPLIT_SLOTS 768
#endif
#ifndef Q4_GEMM_WIDE_SPLIT_SLOTS
#define Q4_GEMM_WIDE_SPLIT_SLOTS 256
#endif

namespace {
int64_t split_slices_for(int64_t M, int64_t N, int64_t K, int64_t bm, int64_t slots) {
  if (M <= 0 || N <= 0 || K % BK != 0) return 1;
  const int64_t tm = (M + bm - 1) / bm, tn = (N + BN - 1) / BN;
  if (tm >= 512 || tn >= 512) return 1;   // never cut; keeps the product in range
  const int64_t tiles = tm * tn;
  if (tiles * 3 >= slots * 2) return 1;
  int64_t s = slots / tiles;
  const int64_t by_k = K / BK / 8;
  if (s > by_k) s = by_k;
  if (s > 64) s = 64;
  if (s < 2) return 1;
  // ceil(kt / s) K steps per slice; as many slices as that needs, so that
  // none is empty
  const int64_t kt = K / BK, per = (kt + s - 1) / s;
  return (kt + per - 1) / per;
}

bool wide_tiles(int64_t M, int64_t K) { return M > BM && K % BK == 0; }
}  // namespace

int64_t gemm_split_slices(int64_t M, int64_t N, int64_t K) {
  return split_slices_for(M, N, K, BM, Q4_GEMM_SPLIT_SLOTS);
}

int64_t gemm_q4_split_slices(int64_t M, int64_t N, int64_t K) {
  return wide_tiles(M, K) ? split_slices_for(M, N, K, WM, Q4_GEMM_WIDE_SPLIT_SLOTS)
                          : gemm_split_slices(M, N, K);
}

// A grid of wide tiles that fills whole rounds of the chip plus a last round
// at most half full leaves most CUs idle for that round: with a workspace,
// the tiles of the last round are cut into K slices (at least 4 steps each)
// so that their workgroups fill it.  full == 0: no plan.
namespace {
struct TailPlan {
  int64_t full = 0, tail = 0, slices = 0, kt = 0;
};

TailPlan wide_tail_plan(int64_t M, int64_t N, int64_t K) {
  TailPlan p;
  if (!wide_tiles(M, K) || N <= 0 || gemm_q4_split_slices(M, N, K) > 1) return p;
  const int64_t slots = Q4_GEMM_WIDE_SPLIT_SLOTS;
  const int64_t tm = (M + WM - 1) / WM, tn = (N + BN - 1) / BN;
  if (tm >= (int64_t(1) << 20) || tn >= (int64_t(1) << 20)) return p;
  const int64_t tiles = tm * tn, rounds = tiles / slots, tail = tiles - rounds * slots;
  if (rounds == 0 || tail == 0 || tail * 2 > slots || tiles > 0x7FFFFFF) return p;
  const int64_t steps = K / BK;
  int64_t s = slots / tail;
  if (s > steps / 4) s = steps / 4;
  if (s < 2) return p;
  p.kt = (steps + s - 1) / s;
  p.slices = (steps + p.kt - 1) / p.kt;   // none empty
  p.full = rounds * slots;
  p.tail = tail;
  return p;
}
}  // namespace

size_t gemm_q4_tail_bytes(int64_t M, int64_t N, int64_t K) {
  const TailPlan p = wide_tail_plan(M, N, K);
  return p.full ? (size_t)(p.tail * p.slices) * WM * BN * 4 : 0;
}

namespace {
template <typename Kernel, typename ScaleT>
hipError_t launch_tiled(Kernel kernel, int64_t bm, int threads, int64_t slices, const uint16_t* x,
                        const uint8_t* wq, const ScaleT* ws, void* y, bool y_bf16, int64_t M,
                        int64_t N, int64_t K, float* partial, hipStream_t stream) {
  const int64_t tm = (M + bm - 1) / bm, tn = (N + BN - 1) / BN;
  if (!partial) slices = 1;
  const int64_t steps = (K + BK - 1) / BK;
  const int64_t kt_slice = (steps + slices - 1) / slices;
  // every slice has at least one K step: (slices - 1) * kt_slice < steps
  if (tm * tn > 0x7FFFFFFF || tm * tn * slices > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(tm * tn * slices)), dim3(threads), 0, stream, x, wq,
                     ws, y, y_bf16 ? 1 : 0, M, N, K, (int)tm, (int)tn, (int)kt_slice,
                     slices > 1 ? partial : nullptr);
  if (slices > 1) {
    const hipError_t e = hipPeekAtLastError();
    if (e != hipSuccess) return e;
    return launch_slice_combine(partial, y, y_bf16, M * N, slices, stream);
  }
  return hipPeekAtLastError();
}

template <typename SP>
hipError_t launch_wide(const uint16_t* x, const uint8_t* wq, const SP* ws, void* y, bool y_bf16,
                       int64_t M, int64_t N, int64_t K, float* partial, hipStream_t stream) {
  const TailPlan p = partial ? wide_tail_plan(M, N, K) : TailPlan();
  if (p.full == 0) {
    const int64_t slices = partial ? gemm_q4_split_slices(M, N, K) : 1;
    const int64_t tm = (M + WM - 1) / WM, tn = (N + BN - 1) / BN;
    const int64_t steps = K / BK, kt_slice = (steps + slices - 1) / slices;
    if (tm * tn > 0x7FFFFFFF || tm * tn * slices > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm_q4_wide_kernel<SP>, dim3((unsigned)(tm * tn * slices)),
                       dim3(kWideThreads), 0, stream, x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K,
                       (int)tm, (int)tn, (int)kt_slice, slices > 1 ? partial : nullptr, 0, 0, 0,
                       nullptr);
    if (slices > 1) {
      const hipError_t e = hipPeekAtLastError();
      if (e != hipSuccess) return e;
      return launch_slice_combine(partial, y, y_bf16, M * N, slices, stream);
    }
    return hipPeekAtLastError();
  }
  const int64_t tm = (M + WM - 1) / WM, tn = (N + BN - 1) / BN;
  hipLaunchKernelGGL(gemm_q4_wide_kernel<SP>, dim3((unsigned)(p.full + p.tail * p.slices)),
                     dim3(kWideThreads), 0, stream, x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K,
                     (int)tm, (int)tn, 0, nullptr, (int)p.full, (int)p.slices, (int)p.kt,
                     partial);
  hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(wide_tail_combine_kernel, dim3((unsigned)(p.tail * (WM * BN / 1024))),
                     dim3(256), 0, stream, partial, y, y_bf16 ? 1 : 0, M, N, (int)tm,
                     (int)p.full, (int)p.tail, (int)p.slices);
  return hipPeekAtLastError();
}

template <typename SP>
hipError_t launch_q4_tiled(const uint16_t* x, const uint8_t* wq, const SP* ws, void* y,
                           bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                           hipStream_t stream) {
  if (wide_tiles(M, K)) return launch_wide(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
  const int64_t slices = gemm_q4_split_slices(M, N, K);
  if (K % BK == 0)
    return launch_tiled(gemm_q4_kernel<SP, true>, BM, kThreads, slices, x, wq, ws, y, y_bf16, M,
                        N, K, partial, stream);
  return launch_tiled(gemm_q4_kernel<SP, false>, BM, kThreads, slices, x, wq, ws, y, y_bf16, M,
                      N, K, partial, stream);
}
}  // namespace

hipError_t launch_gemm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream) {
  return launch_q4_tiled(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_gemm_f32s(const uint16_t* x, const uint8_t* wq, const float* ws, void* y,
                            bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                            hipStream_t stream) {
  return launch_q4_tiled(x, wq, ws, y, y_bf16, M, N, K, partial, stream);
}

hipError_t launch_gemm_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                          hipStream_t stream) {
  if (K % BK != 0) return hipErrorInvalidValue;
  return launch_tiled(gemm_mx_kernel, BM, kThreads, gemm_split_slices(M, N, K), x, wq, we, y,
                      y_bf16, M, N, K, partial, stream);
}

}  // namespace q4
