// q4_gemm.hip -- prefill path (M > 8): dequant to bf16 in LDS + bf16 MFMA.
//
// At prefill shapes every weight is used by hundreds of activation rows, so
// the quantised GEMM of the T0 kernel tier ("spec: specialized model
// runtimes", sections "Architecture", "Feasibility gate" and "Phase 3"'s
// tensor-core GEMM rung) is a dense contraction and belongs on the matrix
// cores.  The pages' own design targets another vendor's block-scaled MMA;
// here the codes are expanded once per workgroup tile into bf16 in LDS and
// the gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16) does the products with
// fp32 accumulation.
//
// Two kernels with the same tiling: gemm_dma_kernel (K a multiple of 64)
// loads the activation tile straight into LDS, gemm_kernel (any K) through
// registers.
//
// Tile: 128 (activation rows) x 128 (weight rows) per workgroup of 4
// wavefronts (2 x 2, each 64 x 64 = 2 x 2 MFMA 32x32 tiles), K step 64.
// Each thread stages 32 activations (4 x 128-bit loads) and one 32-element
// weight block (one 128-bit code load + one scale) per K step; the weights
// are dequantised -- (c - 8) exact in fp16, times the scale exact in fp32,
// rounded to bf16 nearest-even -- straight into LDS.  The next K step's
// global loads are issued before the current step's MFMAs.  LDS rows are
// padded by 8 bf16 so the 128-bit fragment reads of 8 consecutive rows fall
// in distinct banks.  Workgroups are numbered so that the workgroups sharing
// one weight tile land on the same XCD (same L2).
#include <type_traits>

#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;          // padded LDS row, in bf16
constexpr int kThreads = 256;
}  // namespace

__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint16_t* __restrict__ x,
                                                        const uint8_t* __restrict__ wq,
                                                        const uint16_t* __restrict__ ws,
                                                        void* __restrict__ y, int y_bf16,
                                                        int64_t M, int64_t N, int64_t K,
                                                        int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

  // XCD-aware tile order: consecutive workgroup ids go to different XCDs
  // (round robin over 8), so give each XCD a contiguous range of tiles in
  // which the activation-row tiles of one weight tile are adjacent.
  const int total = tiles_m * tiles_n;
  int c = blockIdx.x;
  if (total % 8 == 0) c = (c % 8) * (total / 8) + c / 8;
  const int tile_n = c / tiles_m;
  const int tile_m = c % tiles_m;
  const int64_t m0 = (int64_t)tile_m * BM;
  const int64_t n0 = (int64_t)tile_n * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Staging assignment: thread -> (row, 32-wide half of the K step).
  const int srow = tid >> 1;
  const int shalf = tid & 1;
  const int64_t bpr = K / kBlock;
  const int64_t am = m0 + srow;
  const int64_t bn = n0 + srow;
  const bool a_ok = am < M;
  const bool b_ok = bn < N;
  const uint16_t* a_src = x + (a_ok ? am : 0) * K;
  const uint8_t* b_src = wq + (b_ok ? bn : 0) * (K / 2);
  const uint16_t* s_src = ws + (b_ok ? bn : 0) * bpr;

  const CodeUnpacker unpack;
  uint4 a_reg[4];
  uint4 b_codes;
  float b_scale;

  auto load_step = [&](int64_t k0) {
    const int64_t blk = k0 / kBlock + shalf;
    const bool in_k = blk < bpr;
    if (a_ok && in_k) {
      const uint4* p = reinterpret_cast<const uint4*>(a_src + blk * kBlock);
#pragma unroll
      for (int q = 0; q < 4; ++q) a_reg[q] = p[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) a_reg[q] = make_uint4(0, 0, 0, 0);
    }
    if (b_ok && in_k) {
      b_codes = *reinterpret_cast<const uint4*>(b_src + blk * 16);
      b_scale = fp16_to_f32(s_src[blk]);
    } else {
      b_codes = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);  // code 8 = 0
      b_scale = 0.0f;
    }
  };

  auto store_step = [&]() {
    uint4* ad = reinterpret_cast<uint4*>(As + srow * LDK + shalf * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) ad[q] = a_reg[q];
    const uint32_t dw[4] = {b_codes.x, b_codes.y, b_codes.z, b_codes.w};
    uint4* bd = reinterpret_cast<uint4*>(Bs + srow * LDK + shalf * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v p[4];
      unpack(dw[i], p);
      // elements 8i..8i+7 are p0.lo p1.lo p2.lo p3.lo p0.hi p1.hi p2.hi p3.hi
      // fma(h, s, 0) with an fp16 h is one v_fma_mix_f32: the widening is
      // folded into the multiply, and the product is exact in fp32
      uint4 o;
      o.x = pack_bf16x2(__builtin_fmaf((float)p[0][0], b_scale, 0.0f),
                        __builtin_fmaf((float)p[1][0], b_scale, 0.0f));
      o.y = pack_bf16x2(__builtin_fmaf((float)p[2][0], b_scale, 0.0f),
                        __builtin_fmaf((float)p[3][0], b_scale, 0.0f));
      o.z = pack_bf16x2(__builtin_fmaf((float)p[0][1], b_scale, 0.0f),
                        __builtin_fmaf((float)p[1][1], b_scale, 0.0f));
      o.w = pack_bf16x2(__builtin_fmaf((float)p[2][1], b_scale, 0.0f),
                        __builtin_fmaf((float)p[3][1], b_scale, 0.0f));
      bd[i] = o;
    }
  };

  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t nk = (K + BK - 1) / BK;
  load_step(0);
  store_step();
  __syncthreads();

  const int frow = lane & 31;          // fragment row within a 32-row MFMA tile
  const int fk = (lane >> 5) * 8;      // fragment k offset within a 16-wide MFMA step

  for (int64_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_step((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8v a_frag[2], b_frag[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + frow) * LDK + kk + fk);
        a_frag[i] = __builtin_bit_cast(bf16x8v, v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 32 + frow) * LDK + kk + fk);
        b_frag[j] = __builtin_bit_cast(bf16x8v, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag[i], b_frag[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      store_step();
      __syncthreads();
    }
  }

  // D layout of a 32x32 MFMA tile: lane l holds column l % 32, rows
  // 8 * (v / 4) + 4 * (l / 32) + (v % 4) for v = 0..15.
  const int col = lane & 31;
  const int rbase = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v / 4) + rbase + (v % 4);
        if (m < M) {
          if (y_bf16)
            static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[i][j][v]);
          else
            static_cast<float*>(y)[m * N + n] = acc[i][j][v];
        }
      }
    }
  }
}

// K a multiple of 64: the activation tile goes global -> LDS directly
// (global_load_lds_dwordx4, no registers, no LDS store instructions) into a
// double buffer, so the next tile streams in during the MFMAs; the
// dequantised weights still pass through registers into one LDS buffer.
// Unpadded 128-byte rows (64 bf16) with an XOR swizzle: 16-byte chunk c of
// row r sits at chunk r*8 + (c ^ ((r >> 1) & 7)), which keeps the fragment
// reads (32 rows at one k offset) free of bank conflicts and lets every
// wavefront's load instruction fill 1 KB of consecutive LDS.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

//
// MX: 4-bit float blocks (e2m1 elements, one E8M0 byte E per 32 k).  The tile
// holds e2m1 * 2^(E-129) in bf16, exact for every E < 255 (at most 1.5*2^127,
// at least 2^-130, a bf16 subnormal), and the accumulators are multiplied by 4
// before the store, an exact power-of-two step.  For E >= 2 the scaled fp4 ->
// bf16 conversion does it in one instruction; that instruction reads its
// scale as a power of two from the fp32 exponent field, so 2^-129 and 2^-128
// (fp32 subnormals) would come out as 2^-127, and those two E take an fp32
// multiply instead.
template <bool MX>
__global__ __launch_bounds__(kThreads) void gemm_dma_kernel(const uint16_t* __restrict__ x,
                                                const uint8_t* __restrict__ wq,
                                                const void* __restrict__ wsv,
                                                void* __restrict__ y, int y_bf16,
                                                int64_t M, int64_t N, int64_t K,
                                                int tiles_m, int tiles_n, int kt_slice,
                                                float* __restrict__ partial) {
  using ScaleT = typename std::conditional<MX, uint8_t, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * 64];
  const int total = tiles_m * tiles_n;
  // workgroup b: K slice b / total (its kt_slice K steps), tile b % total
  const int slice = (int)(blockIdx.x / (unsigned)total);
  int c = (int)blockIdx.x - slice * total;
  if (total % 8 == 0) c = (c % 8) * (total / 8) + c / 8;
  const int64_t kbeg = (int64_t)slice * kt_slice * 64;
  const int64_t nk = K / 64 - kbeg / 64 < kt_slice ? K / 64 - kbeg / 64 : kt_slice;
  if (nk <= 0) return;   // the launcher makes no empty slice
  const ScaleT* __restrict__ ws = static_cast<const ScaleT*>(wsv) + kbeg / 32;
  const int tile_n = c / tiles_m, tile_m = c % tiles_m;
  const int64_t m0 = (int64_t)tile_m * 128, n0 = (int64_t)tile_n * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bpr = K / 32;
  // activation tile: wavefront w issues 4 loads j; lane l fills physical
  // chunk p = (w*4 + j)*64 + l, i.e. row p/8, logical chunk (p%8) ^ swizzle.
  // Rows past M read row M-1 (their outputs are discarded).
  const uint16_t* a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = (wave * 4 + j) * 64 + lane;
    const int r = p >> 3, cl = (p & 7) ^ ((r >> 1) & 7);
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    a_src[j] = x + m * K + kbeg + cl * 8;
  }
  auto dma = [&](int buf, int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(a_src[j] + k0),
          (__attribute__((address_space(3))) void*)(&As[buf][(wave * 4 + j) * 64 * 8]), 16, 0, 0);
  };
  // weight staging: thread -> (row srow, half shalf): one 32-element block;
  // rows past N get scale 0.  The 128-bit LDS stores go out 8 lanes at a
  // time, so every 8 consecutive lanes take rows 2q + b (q = 0..3, b fixed)
  // of an 8-row group, both halves: with the XOR swizzle their 16-byte chunks
  // fall in 8 distinct bank groups (lanes 2i, 2i+1 on rows i would pair up).
  const int sl = tid & 63;
  const int srow = (tid >> 6) * 32 + ((sl >> 4) << 3) + (((sl >> 1) & 3) << 1) + ((sl >> 3) & 1);
  const int shalf = sl & 1;
  const int64_t bn = n0 + srow;
  const bool b_ok = bn < N;
  const uint8_t* b_src = wq + (b_ok ? bn : 0) * (K / 2) + kbeg / 2;
  const ScaleT* s_src = ws + (b_ok ? bn : 0) * bpr;
  const CodeUnpacker unpack;
  uint4 b_codes;
  float b_scale;
  uint32_t b_e;
  auto load_b = [&](int64_t k0) __attribute__((always_inline)) {
    const int64_t blk = k0 / 32 + shalf;
    b_codes = *reinterpret_cast<const uint4*>(b_src + blk * 16);
    if constexpr (MX) b_e = s_src[blk];   // columns past N are never stored
    else b_scale = b_ok ? fp16_to_f32(s_src[blk]) : 0.0f;
  };
  auto store_b = [&]() __attribute__((always_inline)) {
    const uint32_t dw[4] = {b_codes.x, b_codes.y, b_codes.z, b_codes.w};
    if constexpr (MX) {
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
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v p[4];
      unpack(dw[i], p);
      u32x4 o;
      o[0] = pack_bf16x2(__builtin_fmaf((float)p[0][0], b_scale, 0.f), __builtin_fmaf((float)p[1][0], b_scale, 0.f));
      o[1] = pack_bf16x2(__builtin_fmaf((float)p[2][0], b_scale, 0.f), __builtin_fmaf((float)p[3][0], b_scale, 0.f));
      o[2] = pack_bf16x2(__builtin_fmaf((float)p[0][1], b_scale, 0.f), __builtin_fmaf((float)p[1][1], b_scale, 0.f));
      o[3] = pack_bf16x2(__builtin_fmaf((float)p[2][1], b_scale, 0.f), __builtin_fmaf((float)p[3][1], b_scale, 0.f));
      *reinterpret_cast<u32x4*>(&Bs[swz(srow, shalf * 4 + i) * 8]) = o;
    }
  };
  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  dma(0, 0);
  load_b(0);
  store_b();
  __builtin_amdgcn_s_waitcnt(0);   // the tile loads are not tied to registers
  __syncthreads();
  const int frow = lane & 31, fh = lane >> 5;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const int64_t kn = (kt + 1 < nk ? kt + 1 : kt) * 64;
    dma(cur ^ 1, kn);
    load_b(kn);
    // 4-bit float staging is light (4 conversions per 8 weights): raising
    // the wave's priority for its MFMA stretch interleaves the workgroups of
    // a CU better; the int4 staging (21 instructions per 8 weights) is slower
    // with it, so only the MX form does this
    if constexpr (MX) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8v af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + frow;
        af[i] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const u32x4*>(&As[cur][swz(r, kk * 2 + fh) * 8]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + frow;
        bfr[j] = __builtin_bit_cast(bf16x8v, *reinterpret_cast<const u32x4*>(&Bs[swz(r, kk * 2 + fh) * 8]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (MX) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    store_b();
    __builtin_amdgcn_s_waitcnt(0);   // next activation tile landed in LDS
    __syncthreads();
  }
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] *= 4.0f;
  }
  const int col = lane & 31, rbase = (lane >> 5) * 4;
  float* const part = partial ? partial + (int64_t)slice * M * N : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + col;
      if (n >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v / 4) + rbase + (v % 4);
        if (m < M) {
          if (part) part[m * N + n] = acc[i][j][v];
          else if (y_bf16) static_cast<uint16_t*>(y)[m * N + n] = to_bf16(acc[i][j][v]);
          else static_cast<float*>(y)[m * N + n] = acc[i][j][v];
        }
      }
    }
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
static hipError_t launch_combine(const float* partial, void* y, bool y_bf16, int64_t MN,
                                 int64_t slices, hipStream_t stream) {
  const hipError_t e = hipGetLastError();   // the product's launch
  if (e != hipSuccess) return e;
  const int64_t grid = (MN + 1023) / 1024;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  gemm_combine_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(partial, y, y_bf16 ? 1 : 0,
                                                                      MN, (int)slices);
  return hipGetLastError();
}

// Workgroup slots the tiled kernel has on the chip (256 CUs, 3 workgroups
// each); a grid with fewer tiles than 2/3 of that is cut along K into slices
// (at least 8 K steps each) when the caller gives a workspace.
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

hipError_t launch_gemm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws, void* y,
                       bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                       hipStream_t stream) {
  const int64_t tm = (M + BM - 1) / BM;
  const int64_t tn = (N + BN - 1) / BN;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (K % BK == 0) {
    const int64_t slices = partial ? gemm_split_slices(M, N, K) : 1;
    const int64_t kt = K / BK;
    const int64_t kt_slice = (kt + slices - 1) / slices;
    if (tm * tn * slices > 0x7FFFFFFF) return hipErrorInvalidValue;
    gemm_dma_kernel<false><<<dim3((unsigned)(tm * tn * slices)), dim3(kThreads), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, (int)tm, (int)tn, (int)kt_slice,
        slices > 1 ? partial : nullptr);
    // every slice has at least one K step: (slices - 1) * kt_slice < kt
    if (slices > 1) return launch_combine(partial, y, y_bf16, M * N, slices, stream);
  } else
    gemm_kernel<<<dim3((unsigned)(tm * tn)), dim3(kThreads), 0, stream>>>(
        x, wq, ws, y, y_bf16 ? 1 : 0, M, N, K, (int)tm, (int)tn);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint16_t* x, const uint8_t* wq, const uint8_t* we, void* y,
                          bool y_bf16, int64_t M, int64_t N, int64_t K, float* partial,
                          hipStream_t stream) {
  const int64_t tm = (M + BM - 1) / BM;
  const int64_t tn = (N + BN - 1) / BN;
  if (tm * tn > 0x7FFFFFFF || K % BK != 0) return hipErrorInvalidValue;
  const int64_t slices = partial ? gemm_split_slices(M, N, K) : 1;
  const int64_t kt = K / BK;
  const int64_t kt_slice = (kt + slices - 1) / slices;
  if (tm * tn * slices > 0x7FFFFFFF) return hipErrorInvalidValue;
  gemm_dma_kernel<true><<<dim3((unsigned)(tm * tn * slices)), dim3(kThreads), 0, stream>>>(
      x, wq, we, y, y_bf16 ? 1 : 0, M, N, K, (int)tm, (int)tn, (int)kt_slice,
      slices > 1 ? partial : nullptr);
  if (slices > 1) return launch_combine(partial, y, y_bf16, M * N, slices, stream);
  return hipGetLastError();
}

}  // namespace q4
