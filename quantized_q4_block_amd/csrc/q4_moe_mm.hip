// q4_moe_mm.hip -- routed expert rows with many pairs per expert: grouped
// matrix-core tiles over each expert's bucket.
//
// The "Layer Package Repository Spec" MoE fixture (paragraph on expert
// execution under "Policy Resolution") sets the expert-indexed
// matrix-matrix product, for batches of routed rows, beside the
// matrix-vector one that wins at a single token.  The gathered
// matrix-vector kernel of q4_moe.hip runs an expert's pairs one after
// another, so its vector-ALU work grows with the pairs per expert; this is
// the matrix-matrix form, for prefill-sized batches.
//
// After the prep kernel has bucketed the (token, slot) pairs by expert, an
// items kernel cuts each touched expert's bucket into slabs of at most 48
// pairs and lists them as (expert, first pair of the slab).  One workgroup
// takes one slab against 128 weight rows of its expert:
//  * the slab's activation rows (gathered: pair p reads token p / topk) are
//    staged through LDS 128 k at a time, double-buffered, so each row is read
//    once per 128 weight rows;
//  * each wavefront owns 32 weight rows (two 16-row groups) over all of K;
//    per 32-element block, (c - 8) is exact in bf16 and one
//    v_mfma_f32_16x16x32_bf16 gives the 16 x 16 partial of 16 slab rows,
//    which the block's fp16 scale multiplies in fp32 (exact weights, as in
//    the few-row kernel).  The codes of a block are converted once per slab
//    and serve all of its pairs;
//  * 16-pair groups of the slab with no pair in them are neither loaded nor
//    multiplied.
// Outputs are per pair: an fp32 partial row for the weighted sum, or, for the
// gate/up product of the routed FFN, silu(gate) * up stored as a bf16 pair
// (hi, lo) whose sum is within 2^-17 of the fp32 value (relative), which the
// down product feeds to the bf16 matrix cores as two exact operands.  Each
// output has one writer and no atomics touch floating point, so results are
// the same from run to run.
#include <type_traits>

#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {

constexpr int kMmWaves = 4;                      // wavefronts per workgroup
constexpr int kMmMg = 3;                         // 16-pair groups per slab
constexpr int kMmRows = 16 * kMmMg;              // pairs per slab
constexpr int kMmNg = 2;                         // 16-row weight groups per wavefront
constexpr int kMmRing = 3;                       // steps of weights in registers
constexpr int kMmCols = kMmWaves * kMmNg * 16;   // weight rows per workgroup
constexpr int kItemsThreads = 256;

enum MmMode { kMmPlain = 0, kMmGlu = 1, kMmSplit = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Before: register j of lane group g (16 lanes) holds E[g][j].
// After:  register j of lane group g holds E[j][g].
__device__ __forceinline__ void transpose_groups(uint32_t v[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[2] = c[1];
  v[1] = d[0];
  v[3] = d[1];
}

}  // namespace

// One workgroup, the active list in ascending order: expert e with c pairs
// gets slabs (e, 0), (e, tm), ... (ceil(c / tm) of them), in the order of the
// active list.
__global__ __launch_bounds__(kItemsThreads) void moe_items_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ active,
    const int32_t* __restrict__ num_active, int32_t* __restrict__ items,
    int32_t* __restrict__ num_items, int tm) {
  __shared__ int32_t s_sum[kItemsThreads];
  __shared__ int32_t s_base;
  const int tid = threadIdx.x;
  const int na = *num_active;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int base = 0; base < na; base += kItemsThreads) {
    const int a = base + tid;
    const int32_t e = a < na ? active[a] : 0;
    const int32_t ns = a < na ? (counts[e] + tm - 1) / tm : 0;
    s_sum[tid] = ns;
    __syncthreads();
    for (int off = 1; off < kItemsThreads; off <<= 1) {   // inclusive scan
      const int32_t v = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += v;
      __syncthreads();
    }
    const int32_t first = s_base + s_sum[tid] - ns;
    for (int32_t j = 0; j < ns; ++j) {
      items[2 * (first + j)] = e;
      items[2 * (first + j) + 1] = j * tm;
    }
    __syncthreads();
    if (tid == kItemsThreads - 1) s_base += s_sum[tid];
    __syncthreads();
  }
  if (tid == 0) *num_items = s_base;
}

// MODE kMmPlain: activation rows a0 [T][K] bf16, pair p reads row p / topk;
//                out: fp32 partial [P][N].
// MODE kMmGlu:   the same rows against gate/up weights (rows 2f, 2f + 1 are
//                the gate and up rows of unit f); out_hi / out_lo: bf16
//                [P][N / 2] with hi + lo ~ silu(gate) * up (times the pair's
//                gate weight when gates is not NULL).
// MODE kMmSplit: activation rows a0 (hi) and a1 (lo) [P][K] bf16, pair p
//                reads row p; each block is two MFMAs (hi, then lo) into one
//                partial; out: fp32 partial [P][N].
// Grid: one workgroup per (slab item, 128 weight rows), item-major.
template <int MODE, bool SCALE4>
__global__ __launch_bounds__(kMmWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void moe_mm_kernel(
    const uint16_t* __restrict__ a0, const uint16_t* __restrict__ a1,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ order, const int32_t* __restrict__ items,
    const int32_t* __restrict__ num_items, const float* __restrict__ gates,
    float* __restrict__ out, uint16_t* __restrict__ out_hi, uint16_t* __restrict__ out_lo,
    int64_t topk, int64_t N, int64_t K, uint32_t col_tiles) {
  constexpr int MG = kMmMg, TM = kMmRows;
  constexpr int NSRC = MODE == kMmSplit ? 2 : 1;
  __shared__ u32x4 As[2][NSRC][TM * 16];   // [buffer][source][row * 16 + swizzled segment]
  __shared__ int32_t s_pair[TM];
  const uint32_t item = blockIdx.x / col_tiles;
  const uint32_t ct = blockIdx.x - item * col_tiles;
  if ((int32_t)item >= *num_items) return;       // whole workgroup
  const int32_t e = items[2 * item], c0 = items[2 * item + 1];
  const int32_t start = offsets[e], cnt = counts[e];
  const int live = cnt - c0 < TM ? cnt - c0 : TM;   // >= 1
  const int lg = (live + 15) >> 4;                  // 16-row groups with a pair
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int64_t bpr = K / 32;
  const int64_t steps = (bpr + 3) / 4;              // 128-k steps

  // Activation staging: thread t moves 16-byte segment (t & 15) of slab rows
  // (t >> 4) + 16 i (groups i with a pair only); rows past the slab's pairs
  // repeat its first pair.
  const int seg = tid & 15, rb = tid >> 4;
  const uint16_t* arow[NSRC][MG];
#pragma unroll
  for (int i = 0; i < MG; ++i) {
    const int row = rb + 16 * i;
    const int32_t p = order[start + c0 + (row < live ? row : 0)];
    const int64_t src = MODE == kMmSplit ? (int64_t)p : (int64_t)p / topk;
    arow[0][i] = a0 + src * K;
    if constexpr (NSRC == 2) arow[1][i] = a1 + src * K;
  }
  if (tid < TM) s_pair[tid] = order[start + c0 + (tid < live ? tid : 0)];

  // This wavefront's weight rows; rows past N read row N - 1 (not stored).
  const int64_t nw = (int64_t)ct * kMmCols + wave * (kMmNg * 16);
  const uint8_t* wq_e = wq + (int64_t)e * N * (K / 2);
  const uint16_t* ws_e = ws + (int64_t)e * N * bpr;
  const uint8_t* wrow[kMmNg];
  const uint16_t* srow[kMmNg];
#pragma unroll
  for (int ng = 0; ng < kMmNg; ++ng) {
    const int64_t n = nw + ng * 16 + r;
    const int64_t nn = n < N ? n : N - 1;
    wrow[ng] = wq_e + nn * (K / 2);
    srow[ng] = ws_e + nn * bpr;
  }
  // Ring of three steps of codes and scales, filled two steps ahead: lane
  // (r, g) loads block 4 s + g of its row (16 bytes) and the row's four fp16
  // scales of the step (kept packed); past the row's end it reads the row's
  // last blocks again (in bounds, skipped when computed).
  uint32_t codes[kMmRing][kMmNg][4];
  uint32_t sc[kMmRing][kMmNg][2];
  auto load_w = [&](int64_t s, auto slot) __attribute__((always_inline)) {
    constexpr int d = decltype(slot)::value;
    int64_t b0 = s * 4;
    if (b0 >= bpr) b0 = (bpr - 1) & ~int64_t(3);
    const int64_t bl = b0 + g < bpr ? b0 + g : bpr - 1;
#pragma unroll
    for (int ng = 0; ng < kMmNg; ++ng) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wrow[ng] + bl * 16);
      codes[d][ng][0] = v[0];
      codes[d][ng][1] = v[1];
      codes[d][ng][2] = v[2];
      codes[d][ng][3] = v[3];
      if constexpr (SCALE4) {
        const u32x2 sv = *reinterpret_cast<const u32x2*>(srow[ng] + b0);
        sc[d][ng][0] = sv[0];
        sc[d][ng][1] = sv[1];
      } else {
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = srow[ng][b0 + j < bpr ? b0 + j : bpr - 1];
        sc[d][ng][0] = h[0] | (h[1] << 16);
        sc[d][ng][1] = h[2] | (h[3] << 16);
      }
    }
  };

  // The main loop and the stores, for LG live 16-row groups (a compile-time
  // count: with a run-time skip of a group's MFMAs the compiler counted the
  // wait states before the reads of an MFMA result on the path that runs the
  // skipped block, not on the path that jumps past it).
  auto run = [&](auto lgc) __attribute__((always_inline)) {
    constexpr int LG = decltype(lgc)::value;
    u32x4 areg[NSRC][LG];
    auto load_a = [&](int64_t s) __attribute__((always_inline)) {
      int64_t koff = s * 128 + 8 * seg;
      if (koff > K - 8) koff = K - 8;   // past the row's end: in bounds, unused
#pragma unroll
      for (int src = 0; src < NSRC; ++src)
#pragma unroll
        for (int i = 0; i < LG; ++i)
          areg[src][i] = *reinterpret_cast<const u32x4*>(arow[src][i] + koff);
    };
    // row & 15 == rb for every row this thread moves
    auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int src = 0; src < NSRC; ++src)
#pragma unroll
        for (int i = 0; i < LG; ++i) As[buf][src][(rb + 16 * i) * 16 + (seg ^ rb)] = areg[src][i];
    };
    const ExactBf16Unpacker unpack;
    const f32x4v zero = {0.f, 0.f, 0.f, 0.f};
    f32x4v acc[kMmNg][LG];
#pragma unroll
    for (int ng = 0; ng < kMmNg; ++ng)
#pragma unroll
      for (int mg = 0; mg < LG; ++mg) acc[ng][mg] = zero;

    // Step s reads ring slot s % 3 and LDS buffer bb = s & 1.
    auto compute = [&](int64_t s, auto slot, int bb) __attribute__((always_inline)) {
      constexpr int d = decltype(slot)::value;
#pragma unroll
      for (int ng = 0; ng < kMmNg; ++ng) transpose_groups(codes[d][ng]);
      auto block = [&](int j) __attribute__((always_inline)) {
        // lane (r, g): slab row 16 mg + r, k = 32 j + 8 g .. + 7 of the step
        bf16x8v af[NSRC][LG];
#pragma unroll
        for (int src = 0; src < NSRC; ++src)
#pragma unroll
          for (int mg = 0; mg < LG; ++mg)
            af[src][mg] = __builtin_bit_cast(bf16x8v, As[bb][src][(mg * 16 + r) * 16 + ((4 * j + g) ^ r)]);
#pragma unroll
        for (int ng = 0; ng < kMmNg; ++ng) {
          uint32_t o[4];
          unpack(codes[d][ng][j], o);
          const u32x4 ov = {o[0], o[1], o[2], o[3]};
          const bf16x8v w = __builtin_bit_cast(bf16x8v, ov);
          const float sj = (float)__builtin_bit_cast(half2v, sc[d][ng][j >> 1])[j & 1];
#pragma unroll
          for (int mg = 0; mg < LG; ++mg) {
            f32x4v p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][mg], w, zero, 0, 0, 0);
            if constexpr (NSRC == 2)
              p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][mg], w, p, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[ng][mg][q] = __builtin_fmaf(sj, p[q], acc[ng][mg][q]);
          }
        }
      };
      // blocks of this step inside the row, again a compile-time count per
      // path, so that every MFMA result is read in the block that made it
      auto blocks = [&](auto nbc) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < decltype(nbc)::value; ++j) block(j);
      };
      const int64_t left = bpr - s * 4;
      if (left >= 4) blocks(std::integral_constant<int, 4>());
      else if (left == 3) blocks(std::integral_constant<int, 3>());
      else if (left == 2) blocks(std::integral_constant<int, 2>());
      else blocks(std::integral_constant<int, 1>());
    };

    // Step s: the activations of step s + 1 and the weights of step s + 2
    // are requested first (in that order: the wait for the activations at
    // the end of the step then leaves the newest weights in flight), step s
    // is computed, and the activations go to the other LDS buffer (last read
    // in step s - 1).
    auto step = [&](int64_t s, auto slot) __attribute__((always_inline)) {
      constexpr int d = decltype(slot)::value;
      const int bb = (int)(s & 1);
      load_a(s + 1);
      load_w(s + 2, std::integral_constant<int, (d + 2) % kMmRing>());
      compute(s, slot, bb);
      store_a(bb ^ 1);
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    load_w(0, I0());
    load_w(1, I1());
    load_a(0);
    store_a(0);
    __syncthreads();
    for (int64_t s = 0; s < steps; s += kMmRing) {
      step(s, I0());
      if (s + 1 >= steps) break;
      step(s + 1, I1());
      if (s + 2 >= steps) break;
      step(s + 2, I2());
    }

    // acc[ng][mg][q]: slab row 16 mg + 4 g + q, weight row nw + 16 ng + r.
    if constexpr (MODE != kMmGlu) {
#pragma unroll
      for (int ng = 0; ng < kMmNg; ++ng) {
        const int64_t n = nw + ng * 16 + r;
#pragma unroll
        for (int mg = 0; mg < LG; ++mg)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = mg * 16 + 4 * g + q;
            if (n < N && m < live) out[(int64_t)s_pair[m] * N + n] = acc[ng][mg][q];
          }
      }
    } else {
      // gate rows are even, up rows odd: lane r ^ 1 holds the partner value
      const int64_t F = N / 2;
#pragma unroll
      for (int ng = 0; ng < kMmNg; ++ng) {
        const int64_t n = nw + ng * 16 + r;
#pragma unroll
        for (int mg = 0; mg < LG; ++mg)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = acc[ng][mg][q];
            const float u = __shfl_xor(v, 1, kWave);
            const int m = mg * 16 + 4 * g + q;
            if ((r & 1) == 0 && n < N && m < live) {
              const int32_t p = s_pair[m];
              float a = v / (1.0f + expf(-v)) * u;
              if (gates != nullptr) a *= gates[p];
              const uint16_t hi = to_bf16(a);
              const float rest = a - __uint_as_float((uint32_t)hi << 16);
              out_hi[(int64_t)p * F + n / 2] = hi;
              out_lo[(int64_t)p * F + n / 2] = to_bf16(rest);
            }
          }
      }
    }
  };
  static_assert(MG == 3, "live-group dispatch is written for three groups");
  if (lg == 3) run(std::integral_constant<int, 3>());
  else if (lg == 2) run(std::integral_constant<int, 2>());
  else run(std::integral_constant<int, 1>());
}

int64_t moe_mm_max_items(int64_t P, int64_t A, int tm) {
  // sum over touched experts of ceil(c / tm) <= (P + A (tm - 1)) / tm
  return (P + A * (tm - 1)) / tm;
}

int moe_mm_rows() { return kMmRows; }

bool moe_use_grouped(int64_t P, int64_t E) {
  const int64_t A = P < E ? P : E;
  return A > 0 && P >= kMoeMmMinPairsPerExpert * A;
}

hipError_t launch_moe_items(const int32_t* counts, const int32_t* active,
                            const int32_t* num_active, int32_t* items, int32_t* num_items,
                            int tm, hipStream_t stream) {
  moe_items_kernel<<<dim3(1), dim3(kItemsThreads), 0, stream>>>(counts, active, num_active,
                                                                items, num_items, tm);
  return hipGetLastError();
}

namespace {

template <int MODE>
hipError_t launch_mm(const uint16_t* a0, const uint16_t* a1, const uint8_t* wq,
                     const uint16_t* ws, const MoeMmTables& t, const float* gates, float* out,
                     uint16_t* out_hi, uint16_t* out_lo, int64_t max_items, int64_t topk,
                     int64_t N, int64_t K, hipStream_t stream) {
  const int64_t col_tiles = (N + kMmCols - 1) / kMmCols;
  if (col_tiles <= 0 || max_items <= 0) return hipSuccess;
  if (col_tiles > 0x7FFFFFFF / max_items) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(col_tiles * max_items));
  if ((K / 32) % 4 == 0)
    moe_mm_kernel<MODE, true><<<grid, dim3(kMmWaves * 64), 0, stream>>>(
        a0, a1, wq, ws, t.counts, t.offsets, t.order, t.items, t.num_items, gates, out, out_hi,
        out_lo, topk, N, K, (uint32_t)col_tiles);
  else
    moe_mm_kernel<MODE, false><<<grid, dim3(kMmWaves * 64), 0, stream>>>(
        a0, a1, wq, ws, t.counts, t.offsets, t.order, t.items, t.num_items, gates, out, out_hi,
        out_lo, topk, N, K, (uint32_t)col_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_mm(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                         const MoeMmTables& t, float* partial, int64_t max_items, int64_t topk,
                         int64_t N, int64_t K, hipStream_t stream) {
  return launch_mm<kMmPlain>(x, nullptr, wq, ws, t, nullptr, partial, nullptr, nullptr,
                             max_items, topk, N, K, stream);
}

hipError_t launch_moe_mm_glu(const uint16_t* x, const uint8_t* w13q, const uint16_t* w13s,
                             const MoeMmTables& t, const float* gates, uint16_t* act_hi,
                             uint16_t* act_lo, int64_t max_items, int64_t topk, int64_t F,
                             int64_t H, hipStream_t stream) {
  return launch_mm<kMmGlu>(x, nullptr, w13q, w13s, t, gates, nullptr, act_hi, act_lo, max_items,
                           topk, 2 * F, H, stream);
}

hipError_t launch_moe_mm_down(const uint16_t* act_hi, const uint16_t* act_lo,
                              const uint8_t* w2q, const uint16_t* w2s, const MoeMmTables& t,
                              float* partial, int64_t max_items, int64_t H, int64_t F,
                              hipStream_t stream) {
  return launch_mm<kMmSplit>(act_hi, act_lo, w2q, w2s, t, nullptr, partial, nullptr, nullptr,
                             max_items, 1, H, F, stream);
}

}  // namespace q4
