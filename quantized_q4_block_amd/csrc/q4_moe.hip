// q4_moe.hip -- expert-routed rows: y[t] = sum_j g[t][j] * (x[t] . W_{id[t][j]}).
//
// The routed expert matmul plus weighted sum that the "Layer Package
// Repository Spec" measures on its MoE decode fixture (paragraph on MoE
// expert execution under "Policy Resolution": routed gate/up/down expert
// matmuls are nearly all of a routed FFN layer's time, the matrix-vector
// kernel wins at one token, and a separate weighted-sum op closes the layer).
//
// Three kernels, all on the caller's stream, no host round trip:
//  1. prep (one workgroup): count the (token, slot) pairs per expert,
//     exclusive-scan the counts, list the experts that got any pair, and
//     bucket the pair indices by expert (counting in LDS when the experts
//     fit, else in the workspace).  Everything it writes is rebuilt from
//     scratch on every call (the workspace needs no clearing).  With at
//     most 64 pairs over at most 256 experts the plain routed product skips
//     it: each of its wavefronts finds its expert's pairs from the ids.
//  2. gathered matrix-vector product: one workgroup per (touched expert,
//     16 weight rows).  Each wavefront issues every code and scale load of
//     its 2 rows once, then runs the expert's tokens one after another
//     against those registers (each token's activations staged as fp32 in
//     LDS), writing one fp32 partial row per (token, slot) pair.  Rows
//     longer than the LDS path allows take a chunked kernel that reads the
//     activations from global memory instead.  A token's partial does not
//     depend on which other tokens share the expert.
//  3. weighted sum: y[t][n] = sum over slots j in order of g[t][j] * partial.
// Results are bit-identical from run to run: atomics only assign bucket
// slots (integers), never sum floating point.
#include <atomic>

#include "q4_device.h"
#include "q4_gemv.h"
#include "q4_launch.h"

namespace q4 {

namespace {
constexpr int kPrepThreads = 256;
constexpr int kRowsPerWg = 64;     // weight rows per workgroup (16 per wavefront)
constexpr int kRowsPerWave = 16;
constexpr int kMaxTok = 8;         // tokens per gathered pass
constexpr int kPrepLdsExperts = 4096;   // experts counted in LDS by the prep kernel
// At most this many routed pairs (one per lane of a wavefront) over at most
// this many experts take the plain routed product without the prep kernel.
// (The routed FFN keeps the prep: its two products would each pay the
// direct form's longer prologue, which costs more than the launch saved.)
constexpr int kMoeDirectPairs = 64;
constexpr int kMoeDirectExperts = 256;   // 1 KB owner table per wavefront

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }
}  // namespace

MoeLayout moe_workspace_layout(int64_t T, int64_t topk, int64_t E, int64_t N) {
  const size_t P = (size_t)T * (size_t)topk;
  const size_t A = (size_t)(P < (size_t)E ? P : (size_t)E);
  MoeLayout L;
  size_t o = 0;
  L.counts = o;     o = align_up(o + 4 * (size_t)E);
  L.fill = o;       o = align_up(o + 4 * (size_t)E);
  L.offsets = o;    o = align_up(o + 4 * (size_t)E);
  L.order = o;      o = align_up(o + 4 * P);
  L.active = o;     o = align_up(o + 4 * A);
  L.num_active = o; o = align_up(o + 4);
  // slab list of the grouped product (at its smallest slab)
  const size_t U = (size_t)moe_mm_max_items((int64_t)P, (int64_t)A, moe_mm_rows());
  L.items = o;      o = align_up(o + 8 * U);
  L.num_items = o;  o = align_up(o + 4);
  L.partial = o;    o = align_up(o + 4 * P * (size_t)N);
  L.total = o;
  return L;
}

// Prep with the per-expert counters in LDS (E <= kPrepLdsExperts).  Each
// thread scans a contiguous run of experts, so the active list comes out in
// ascending expert order.
__global__ __launch_bounds__(kPrepThreads) void moe_prep_lds_kernel(
    const int32_t* __restrict__ ids, int64_t P, int64_t E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ order, int32_t* __restrict__ active,
    int32_t* __restrict__ num_active) {
  __shared__ int32_t s_cnt[kPrepLdsExperts];
  __shared__ int32_t s_cur[kPrepLdsExperts];   // bucket cursors
  __shared__ int32_t s_sc[kPrepThreads], s_sa[kPrepThreads];
  const int tid = threadIdx.x;
  const int ne = (int)E;
  for (int e = tid; e < ne; e += kPrepThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int64_t p = tid; p < P; p += kPrepThreads) {
    const int32_t e = ids[p];
    if (e >= 0 && e < ne) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  // per-thread run [lo, hi) of experts; inclusive scan of the run totals
  const int chunk = (ne + kPrepThreads - 1) / kPrepThreads;
  const int lo = tid * chunk < ne ? tid * chunk : ne;
  const int hi = lo + chunk < ne ? lo + chunk : ne;
  int c_sum = 0, a_sum = 0;
  for (int e = lo; e < hi; ++e) {
    c_sum += s_cnt[e];
    a_sum += s_cnt[e] > 0 ? 1 : 0;
  }
  s_sc[tid] = c_sum;
  s_sa[tid] = a_sum;
  __syncthreads();
  for (int off = 1; off < kPrepThreads; off <<= 1) {
    const int vc = tid >= off ? s_sc[tid - off] : 0;
    const int va = tid >= off ? s_sa[tid - off] : 0;
    __syncthreads();
    s_sc[tid] += vc;
    s_sa[tid] += va;
    __syncthreads();
  }
  int c_run = s_sc[tid] - c_sum, a_run = s_sa[tid] - a_sum;
  for (int e = lo; e < hi; ++e) {
    const int c = s_cnt[e];
    counts[e] = c;
    offsets[e] = c_run;
    s_cur[e] = c_run;
    if (c > 0) active[a_run++] = e;
    c_run += c;
  }
  if (tid == kPrepThreads - 1) *num_active = s_sa[tid];
  __syncthreads();
  for (int64_t p = tid; p < P; p += kPrepThreads) {
    const int32_t e = ids[p];
    if (e >= 0 && e < ne) order[atomicAdd(&s_cur[e], 1)] = (int32_t)p;
  }
}

// Prep with the counters in the workspace, for any number of experts.
__global__ __launch_bounds__(kPrepThreads) void moe_prep_kernel(
    const int32_t* __restrict__ ids, int64_t P, int64_t E, int32_t* __restrict__ counts,
    int32_t* __restrict__ fill, int32_t* __restrict__ offsets, int32_t* __restrict__ order,
    int32_t* __restrict__ active, int32_t* __restrict__ num_active) {
  __shared__ int32_t s_cnt[kPrepThreads];
  __shared__ int32_t s_act[kPrepThreads];
  __shared__ int32_t s_base[2];
  const int tid = threadIdx.x;

  for (int64_t e = tid; e < E; e += kPrepThreads) {
    counts[e] = 0;
    fill[e] = 0;
  }
  __threadfence();
  __syncthreads();
  for (int64_t p = tid; p < P; p += kPrepThreads) {
    const int32_t e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  }
  __threadfence();
  __syncthreads();

  if (tid == 0) { s_base[0] = 0; s_base[1] = 0; }
  __syncthreads();
  for (int64_t base = 0; base < E; base += kPrepThreads) {
    const int64_t e = base + tid;
    const int32_t c = e < E ? counts[e] : 0;
    const int32_t a = c > 0 ? 1 : 0;
    s_cnt[tid] = c;
    s_act[tid] = a;
    __syncthreads();
    for (int off = 1; off < kPrepThreads; off <<= 1) {   // inclusive scan
      const int32_t vc = tid >= off ? s_cnt[tid - off] : 0;
      const int32_t va = tid >= off ? s_act[tid - off] : 0;
      __syncthreads();
      s_cnt[tid] += vc;
      s_act[tid] += va;
      __syncthreads();
    }
    if (e < E) {
      offsets[e] = s_base[0] + s_cnt[tid] - c;
      if (a) active[s_base[1] + s_act[tid] - 1] = (int32_t)e;
    }
    __syncthreads();
    if (tid == kPrepThreads - 1) {
      s_base[0] += s_cnt[tid];
      s_base[1] += s_act[tid];
    }
    __syncthreads();
  }
  if (tid == 0) *num_active = s_base[1];
  __threadfence();
  __syncthreads();

  for (int64_t p = tid; p < P; p += kPrepThreads) {
    const int32_t e = ids[p];
    if (e >= 0 && e < E) {
      const int32_t slot = atomicAdd(&fill[e], 1);
      order[offsets[e] + slot] = (int32_t)p;
    }
  }
}

template <int M>
__device__ __forceinline__ void moe_rows(const uint16_t* __restrict__ x,
                                         const uint8_t* __restrict__ wq_e,
                                         const uint16_t* __restrict__ ws_e,
                                         const int32_t* pairs, int64_t topk,
                                         float* __restrict__ partial, int64_t row0,
                                         int64_t row_end, int64_t N, int64_t K) {
  constexpr int R = GemvRows<M>::R;
  const int lane = threadIdx.x & 63;
  const uint16_t* xrow[M];
  int32_t pr[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    pr[m] = __builtin_amdgcn_readfirstlane(pairs[m]);
    xrow[m] = x + (int64_t)(pr[m] / topk) * K;
  }
  for (int64_t n0 = row0; n0 < row_end; n0 += R) {
    float out[R][M];
    gemv_task<M, R>(xrow, wq_e, ws_e, n0, N - 1, K, out);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (n0 + r < row_end) partial[(int64_t)pr[m] * N + n0 + r] = out[r][m];
    }
  }
}

__global__ __launch_bounds__(256) void moe_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ ws, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ order,
    const int32_t* __restrict__ active, const int32_t* __restrict__ num_active,
    float* __restrict__ partial, int64_t topk, int64_t N, int64_t K) {
  const int slot = blockIdx.y;
  if (slot >= *num_active) return;
  const int32_t e = active[slot];
  const int32_t start = offsets[e];
  const int32_t cnt = counts[e];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWg + wave * kRowsPerWave;
  if (row0 >= N) return;
  const int64_t row_end = row0 + kRowsPerWave < N ? row0 + kRowsPerWave : N;
  const uint8_t* wq_e = wq + (int64_t)e * N * (K / 2);
  const uint16_t* ws_e = ws + (int64_t)e * N * (K / kBlock);

  for (int32_t c0 = 0; c0 < cnt; c0 += kMaxTok) {
    const int32_t* pairs = order + start + c0;
    const int32_t mc = cnt - c0 < kMaxTok ? cnt - c0 : kMaxTok;
    switch (mc) {
      case 1: moe_rows<1>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 2: moe_rows<2>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 3: moe_rows<3>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 4: moe_rows<4>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 5: moe_rows<5>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 6: moe_rows<6>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      case 7: moe_rows<7>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
      default: moe_rows<8>(x, wq_e, ws_e, pairs, topk, partial, row0, row_end, N, K); break;
    }
  }
}

// Gathered product with the expert's rows loaded once: wavefront w of
// workgroup (bx, slot) owns rows n0 = (bx * kLdsWaves + w) * RT ..
// n0 + RT - 1 of expert active[slot]; row geometry fixed at compile
// time as in the dense decode kernel.
//
// MODE selects the activation rows and the output:
//  kRowsPlain  x: bf16 token rows (pair p reads token p / topk); writes the
//              fp32 partial row of pair p;
//  kRowsGlu    the same rows against a gate/up matrix whose rows 2f, 2f+1 are
//              the gate and up rows of unit f (a wavefront's 2 rows are one
//              such pair); writes act[p][f] = silu(gate) * up (fp32), times
//              gates[p] when gates is not NULL;
//  kRowsDown   x: fp32 rows, one per pair (the SwiGLU output); writes the
//              fp32 partial row of pair p.
enum MoeRows { kRowsPlain = 0, kRowsGlu = 1, kRowsDown = 2 };

#ifndef Q4_MOE_SHORT_ROWS
#define Q4_MOE_SHORT_ROWS 4
#endif
// Rows per wavefront task when a row is at most one stage (K <= 2048).
constexpr int kMoeShortRows = Q4_MOE_SHORT_ROWS;

//
// DIRECT (at most 64 routed pairs, E <= kMoeDirectExperts): no routing
// tables.  Every wavefront loads the pairs' expert ids, one per lane (ids
// outside [0, E) take no part, as the prep would drop them), and in an LDS
// table of its own takes the atomic min of the lane index at each id: the
// lowest lane holding each touched expert becomes its representative (the
// same in every wavefront and workgroup).  grid.y picks the slot-th
// representative (a workgroup past the last returns before loading anything
// else), and a ballot of id == e gives the expert's pairs in ascending
// order.  Which slot serves an expert decides no result.  Otherwise grid.y
// is a slot of the active-expert list the prep kernel built.
template <int FULL, int TAIL, int MODE, int RT, bool DIRECT = false>
__global__ __launch_bounds__(kLdsWaves * 64) void moe_lds_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ ws, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ order,
    const int32_t* __restrict__ active, const int32_t* __restrict__ num_active,
    const float* __restrict__ gates, float* __restrict__ partial, int64_t topk, int64_t N,
    int64_t K, int rem, const int32_t* __restrict__ ids = nullptr, int P = 0, int E = 0) {
  constexpr int R = RT;
  static_assert(MODE != kRowsGlu || R == 2, "a gate/up pair is one wavefront task");
  constexpr int S = FULL + (TAIL != kNoTail ? 1 : 0);
  __shared__ float4 xs[S * 8 * kWave];
  __shared__ uint32_t owner[DIRECT ? kLdsWaves : 1][DIRECT ? kMoeDirectExperts : 1];
  const int lane = threadIdx.x & 63;
  int32_t e, start = 0, cnt;
  uint64_t pairs = 0;   // DIRECT: the expert's pairs not yet taken (wave-uniform)
  if constexpr (DIRECT) {
    const int32_t id = lane < P ? ids[lane] : -1;
    const bool valid = id >= 0 && id < E;
    // the wavefront's own table: each step completes (lgkmcnt 0) before the
    // next is issued, so no workgroup barrier is needed
    uint32_t* own = owner[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
    if (valid) own[id] = 0xFFFFFFFFu;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (valid) atomicMin(&own[id], (uint32_t)lane);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    const bool rep = valid && own[id] == (uint32_t)lane;
    const uint64_t reps = __ballot(rep);
    const int slot = blockIdx.y;
    if (slot >= __builtin_popcountll(reps)) return;   // whole workgroup
    const uint32_t below = __builtin_amdgcn_mbcnt_hi(
        (uint32_t)(reps >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)reps, 0u));
    const int src = __builtin_ctzll(__ballot(rep && below == (uint32_t)slot));
    e = __builtin_amdgcn_readlane(id, src);
    pairs = __ballot(id == e);
    cnt = __builtin_popcountll(pairs);
  } else {
    const int slot = blockIdx.y;
    // the active count and this slot's expert in one round trip (grid.y is
    // the length of the active list, so the read is in bounds)
    const int na = *num_active;
    e = active[slot];
    asm volatile("" :: "s"(e), "s"(na));
    if (slot >= na) return;                        // whole workgroup
    start = offsets[e];
    cnt = counts[e];
  }
  // next pair of the expert, in order
  auto next_pair = [&](int32_t i) __attribute__((always_inline)) -> int32_t {
    if constexpr (DIRECT) {
      const int32_t q = (int32_t)__builtin_ctzll(pairs);
      pairs &= pairs - 1;
      return q;
    } else {
      return order[start + i];
    }
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = ((int64_t)blockIdx.x * kLdsWaves + wave) * R;
  const bool live = n0 < N;
  const int64_t nl = live ? n0 : N - 1;
  const int room = (int)((N - 1 - nl) < R ? (N - 1 - nl) : R);
  const uint8_t* wq_e = wq + (int64_t)e * N * (K / 2);
  const uint16_t* ws_e = ws + (int64_t)e * N * (K / kBlock);
  // the weight loads go out as soon as the expert is known; the first pair's
  // activation loads follow once its index has come back from the bucket
  using Stager = typename std::conditional<MODE == kRowsDown, XStagerF32<S, kLdsWaves * 64>,
                                           XStager<1, S, kLdsWaves * 64>>::type;
  Stager xst;
  auto stage = [&](int32_t pp) __attribute__((always_inline)) {
    if constexpr (MODE == kRowsDown)
      xst.load(static_cast<const float*>(xv) + (int64_t)pp * K, K);
    else
      xst.load(static_cast<const uint16_t*>(xv) + (int64_t)(pp / topk) * K, K, K);
  };
  const uint32_t row_bytes = (uint32_t)(K / 2), row_sc = (uint32_t)(K / kBlock);
  UpfrontLoads<R, FULL, TAIL> b;
  upfront_load<R, FULL, TAIL>(b, wq_e + nl * (int64_t)row_bytes, ws_e + nl * (int64_t)row_sc,
                              row_bytes, row_sc, room, rem, lane, row_sc);
  __builtin_amdgcn_sched_barrier(0);
  int32_t p = next_pair(0);   // an active expert has at least one pair
  stage(p);
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the staging
  xst.pin();
  for (int32_t i = 0; i < cnt; ++i) {
    if (i > 0) {
      p = next_pair(i);
      stage(p);
      __syncthreads();                             // xs no longer read
    }
    // fp32 activations: one compute path keeps the register count (and with
    // it the occupancy) of this token loop low
    xst.store_f32(xs);
    __syncthreads();
    float out[R][1];   // computed by all waves (no load sinking)
    upfront_compute<1, R, FULL, TAIL>(b, xs, rem, lane, out);
    if (live) {
      if (lane == 0) {
        if constexpr (MODE == kRowsGlu) {
          const float g = out[0][0], u = out[1][0];
          float a = g / (1.0f + expf(-g)) * u;
          if (gates != nullptr) a *= gates[p];   // route weight before the down product
          partial[(int64_t)p * (N / 2) + n0 / 2] = a;
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r)
            if (n0 + r < N) partial[(int64_t)p * N + n0 + r] = out[r][0];
        }
      }
    }
  }
}

// y[t][n] = sum_j g[t][j] * partial[t * topk + j][n], j ascending; slots
// with an id outside [0, E) add nothing.  The ids, gates and partials of
// eight slots are loaded before any is used.
// With gates NULL the partials already carry their route weights and are
// added as they are.
__global__ __launch_bounds__(256) void moe_combine_kernel(const int32_t* __restrict__ ids,
                                                          const float* __restrict__ gates,
                                                          const float* __restrict__ partial,
                                                          float* __restrict__ y, int64_t T,
                                                          int64_t topk, int64_t E, int64_t N) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T * N; i += stride) {
    const int64_t t = i / N, n = i - t * N;
    float acc = 0.0f;
    for (int64_t j0 = 0; j0 < topk; j0 += 8) {
      int32_t e[8];
      float g[8], v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int64_t j = j0 + jj < topk ? j0 + jj : topk - 1;   // in bounds
        const int64_t p = t * topk + j;
        e[jj] = ids[p];
        g[jj] = gates != nullptr ? gates[p] : 1.0f;
        v[jj] = partial[p * N + n];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < topk && e[jj] >= 0 && e[jj] < E) acc = __builtin_fmaf(g[jj], v[jj], acc);
    }
    y[i] = acc;
  }
}

namespace {

struct MoeBuffers {
  int32_t *counts, *fill, *offsets, *order, *active, *num_active, *items, *num_items;
};

MoeBuffers moe_buffers(void* workspace, const MoeLayout& L) {
  char* w = static_cast<char*>(workspace);
  return {reinterpret_cast<int32_t*>(w + L.counts), reinterpret_cast<int32_t*>(w + L.fill),
          reinterpret_cast<int32_t*>(w + L.offsets), reinterpret_cast<int32_t*>(w + L.order),
          reinterpret_cast<int32_t*>(w + L.active), reinterpret_cast<int32_t*>(w + L.num_active),
          reinterpret_cast<int32_t*>(w + L.items), reinterpret_cast<int32_t*>(w + L.num_items)};
}

// The slab list for the grouped product; its tables and list bound.
hipError_t moe_grouped_items(const MoeBuffers& b, int tm, hipStream_t stream) {
  return launch_moe_items(b.counts, b.active, b.num_active, b.items, b.num_items, tm, stream);
}

MoeMmTables moe_tables(const MoeBuffers& b) {
  return {b.counts, b.offsets, b.order, b.items, b.num_items};
}

hipError_t moe_prep(const int32_t* ids, int64_t P, int64_t E, const MoeBuffers& b,
                    hipStream_t stream) {
  if (E <= kPrepLdsExperts)
    moe_prep_lds_kernel<<<dim3(1), dim3(kPrepThreads), 0, stream>>>(
        ids, P, E, b.counts, b.offsets, b.order, b.active, b.num_active);
  else
    moe_prep_kernel<<<dim3(1), dim3(kPrepThreads), 0, stream>>>(
        ids, P, E, b.counts, b.fill, b.offsets, b.order, b.active, b.num_active);
  return hipGetLastError();
}

bool moe_direct(int64_t P, int64_t E, int64_t K) {
  return P <= kMoeDirectPairs && E <= kMoeDirectExperts && x_stages(K) <= kLdsMaxStages;
}

// One gathered product over every touched expert (LDS kernel; rows of at
// most kLdsMaxStages stages).  ids != NULL: the DIRECT form (grid.y =
// min(P, E) slots, no prep); otherwise over the prep's active list (grid.y =
// max_active).
template <int MODE>
hipError_t moe_stage_lds(const void* x, const uint8_t* wq, const uint16_t* ws,
                         const MoeBuffers& b, float* out, int64_t topk, int64_t N, int64_t K,
                         int64_t max_active, hipStream_t stream,
                         const float* gates = nullptr, const int32_t* ids = nullptr,
                         int64_t P = 0, int64_t E = 0) {
  const int rem = row_leftover(K);
  return dispatch_row_geometry(K, [&](auto full, auto tail) {
    constexpr int FULL = decltype(full)::value;
    // a row of one (partial) stage is little work for a wavefront: give it
    // more rows, so the activation staging and the reduction are shared by
    // more weight bytes (gate/up tasks stay one gate and one up row)
    constexpr int RT = (MODE != kRowsGlu && FULL == 0) ? kMoeShortRows : kLdsRows;
    const int64_t row_blocks = (N + kLdsWaves * RT - 1) / (kLdsWaves * RT);
    if (row_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    constexpr int TAIL = decltype(tail)::value;
    auto launch = [&](auto tail_kind) __attribute__((always_inline)) {
      constexpr int TK = decltype(tail_kind)::value;
      if (ids != nullptr) {
        const int64_t slots = P < E ? P : E;
        moe_lds_kernel<FULL, TK, MODE, RT, true>
            <<<dim3((unsigned)row_blocks, (unsigned)slots), dim3(kLdsWaves * 64), 0, stream>>>(
                x, wq, ws, nullptr, nullptr, nullptr, nullptr, nullptr, gates, out, topk, N, K,
                rem, ids, (int)P, (int)E);
      } else {
        moe_lds_kernel<FULL, TK, MODE, RT>
            <<<dim3((unsigned)row_blocks, (unsigned)max_active), dim3(kLdsWaves * 64), 0,
               stream>>>(x, wq, ws, b.counts, b.offsets, b.order, b.active, b.num_active, gates,
                         out, topk, N, K, rem);
      }
      return hipGetLastError();
    };
    // 4 rows of a single leftover stage of at most 48 blocks: the flat
    // layout (no idle lanes at 48 blocks)
    if constexpr (FULL == 0 && TAIL == kWideTail && RT % 4 == 0)
      if (rem <= kFlatMaxBlocks) return launch(std::integral_constant<int, kFlatTail>{});
    return launch(std::integral_constant<int, TAIL>{});
  });
}

hipError_t moe_combine(const int32_t* ids, const float* gates, const float* partial, float* y,
                       int64_t T, int64_t topk, int64_t E, int64_t N, hipStream_t stream) {
  int64_t grid = (T * N + 255) / 256;
  if (grid > 65536) grid = 65536;
  moe_combine_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(ids, gates, partial, y, T,
                                                                     topk, E, N);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                      const int32_t* ids, const float* gates, float* y, int64_t T,
                      int64_t topk, int64_t E, int64_t N, int64_t K, void* workspace,
                      hipStream_t stream) {
  const MoeLayout L = moe_workspace_layout(T, topk, E, N);
  const MoeBuffers b = moe_buffers(workspace, L);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.partial);
  const int64_t P = T * topk;
  const int64_t max_active = P < E ? P : E;
  if (max_active > 0 && !moe_use_grouped(P, E) && moe_direct(P, E, K)) {
    const hipError_t err = moe_stage_lds<kRowsPlain>(x, wq, ws, b, partial, topk, N, K, 0,
                                                     stream, nullptr, ids, P, E);
    if (err != hipSuccess) return err;
    return moe_combine(ids, gates, partial, y, T, topk, E, N, stream);
  }
  hipError_t err = moe_prep(ids, P, E, b, stream);
  if (err != hipSuccess) return err;
  if (max_active > 65535) return hipErrorInvalidValue;
  if (max_active > 0 && moe_use_grouped(P, E)) {
    const int tm = moe_mm_rows();
    err = moe_grouped_items(b, tm, stream);
    if (err != hipSuccess) return err;
    err = launch_moe_mm(x, wq, ws, moe_tables(b), partial, moe_mm_max_items(P, max_active, tm),
                        topk, N, K, stream);
    if (err != hipSuccess) return err;
  } else if (max_active > 0) {
    if (x_stages(K) <= kLdsMaxStages) {
      err = moe_stage_lds<kRowsPlain>(x, wq, ws, b, partial, topk, N, K, max_active, stream);
    } else {
      const int64_t row_blocks = (N + kRowsPerWg - 1) / kRowsPerWg;
      if (row_blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
      moe_gemv_kernel<<<dim3((unsigned)row_blocks, (unsigned)max_active), dim3(256), 0, stream>>>(
          x, wq, ws, b.counts, b.offsets, b.order, b.active, b.num_active, partial, topk, N, K);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
  }
  return moe_combine(ids, gates, partial, y, T, topk, E, N, stream);
}

// ---- the MoE call without a caller-owned workspace --------------------------
//
// For callers that cannot allocate device memory: the workspace lives in this
// file-scope array, one copy per GPU, held until the process ends.  Every call
// on a GPU shares that GPU's copy (calls that overlap on one GPU race); the
// prep kernel rebuilds everything the later kernels read on every call, so
// nothing needs clearing.  In host code the name `scratch` is a host-side
// stand-in, not a device address: the device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) on
// its first call and kept per device.
static __device__ __align__(256) unsigned char scratch[kMoeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
}  // namespace

hipError_t moe_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_moe_noalloc(const uint16_t* x, const uint8_t* wq, const uint16_t* ws,
                              const int32_t* ids, const float* gates, float* y, int64_t T,
                              int64_t topk, int64_t E, int64_t N, int64_t K, hipStream_t stream) {
  if (moe_workspace_layout(T, topk, E, N).total > kMoeScratchBytes) return hipErrorInvalidValue;
  void* p = nullptr;
  const hipError_t e = moe_scratch_address(&p);
  if (e != hipSuccess) return e;
  return launch_moe(x, wq, ws, ids, gates, y, T, topk, E, N, K, p, stream);
}

MoeFfnLayout moe_ffn_workspace_layout(int64_t T, int64_t topk, int64_t E, int64_t H,
                                      int64_t F) {
  MoeFfnLayout L;
  L.base = moe_workspace_layout(T, topk, E, H);
  L.act = L.base.total;
  L.total = align_up(L.act + 4 * (size_t)T * (size_t)topk * (size_t)F);
  return L;
}

// Routed expert FFN: prep, gate/up product with the SwiGLU in its store
// (act[p][f], fp32), down product over the same buckets with act as the
// activation rows, weighted sum.
hipError_t launch_moe_ffn(const uint16_t* x, const uint8_t* w13q, const uint16_t* w13s,
                          const uint8_t* w2q, const uint16_t* w2s, const int32_t* ids,
                          const float* gates, float* y, int64_t T, int64_t topk, int64_t E,
                          int64_t H, int64_t F, bool weighted_down, void* workspace,
                          hipStream_t stream) {
  // weighted_down: the route weights multiply the SwiGLU outputs, so the
  // down products come out weighted and the final sum adds them unweighted
  const float* act_gates = weighted_down ? gates : nullptr;
  const float* sum_gates = weighted_down ? nullptr : gates;
  const MoeFfnLayout L = moe_ffn_workspace_layout(T, topk, E, H, F);
  const MoeBuffers b = moe_buffers(workspace, L.base);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.base.partial);
  float* act = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.act);
  const int64_t P = T * topk;
  const int64_t max_active = P < E ? P : E;
  if (x_stages(H) > kLdsMaxStages || x_stages(F) > kLdsMaxStages) return hipErrorInvalidValue;
  hipError_t err = moe_prep(ids, P, E, b, stream);
  if (err != hipSuccess) return err;
  if (max_active > 65535) return hipErrorInvalidValue;
  if (max_active > 0 && moe_use_grouped(P, E)) {
    // act as bf16 hi [P][F] then lo [P][F]: the same bytes as fp32 [P][F]
    uint16_t* act_hi = reinterpret_cast<uint16_t*>(act);
    uint16_t* act_lo = act_hi + P * F;
    const int tm = moe_mm_rows();
    const int64_t max_items = moe_mm_max_items(P, max_active, tm);
    err = moe_grouped_items(b, tm, stream);
    if (err != hipSuccess) return err;
    err = launch_moe_mm_glu(x, w13q, w13s, moe_tables(b), act_gates, act_hi, act_lo, max_items,
                            topk, F, H, stream);
    if (err != hipSuccess) return err;
    err = launch_moe_mm_down(act_hi, act_lo, w2q, w2s, moe_tables(b), partial, max_items, H, F,
                             stream);
    if (err != hipSuccess) return err;
  } else if (max_active > 0) {
    err = moe_stage_lds<kRowsGlu>(x, w13q, w13s, b, act, topk, 2 * F, H, max_active, stream,
                                  act_gates);
    if (err != hipSuccess) return err;
    err = moe_stage_lds<kRowsDown>(act, w2q, w2s, b, partial, 1, H, F, max_active, stream);
    if (err != hipSuccess) return err;
  }
  return moe_combine(ids, sum_gates, partial, y, T, topk, E, H, stream);
}

}  // namespace q4
