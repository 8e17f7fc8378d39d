// q4_api.hip -- the C ABI (include/q4.h): argument checks, device check,
// path dispatch, launches.
//
// The conventions follow the spec "spec: specialized model runtimes": a
// runtime is an in-process library behind a C ABI whose version is pinned
// (section "Prototype ABI scope"), failures come back as a clean value the
// caller already handles (same section), and a runtime is only used on the
// exact GPU architecture it was built for (section "Runtime selection",
// condition 3).  Every check here runs on the host before anything is
// enqueued, so an error never leaves partial work or a written output.
#include <atomic>

#include "../../include/q4.h"
#include "q4_launch.h"

namespace {

// Path choice (measured on MI355X; see q4_matmul_path in q4.h):
//  * M <= 2: the matrix-vector kernel streams W at close to HBM rate;
//  * 3 <= M <= 32: the exact-weight matrix-core kernel (the vector kernel is
//    bound by one fma per weight per row from 3 rows on);
//  * M <= 128 while the tiled kernel would have fewer 128 x 128 tiles than
//    the chip has compute units: still the exact-weight kernel, in slabs of
//    32 rows (the tiled kernel would leave most of the chip idle);
//  * otherwise the tiled bf16 kernel.
constexpr int64_t kGemvMaxRows = 2;
constexpr int64_t kSmallMaxRows = 32;
constexpr int64_t kSmallSlabMaxRows = 128;
constexpr int64_t kTiledMinTiles = 256;
constexpr int kMaxDevices = 64;

// 0 = unknown, 1 = gfx950, 2 = other.
std::atomic<int> g_arch[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b without signed overflow, both >= 0; false on overflow past 2^62.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > (int64_t(1) << 62) / a) return false;
  *out = a * b;
  return true;
}

// The current device must be gfx950 (cached per device after the first
// query).  A failed query's error is left as the runtime set it.
int32_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return Q4_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int known = g_arch[dev].load(std::memory_order_relaxed);
    if (known == 1) return Q4_OK;
    if (known == 2) return Q4_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q4_ERR_DEVICE;
  const char* a = prop.gcnArchName;
  const bool ok = a[0] == 'g' && a[1] == 'f' && a[2] == 'x' && a[3] == '9' && a[4] == '5' &&
                  a[5] == '0' && (a[6] == '\0' || a[6] == ':');
  if (dev < kMaxDevices) g_arch[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? Q4_OK : Q4_ERR_DEVICE;
}

int32_t check_weights(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % 32 != 0) return Q4_ERR_SHAPE;
  int64_t nk;
  if (!mul_ok(N, K, &nk)) return Q4_ERR_SHAPE;
  return Q4_OK;
}

// Run right before anything is enqueued: the device check, then a HIP error
// already pending from the caller's own work is left in place (not cleared,
// not taken for this call's) and nothing is launched.
int32_t ready() {
  if (int32_t s = check_device()) return s;
  if (hipPeekAtLastError() != hipSuccess) return Q4_ERR_PENDING;
  return Q4_OK;
}

// Status of the launches: the error state was clean when they were enqueued,
// so an error pending now is theirs; it is consumed here, so no HIP error
// state leaves the call.
int32_t launched(hipError_t e) {
  const hipError_t own = hipGetLastError();
  return e == hipSuccess && own == hipSuccess ? Q4_OK : Q4_ERR_LAUNCH;
}

}  // namespace

extern "C" {

Q4_API int32_t q4_abi_version(void) { return Q4_ABI_VERSION; }

Q4_API const char* q4_status_str(int32_t status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "null pointer argument";
    case Q4_ERR_SHAPE: return "invalid shape (negative size, K not a positive multiple of 32, or overflow)";
    case Q4_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case Q4_ERR_DTYPE: return "unknown output dtype";
    case Q4_ERR_WORKSPACE: return "workspace missing (MoE), misaligned or too small";
    case Q4_ERR_DEVICE: return "no current HIP device or it is not gfx950";
    case Q4_ERR_LAUNCH: return "HIP runtime error at enqueue";
    case Q4_ERR_PENDING: return "a HIP error from before the call is pending (left in place; nothing launched)";
    case Q4_ERR_SCRATCH: return "the call needs more than the library's built-in scratch (no-allocation entry point)";
    case Q4_ERR_FLAGS: return "unknown bits in a flags argument";
    default: return "unknown status";
  }
}

Q4_API int32_t q4_matmul_path(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return -1;
  if (M <= kGemvMaxRows) return Q4_PATH_GEMV;
  if (M <= kSmallMaxRows) return Q4_PATH_SMALL;
  // at most 128 rows: one row of 128 x 128 tiles
  if (M <= kSmallSlabMaxRows && (N + 127) / 128 < kTiledMinTiles) return Q4_PATH_SMALL;
  return Q4_PATH_MFMA;
}

// With a workspace, 33..128 rows on a grid of few tiles take the tiled kernel
// cut along K instead of the few-row kernel's slabs (each slab streams every
// weight again), for weight matrices of at least 2^24 entries: 1.3-3x faster
// from 5120 x 17408 up, even at 5120 x 5120, slower on small matrices, which
// the slabs finish in 10-15 us.
constexpr int64_t kSlabsToTiledMinWeights = int64_t(1) << 24;

static bool slabs_to_tiled(int64_t M, int64_t N, int64_t K) {
  // N * K >= 2^24 without forming the product (sizes are not checked here)
  return M > kSmallMaxRows && K % 64 == 0 && N > 0 &&
         K >= (kSlabsToTiledMinWeights + N - 1) / N &&
         q4_matmul_path(M, N, K) == Q4_PATH_SMALL && q4::gemm_q4_split_slices(M, N, K) > 1;
}

Q4_API int32_t q4_matmul_path_ex(int64_t M, int64_t N, int64_t K, int32_t with_workspace) {
  const int32_t path = q4_matmul_path(M, N, K);
  if (with_workspace && path == Q4_PATH_SMALL && slabs_to_tiled(M, N, K)) return Q4_PATH_MFMA;
  return path;
}

Q4_API size_t q4_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return 0;
  const int32_t path = q4_matmul_path_ex(M, N, K, 1);
  int64_t slices;   // 0: the call never cuts its rows
  if (path == Q4_PATH_GEMV) {
    slices = q4::gemv_split_slices(M, K);
  } else if (path == Q4_PATH_SMALL) {
    slices = q4::small_split_slices(M, N, K);
    if (slices == 1) slices = 0;
  } else {
    slices = q4::gemm_q4_split_slices(M, N, K);
    if (slices == 1) return q4::gemm_q4_tail_bytes(M, N, K);
  }
  int64_t mn, total;
  if (slices == 0 || !mul_ok(M, N, &mn) || !mul_ok(mn, slices * 4, &total)) return 0;
  return (size_t)total;
}

Q4_API int32_t q4_matmul_ex(const void* x, const void* w_q, const void* w_s, void* y,
                            int32_t y_dtype, int64_t M, int64_t N, int64_t K, void* workspace,
                            size_t workspace_bytes, q4_stream_t stream) {
  if (y_dtype != Q4_F32 && y_dtype != Q4_BF16) return Q4_ERR_DTYPE;
  if (M < 0) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t mk, mn;
  if (!mul_ok(M, K, &mk) || !mul_ok(M, N, &mn)) return Q4_ERR_SHAPE;
  if (M == 0 || N == 0) return Q4_OK;
  if (!x || !w_q || !w_s || !y) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y)) return Q4_ERR_ALIGN;
  float* partial = nullptr;
  if (workspace) {
    const size_t need = q4_matmul_workspace_bytes(M, N, K);
    if (!aligned16(workspace) || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (need > 0) partial = static_cast<float*>(workspace);
  }
  if (int32_t s = ready()) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = y_dtype == Q4_BF16;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint8_t*>(w_q);
  const auto* sp = static_cast<const uint16_t*>(w_s);
  switch (q4_matmul_path_ex(M, N, K, partial != nullptr)) {
    case Q4_PATH_GEMV: return launched(q4::launch_gemv(xp, wp, sp, y, bf16, M, N, K, partial, st));
    case Q4_PATH_SMALL:
      return launched(q4::launch_small(xp, wp, sp, y, bf16, M, N, K, partial, st));
    default: return launched(q4::launch_gemm(xp, wp, sp, y, bf16, M, N, K, partial, st));
  }
}

Q4_API int32_t q4_matmul(const void* x, const void* w_q, const void* w_s, void* y,
                         int32_t y_dtype, int64_t M, int64_t N, int64_t K,
                         q4_stream_t stream) {
  return q4_matmul_ex(x, w_q, w_s, y, y_dtype, M, N, K, nullptr, 0, stream);
}

Q4_API size_t q4_rmsnorm_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return 0;
  int64_t mk;
  if (!mul_ok(M, K, &mk) || mk > (int64_t(1) << 40)) return 0;
  if (M == 0 || N == 0 || q4::gemv_norm_fits(M, K)) return 0;
  return q4::rmsnorm_act_bytes(M, K) + q4_matmul_workspace_bytes(M, N, K);
}

Q4_API int32_t q4_rmsnorm_matmul(const void* x, const void* gamma, float eps, const void* w_q,
                                 const void* w_s, void* y, int32_t y_dtype, int64_t M,
                                 int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                 q4_stream_t stream) {
  if (y_dtype != Q4_F32 && y_dtype != Q4_BF16) return Q4_ERR_DTYPE;
  if (M < 0 || !(eps >= 0.0f) || eps > 3.4e38f) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t mk, mn;
  if (!mul_ok(M, K, &mk) || !mul_ok(M, N, &mn) || mk > (int64_t(1) << 40)) return Q4_ERR_SHAPE;
  if (M == 0 || N == 0) return Q4_OK;
  if (!x || !gamma || !w_q || !w_s || !y) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(w_q) || !aligned16(w_s) || !aligned16(y))
    return Q4_ERR_ALIGN;
  if (!q4::gemv_norm_fits(M, K)) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < q4::rmsnorm_act_bytes(M, K))
      return Q4_ERR_WORKSPACE;
  }
  if (int32_t s = ready()) return s;
  return launched(q4::launch_rmsnorm_matmul(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma), eps,
      static_cast<const uint8_t*>(w_q), static_cast<const uint16_t*>(w_s), y, y_dtype == Q4_BF16,
      M, N, K, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

Q4_API size_t q4_sb_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 256 != 0) return 0;
  int64_t nk;
  if (!mul_ok(N, K, &nk) || nk > (int64_t(1) << 44)) return 0;
  if (M == 0 || N == 0) return 0;
  return q4::sb_scale_bytes(N, K) + q4_matmul_workspace_bytes(M, N, K);
}

Q4_API int32_t q4_sb_matmul(const void* x, const void* w_q, const void* w_d, const void* w_sc,
                            void* y, int32_t y_dtype, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  if (y_dtype != Q4_F32 && y_dtype != Q4_BF16) return Q4_ERR_DTYPE;
  if (M < 0 || K % 256 != 0) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t mk, mn, nk;
  if (!mul_ok(M, K, &mk) || !mul_ok(M, N, &mn) || !mul_ok(N, K, &nk) || nk > (int64_t(1) << 44))
    return Q4_ERR_SHAPE;
  if (M == 0 || N == 0) return Q4_OK;
  if (!x || !w_q || !w_d || !w_sc || !y) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_d) || !aligned16(w_sc) || !aligned16(y))
    return Q4_ERR_ALIGN;
  if (!workspace || !aligned16(workspace) || workspace_bytes < q4::sb_scale_bytes(N, K))
    return Q4_ERR_WORKSPACE;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_sb_matmul(
      static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w_q),
      static_cast<const uint16_t*>(w_d), static_cast<const uint8_t*>(w_sc), y,
      y_dtype == Q4_BF16, M, N, K, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

// Tiled-path K slices of q4_mx_matmul_ex (0: the call never cuts K).
static int64_t mx_split_slices(int64_t M, int64_t N, int64_t K) {
  if (M <= kGemvMaxRows || K % 64 != 0 || q4_matmul_path_ex(M, N, K, 1) != Q4_PATH_MFMA) return 0;
  const int64_t s = q4::gemm_split_slices(M, N, K);
  return s > 1 ? s : 0;
}

Q4_API size_t q4_mx_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0 || K % 32 != 0) return 0;
  const int64_t slices = mx_split_slices(M, N, K);
  int64_t mn, total;
  if (slices == 0 || !mul_ok(M, N, &mn) || !mul_ok(mn, slices * 4, &total)) return 0;
  return (size_t)total;
}

Q4_API int32_t q4_mx_matmul_ex(const void* x, const void* w_q, const void* w_e, void* y,
                               int32_t y_dtype, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  if (y_dtype != Q4_F32 && y_dtype != Q4_BF16) return Q4_ERR_DTYPE;
  // from 3 rows on, slabs of 32 activation rows in the grid's y dimension
  if (M < 0 || M > int64_t(65535) * 32) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t mk, mn;
  if (!mul_ok(M, K, &mk) || !mul_ok(M, N, &mn)) return Q4_ERR_SHAPE;
  if (M == 0 || N == 0) return Q4_OK;
  if (!x || !w_q || !w_e || !y) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_e) || !aligned16(y)) return Q4_ERR_ALIGN;
  float* partial = nullptr;
  if (workspace) {
    const size_t need = q4_mx_matmul_workspace_bytes(M, N, K);
    if (!aligned16(workspace) || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (need > 0) partial = static_cast<float*>(workspace);
  }
  if (int32_t s = ready()) return s;
  const auto* xp = static_cast<const uint16_t*>(x);
  const auto* wp = static_cast<const uint8_t*>(w_q);
  const auto* ep = static_cast<const uint8_t*>(w_e);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = y_dtype == Q4_BF16;
  if (M <= kGemvMaxRows) return launched(q4::launch_mx_gemv(xp, wp, ep, y, bf16, M, N, K, st));
  // the tiled kernel stages 64 k per step; other K stay on the few-row slabs
  if (q4_matmul_path_ex(M, N, K, partial != nullptr) == Q4_PATH_MFMA && K % 64 == 0)
    return launched(q4::launch_gemm_mx(xp, wp, ep, y, bf16, M, N, K, partial, st));
  return launched(q4::launch_small_mx(xp, wp, ep, y, bf16, M, N, K, st));
}

Q4_API int32_t q4_mx_matmul(const void* x, const void* w_q, const void* w_e, void* y,
                            int32_t y_dtype, int64_t M, int64_t N, int64_t K,
                            q4_stream_t stream) {
  return q4_mx_matmul_ex(x, w_q, w_e, y, y_dtype, M, N, K, nullptr, 0, stream);
}

Q4_API int32_t q4_dequantize(const void* w_q, const void* w_s, void* w_out, int32_t out_dtype,
                             int64_t N, int64_t K, q4_stream_t stream) {
  if (out_dtype != Q4_F32 && out_dtype != Q4_BF16) return Q4_ERR_DTYPE;
  if (int32_t s = check_weights(N, K)) return s;
  if (N == 0) return Q4_OK;
  if (!w_q || !w_s || !w_out) return Q4_ERR_NULL;
  if (!aligned16(w_q) || !aligned16(w_s) || !aligned16(w_out)) return Q4_ERR_ALIGN;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_dequant(static_cast<const uint8_t*>(w_q),
                                     static_cast<const uint16_t*>(w_s), w_out,
                                     out_dtype == Q4_BF16, N, K,
                                     static_cast<hipStream_t>(stream)));
}

Q4_API int32_t q4_quantize(const void* w, void* w_q, void* w_s, int64_t N, int64_t K,
                           q4_stream_t stream) {
  if (int32_t s = check_weights(N, K)) return s;
  if (N == 0) return Q4_OK;
  if (!w || !w_q || !w_s) return Q4_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_q) || !aligned16(w_s)) return Q4_ERR_ALIGN;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_quantize(static_cast<const uint16_t*>(w),
                                      static_cast<uint8_t*>(w_q), static_cast<uint16_t*>(w_s),
                                      N, K, static_cast<hipStream_t>(stream)));
}

Q4_API int32_t q4_stream_read_sink_words(void) { return q4::kStreamReadBlocks * 4; }

Q4_API int32_t q4_stream_read(const void* src, size_t bytes, uint32_t* sink,
                              q4_stream_t stream) {
  if (bytes == 0 || bytes % 16 != 0) return Q4_ERR_SHAPE;
  if (!src || !sink) return Q4_ERR_NULL;
  if (!aligned16(src) || !aligned16(sink)) return Q4_ERR_ALIGN;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

Q4_API size_t q4_moe_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t N) {
  int64_t P, PN;
  if (T < 0 || topk < 0 || E < 0 || N < 0) return 0;
  if (!mul_ok(T, topk, &P) || !mul_ok(P, N, &PN) || PN > (int64_t(1) << 40)) return 0;
  if (E > (int64_t(1) << 40)) return 0;
  return q4::moe_workspace_layout(T, topk, E, N).total;
}

Q4_API int32_t q4_moe_matmul(const void* x, const void* w_q, const void* w_s,
                             const int32_t* topk_ids, const float* topk_w, float* y, int64_t T,
                             int64_t topk, int64_t E, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, q4_stream_t stream) {
  if (T < 0 || topk < 0 || E < 0) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t P, tk, en, enk;
  if (!mul_ok(T, topk, &P) || !mul_ok(T, K, &tk) || !mul_ok(E, N, &en) || !mul_ok(en, K, &enk))
    return Q4_ERR_SHAPE;
  // the gathered kernel puts one workgroup row per touched expert (<= 65535)
  if ((P < E ? P : E) > 65535) return Q4_ERR_SHAPE;
  if (T == 0 || N == 0) return Q4_OK;
  if (!y || !x || (topk > 0 && (!topk_ids || !topk_w))) return Q4_ERR_NULL;
  if (E > 0 && topk > 0 && (!w_q || !w_s)) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_w && !aligned16(topk_w)) || (w_q && !aligned16(w_q)) || (w_s && !aligned16(w_s)))
    return Q4_ERR_ALIGN;
  const size_t need = q4_moe_workspace_bytes(T, topk, E, N);
  if (need == 0 || !workspace || !aligned16(workspace) || workspace_bytes < need)
    return Q4_ERR_WORKSPACE;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_moe(static_cast<const uint16_t*>(x),
                                 static_cast<const uint8_t*>(w_q),
                                 static_cast<const uint16_t*>(w_s), topk_ids, topk_w, y, T, topk,
                                 E, N, K, workspace, static_cast<hipStream_t>(stream)));
}

static_assert(Q4_MOE_NOALLOC_MAX_BYTES == q4::kMoeScratchBytes,
              "the header's scratch limit is the array's size");

Q4_API int32_t q4_moe_matmul_noalloc(const void* x, const void* w_q, const void* w_s,
                                     const int32_t* topk_ids, const float* topk_w, float* y,
                                     int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K,
                                     q4_stream_t stream) {
  if (T < 0 || topk < 0 || E < 0) return Q4_ERR_SHAPE;
  if (int32_t s = check_weights(N, K)) return s;
  int64_t P, tk, en, enk;
  if (!mul_ok(T, topk, &P) || !mul_ok(T, K, &tk) || !mul_ok(E, N, &en) || !mul_ok(en, K, &enk))
    return Q4_ERR_SHAPE;
  if ((P < E ? P : E) > 65535) return Q4_ERR_SHAPE;
  if (T == 0 || N == 0) return Q4_OK;
  if (!y || !x || (topk > 0 && (!topk_ids || !topk_w))) return Q4_ERR_NULL;
  if (E > 0 && topk > 0 && (!w_q || !w_s)) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_w && !aligned16(topk_w)) || (w_q && !aligned16(w_q)) || (w_s && !aligned16(w_s)))
    return Q4_ERR_ALIGN;
  const size_t need = q4_moe_workspace_bytes(T, topk, E, N);
  if (need == 0 || need > Q4_MOE_NOALLOC_MAX_BYTES) return Q4_ERR_SCRATCH;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_moe_noalloc(
      static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w_q),
      static_cast<const uint16_t*>(w_s), topk_ids, topk_w, y, T, topk, E, N, K,
      static_cast<hipStream_t>(stream)));
}

Q4_API size_t q4_moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t E, int64_t H,
                                         int64_t F) {
  int64_t P, PH, PF;
  if (T < 0 || topk < 0 || E < 0 || H < 0 || F < 0) return 0;
  if (!mul_ok(T, topk, &P) || !mul_ok(P, H, &PH) || !mul_ok(P, F, &PF)) return 0;
  if (PH > (int64_t(1) << 40) || PF > (int64_t(1) << 40) || E > (int64_t(1) << 40)) return 0;
  return q4::moe_ffn_workspace_layout(T, topk, E, H, F).total;
}

Q4_API int32_t q4_moe_ffn_ex(const void* x, const void* w13_q, const void* w13_s,
                             const void* w2_q, const void* w2_s, const int32_t* topk_ids,
                             const float* topk_w, float* y, int64_t T, int64_t topk, int64_t E,
                             int64_t H, int64_t F, uint32_t flags, void* workspace,
                             size_t workspace_bytes, q4_stream_t stream) {
  if ((flags & ~Q4_MOE_WEIGHTED_DOWN) != 0) return Q4_ERR_FLAGS;
  if (T < 0 || topk < 0 || E < 0) return Q4_ERR_SHAPE;
  if (H <= 0 || F <= 0 || H % 32 != 0 || F % 32 != 0) return Q4_ERR_SHAPE;
  if (H > q4::kMoeFfnMaxWidth || F > q4::kMoeFfnMaxWidth) return Q4_ERR_SHAPE;
  int64_t P, th, e2f, e2fh, eh, ehf;
  if (!mul_ok(T, topk, &P) || !mul_ok(T, H, &th) || !mul_ok(E, 2 * F, &e2f) ||
      !mul_ok(e2f, H, &e2fh) || !mul_ok(E, H, &eh) || !mul_ok(eh, F, &ehf))
    return Q4_ERR_SHAPE;
  if ((P < E ? P : E) > 65535) return Q4_ERR_SHAPE;
  if (T == 0) return Q4_OK;
  if (!y || !x || (topk > 0 && (!topk_ids || !topk_w))) return Q4_ERR_NULL;
  if (E > 0 && topk > 0 && (!w13_q || !w13_s || !w2_q || !w2_s)) return Q4_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (topk_ids && !aligned16(topk_ids)) ||
      (topk_w && !aligned16(topk_w)) || (w13_q && !aligned16(w13_q)) ||
      (w13_s && !aligned16(w13_s)) || (w2_q && !aligned16(w2_q)) || (w2_s && !aligned16(w2_s)))
    return Q4_ERR_ALIGN;
  const size_t need = q4_moe_ffn_workspace_bytes(T, topk, E, H, F);
  if (need == 0 || !workspace || !aligned16(workspace) || workspace_bytes < need)
    return Q4_ERR_WORKSPACE;
  if (int32_t s = ready()) return s;
  return launched(q4::launch_moe_ffn(
      static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w13_q),
      static_cast<const uint16_t*>(w13_s), static_cast<const uint8_t*>(w2_q),
      static_cast<const uint16_t*>(w2_s), topk_ids, topk_w, y, T, topk, E, H, F,
      (flags & Q4_MOE_WEIGHTED_DOWN) != 0, workspace, static_cast<hipStream_t>(stream)));
}

Q4_API int32_t q4_moe_ffn(const void* x, const void* w13_q, const void* w13_s, const void* w2_q,
                          const void* w2_s, const int32_t* topk_ids, const float* topk_w,
                          float* y, int64_t T, int64_t topk, int64_t E, int64_t H, int64_t F,
                          void* workspace, size_t workspace_bytes, q4_stream_t stream) {
  return q4_moe_ffn_ex(x, w13_q, w13_s, w2_q, w2_s, topk_ids, topk_w, y, T, topk, E, H, F, 0,
                       workspace, workspace_bytes, stream);
}

}  // extern "C"
