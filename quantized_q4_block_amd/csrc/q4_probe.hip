// q4_probe.hip -- the benchmark's streaming ceiling: a read-only pass over
// a byte range with the decode kernel's access width and cache hint (16
// bytes per lane and load, non-temporal), each wavefront streaming a
// contiguous stretch with six 1 KB loads in flight (the fastest of the
// read-only patterns measured on this chip), so that the decode kernel's
// HBM rate can be set beside what a plain read stream reaches on the same
// bytes.  Not on any product path.
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeDepth = 6;   // 1 KB wavefront loads in flight
typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

// Wavefront w of the grid reads units [w * per_wave, (w + 1) * per_wave) of
// 16 bytes (past the range: nothing), kProbeDepth loads of 64 consecutive
// units in flight, and writes the XOR of what it read to sink[w]: every
// load is used, and the XOR of the whole sink is the XOR of every 32-bit
// word of the range.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const probe_u32x4* __restrict__ src, int64_t units, int64_t per_wave,
    uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const int64_t beg = w * per_wave;
  const int64_t end = beg + per_wave < units ? beg + per_wave : units;
  uint32_t acc = 0;
  for (int64_t o = beg; o < end; o += kProbeDepth * 64) {
    probe_u32x4 v[kProbeDepth];
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) {
      const int64_t u = o + d * 64 + lane;
      v[d] = u < end ? __builtin_nontemporal_load(src + u) : probe_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) acc ^= v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if (lane == 0) sink[w] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t units = (int64_t)(bytes / 16);
  const int64_t waves = (int64_t)kStreamReadBlocks * (kProbeThreads / 64);
  // each wavefront's stretch a whole number of 1 KB loads
  const int64_t per_wave = ((units + waves - 1) / waves + 63) / 64 * 64;
  stream_read_kernel<<<dim3(kStreamReadBlocks), dim3(kProbeThreads), 0, stream>>>(
      static_cast<const probe_u32x4*>(src), units, per_wave, sink);
  return hipGetLastError();
}

}  // namespace q4
