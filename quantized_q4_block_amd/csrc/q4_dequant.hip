// q4_dequant.hip -- W -> fp32 or bf16 [N][K].
//
// Dequantisation is the "quant/dequant" op of the T0 kernel tier in the spec
// "spec: specialized model runtimes" (section "Architecture").  Each thread
// owns one 32-element block: one 128-bit load of codes, one fp16 scale, and
// 32 outputs.  (c - 8) is formed exactly in fp16 and multiplied by the scale
// in fp32, where the product (at most 15 significant bits) is exact.  The
// bf16 variant rounds that exact value to nearest even.  Memory-bound:
// 18 bytes in, 128 (fp32) or 64 (bf16) bytes out per block.
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

template <bool kBf16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ ws,
                                                      void* __restrict__ out,
                                                      int64_t n_blocks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const CodeUnpacker unpack;
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < n_blocks;
       blk += stride) {
    const uint4 codes = *reinterpret_cast<const uint4*>(wq + blk * 16);
    const float s = fp16_to_f32(ws[blk]);
    const uint32_t dw[4] = {codes.x, codes.y, codes.z, codes.w};
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v p[4];
      unpack(dw[i], p);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + j] = (float)p[j][0] * s;      // elements 8i + j
        v[8 * i + j + 4] = (float)p[j][1] * s;  // elements 8i + j + 4
      }
    }
    if constexpr (kBf16) {
      uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + blk * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 w;
        w.x = pack_bf16x2(v[8 * q + 0], v[8 * q + 1]);
        w.y = pack_bf16x2(v[8 * q + 2], v[8 * q + 3]);
        w.z = pack_bf16x2(v[8 * q + 4], v[8 * q + 5]);
        w.w = pack_bf16x2(v[8 * q + 6], v[8 * q + 7]);
        o[q] = w;
      }
    } else {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + blk * 32);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        o[q] = make_float4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  }
}

hipError_t launch_dequant(const uint8_t* wq, const uint16_t* ws, void* out, bool bf16,
                          int64_t N, int64_t K, hipStream_t stream) {
  const int64_t n_blocks = N * (K / kBlock);
  const int threads = 256;
  int64_t grid = (n_blocks + threads - 1) / threads;
  if (grid > 65536) grid = 65536;
  if (bf16)
    dequant_kernel<true><<<dim3((unsigned)grid), dim3(threads), 0, stream>>>(wq, ws, out, n_blocks);
  else
    dequant_kernel<false><<<dim3((unsigned)grid), dim3(threads), 0, stream>>>(wq, ws, out, n_blocks);
  return hipGetLastError();
}

}  // namespace q4
