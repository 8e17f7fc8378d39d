// q4_quant.hip -- bf16 weights -> this library's 4-bit block format.
//
// The convert step of the specialised-runtime spec's build flow ("spec:
// specialized model runtimes", section "Target package and artifact": model
// weights are converted into the runtime's weight profile, then qualified).
// The pages fix no method; per 32-element block of a row:
//   m   = the element of largest |w| (the first one in k on ties)
//   s   = fp16(m / -8), nearest-even, |m / 8| clamped to 65504 first
//   c_k = clamp(rint(w_k / s) + 8, 0, 15)   (s == 0: every c_k = 8)
// so the largest-magnitude element lands exactly on code 0.  The quotient is
// an IEEE fp32 division and rint rounds half to even, as written.
//
// One thread per block: four 16-byte loads of bf16, one 16-byte store of
// codes and one 2-byte store of the scale; consecutive threads take
// consecutive blocks of a row, so every access is coalesced.  Memory-bound:
// 64 bytes in, 18 bytes out per block.
#include "q4_device.h"
#include "q4_launch.h"

namespace q4 {

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w,
                                                       uint8_t* __restrict__ wq,
                                                       uint16_t* __restrict__ ws,
                                                       int64_t n_blocks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < n_blocks;
       blk += stride) {
    const uint4* src = reinterpret_cast<const uint4*>(w + blk * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = src[i];
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * i + 2 * h] = bf16_lo(d[h]);
        v[8 * i + 2 * h + 1] = bf16_hi(d[h]);
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (__builtin_fabsf(v[k]) > __builtin_fabsf(m)) m = v[k];
    // m / -8 is exact in fp32 (a power-of-two step of a bf16 value)
    const float d = __builtin_fminf(__builtin_fmaxf(m / -8.0f, -65504.0f), 65504.0f);
    const _Float16 sh = (_Float16)d;   // nearest-even
    const float s = (float)sh;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      uint32_t c = 8u;
      if (s != 0.0f) {
        const float q = __builtin_rintf(v[k] / s);
        c = (uint32_t)__builtin_fminf(15.0f, __builtin_fmaxf(0.0f, q + 8.0f));
      }
      packed[k / 8] |= c << (4 * (k % 8));   // k = 2j low nibble of byte j
    }
    *reinterpret_cast<uint4*>(wq + blk * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    ws[blk] = __builtin_bit_cast(uint16_t, sh);
  }
}

hipError_t launch_quantize(const uint16_t* w, uint8_t* wq, uint16_t* ws, int64_t N, int64_t K,
                           hipStream_t stream) {
  const int64_t n_blocks = N * (K / 32);
  int64_t grid = (n_blocks + 255) / 256;
  if (grid > 65536) grid = 65536;   // grid-stride loop past that
  quantize_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(w, wq, ws, n_blocks);
  return hipGetLastError();
}

}  // namespace q4
