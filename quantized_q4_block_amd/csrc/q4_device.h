// q4_device.h -- device helpers shared by the gfx950 kernels of libq4.
//
// Weight format (the library's layout of the groupwise-int weights that the
// spec "spec: specialized model runtimes" plans for its T0 quantised GEMM,
// section "Target package and artifact"): codes c in 0..15 stand for c - 8,
// two per byte (even k in the low nibble), one fp16 scale per 32 k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kBlock = 32;          // elements per scale block
constexpr int kWave = 64;           // gfx950 wavefront width

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

// A value the compiler must treat as unknown, kept in a VGPR.  Used for the
// unpack masks: gfx9 VOP3 encodings take no literal and read at most one
// SGPR, so v_and_or_b32(codes, mask, magic) needs the mask in a VGPR (the
// magic then rides in an SGPR); with both as constants the compiler falls
// back to separate AND and OR instructions.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Raw buffer loads: a wave-uniform base becomes a buffer descriptor (scalar
// registers) whose extent bounds the loads -- an offset past it reads zero,
// never another allocation.  Offsets are 32-bit, a per-lane vector part and
// a scalar part, so no 64-bit address is formed per load and lane on the
// vector unit (the streaming kernels are bound by vector instruction issue).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  // word 3 of a gfx9 raw-buffer descriptor (untyped loads)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Workgroup barrier that orders LDS accesses only: it waits for this
// wavefront's LDS (and scalar) operations but, unlike __syncthreads, whose
// fence also waits for every global load in flight, lets earlier global
// loads stay outstanding across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), no vmcnt or expcnt wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum over slices s = 0 .. slices-1, in this order, of p[s * stride].  The
// partial sums come from an earlier kernel's stores (a round trip to the
// far caches or HBM each), so the loads of B slices at a time are issued
// before any of them is added.  Slots past the last slice read the last
// slice again (in bounds) and are not added.
template <int B, typename T>
__device__ __forceinline__ T sum_slices(const T* __restrict__ p, int64_t stride, int slices) {
  T acc = {};
  for (int s0 = 0; s0 < slices; s0 += B) {
    T v[B];
#pragma unroll
    for (int j = 0; j < B; ++j)
      v[j] = p[(int64_t)(s0 + j < slices ? s0 + j : slices - 1) * stride];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (s0 + j < slices) acc = s0 + j == 0 ? v[j] : acc + v[j];
  }
  return acc;
}

// Unpacks codes into exact fp16 (c - 8) pairs.
//
// A dword's bytes b0..b3 hold elements e0..e7 (b_i low nibble = e_{2i},
// high nibble = e_{2i+1}).  Masking one nibble per 16-bit half and OR-ing an
// fp16 exponent makes each half an fp16 whose value is a constant plus the
// code: with exponent 2^10 the low nibble (bits 0..3) is worth 1..8, with
// exponent 2^6 the next nibble (bits 4..7) is worth 1..8 too.  One packed
// fp16 subtract of (constant + 8) then leaves exactly c - 8 in each half.
// Result pairs: p[0] = (e0, e4), p[1] = (e1, e5), p[2] = (e2, e6),
// p[3] = (e3, e7) as (low half, high half).  Cost per dword: one shift, four
// v_and_or_b32, four v_pk_add_f16.
struct CodeUnpacker {
  uint32_t m_lo, m_hi;
  __device__ __forceinline__ CodeUnpacker()
      : m_lo(opaque_vgpr(0x000F000Fu)), m_hi(opaque_vgpr(0x00F000F0u)) {}
  __device__ __forceinline__ void operator()(uint32_t d, half2v p[4]) const {
    const half2v b_lo = {(_Float16)1032.0f, (_Float16)1032.0f};  // 1024 + 8
    const half2v b_hi = {(_Float16)72.0f, (_Float16)72.0f};      // 64 + 8
    const uint32_t d8 = d >> 8;
    p[0] = __builtin_bit_cast(half2v, (d & m_lo) | 0x64006400u) - b_lo;
    p[1] = __builtin_bit_cast(half2v, (d & m_hi) | 0x54005400u) - b_hi;
    p[2] = __builtin_bit_cast(half2v, (d8 & m_lo) | 0x64006400u) - b_lo;
    p[3] = __builtin_bit_cast(half2v, (d8 & m_hi) | 0x54005400u) - b_hi;
  }
};

// Unpacks codes into exact bf16 (c - 8) values for the matrix cores, in k
// order: o[i] holds elements 2i (low half) and 2i + 1 (high half).
//
// The same magic-exponent fp16 halves as CodeUnpacker (1024 + c for the low
// nibble of each 16-bit half, 64 + c for the next one) are widened by
// v_fma_mix_f32, which subtracts the constant in the same instruction:
// h * 1 - 1032 (or - 72) is c - 8 exactly in fp32.  The multiplier is kept in a
// register so the compiler cannot fold the multiply away and split the
// instruction into a conversion and an add.  v_cvt_pk_bf16_f32 then packs two
// small integers (exact in bf16).  Cost per dword: one shift, four
// v_and_or_b32, eight v_fma_mix_f32 and four v_cvt_pk_bf16_f32.
struct ExactBf16Unpacker {
  uint32_t m_lo, m_hi;
  float one;
  __device__ __forceinline__ ExactBf16Unpacker()
      : m_lo(opaque_vgpr(0x000F000Fu)), m_hi(opaque_vgpr(0x00F000F0u)),
        one(__uint_as_float(opaque_vgpr(0x3F800000u))) {}
  __device__ __forceinline__ void operator()(uint32_t d, uint32_t o[4]) const {
    const uint32_t d8 = d >> 8;
    const half2v h0 = __builtin_bit_cast(half2v, (d & m_lo) | 0x64006400u);   // e0, e4
    const half2v h1 = __builtin_bit_cast(half2v, (d & m_hi) | 0x54005400u);   // e1, e5
    const half2v h2 = __builtin_bit_cast(half2v, (d8 & m_lo) | 0x64006400u);  // e2, e6
    const half2v h3 = __builtin_bit_cast(half2v, (d8 & m_hi) | 0x54005400u);  // e3, e7
    const float lo = -1032.0f, hi = -72.0f;
    o[0] = pack2(__builtin_fmaf((float)h0[0], one, lo), __builtin_fmaf((float)h1[0], one, hi));
    o[1] = pack2(__builtin_fmaf((float)h2[0], one, lo), __builtin_fmaf((float)h3[0], one, hi));
    o[2] = pack2(__builtin_fmaf((float)h0[1], one, lo), __builtin_fmaf((float)h1[1], one, hi));
    o[3] = pack2(__builtin_fmaf((float)h2[1], one, lo), __builtin_fmaf((float)h3[1], one, hi));
  }

 private:
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    bf16x2v v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Two fp32 -> packed fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  half2v v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// 4-bit float blocks (e2m1 elements, one E8M0 scale byte per 32 k).
typedef float f32x2v __attribute__((ext_vector_type(2)));

// E8M0 scale byte -> fp32 2^(E-127) (E = 0 is the fp32 subnormal 2^-127,
// E = 255 is NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23);
  return __uint_as_float(bits);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.  The
// butterfly order is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace q4
