// Shared device helpers of libfp8attn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8attn {

constexpr int kHeadDim = 128;  // D; the only head size the library supports
constexpr int kBlock = 64;     // Q/K scale block and softmax max-update granularity
constexpr int kVBlock = 128;   // V-Smooth mean block

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// IEEE round-to-nearest-even of a finite FP32 value to BF16 (NaN is not produced here).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two FP32 values -> two OCP E4M3 bytes (RNE) in the low 16 bits of the result.
// The hardware conversion agrees with RNE onto the E4M3 grid for |x| < 464; every caller
// feeds values of magnitude <= 448 * (1 + 2^-23).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Four FP32 values -> four E4M3 bytes packed little-endian.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// Exact value of an OCP E4M3 byte (finite codes; the encoders saturate, so 0x7F/0xFF never occur).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? static_cast<float>(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace fp8attn
