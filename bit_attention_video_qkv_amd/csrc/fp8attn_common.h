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

typedef float f32x2 __attribute__((ext_vector_type(2)));

// The two E4M3 bytes of one half of a packed word (high: bytes 2 and 3) as FP32, on the
// conversion unit (OCP E4M3, the format of the encoders above; the encoders saturate, so the
// NaN codes 0x7F/0xFF never occur).
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w, bool high) {
  return high ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true)
              : __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}

// One E4M3 byte (bits 0..7 of c) as FP32, on the conversion unit.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(c), 0);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Waits until at most N vector-memory operations of this wave are outstanding (they complete
// in issue order, so every older global->LDS copy has landed).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier without the release/acquire fence of __syncthreads(): that fence makes the
// compiler wait for every outstanding global->LDS copy, including those meant to stay in flight
// across the barrier. Callers order their own LDS traffic with explicit waits; the "memory"
// clobber keeps the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Direct global->LDS copies (each lane: 16 or 4 bytes from gbase + voff to LDS lds_addr + 16 *
// lane or + 4 * lane). Issued as opaque instructions: the compiler would otherwise treat every
// later LDS read as possibly overlapping a copy still in flight and drain all of them first,
// which would cost the copies' prefetch distance. The kernel orders them itself (explicit
// vmcnt waits and barriers).
__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)p));
}
// A wave-uniform pointer as an SGPR pair (the copies take their base from scalar registers).
__device__ __forceinline__ const void* uniform_ptr(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}
// Read of a read-only int array at a wave-uniform index as a scalar load (through the constant
// address space). A plain load would become a vector load whose use waits on vmcnt, the
// counter that also tracks the K/V copies in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* base, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)base)[i];
}
__device__ __forceinline__ void copy16_to_lds(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(gbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
}  // namespace fp8attn
