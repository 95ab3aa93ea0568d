// Diagnostics of the two pieces of device arithmetic the parity contract rests on, each run
// exactly as the production kernels run it:
//  * the E4M3 encoder of the quantisation kernels (e4m3x4: v_cvt_pk_fp8_f32, round to nearest
//    even onto the OCP E4M3 grid), applied to consecutive FP32 bit patterns, so that a test can
//    compare it with an independent encoder over every input the quantiser can produce
//    (TeleFuser blog "FP8 Sol-Attn", section "面向注意力的 FP8 Preparation": codes of x / s with
//    s = amax / 448, so |x / s| <= 448 up to one FP32 rounding);
//  * the E4M3 decoders of the Sol preparation and the V bias correction (e4m3x2_to_f32 and
//    e4m3_to_f32 on the conversion unit), applied to given codes, so that a test can compare them
//    with the exact values of every finite code;
//  * one E4M3 x E4M3 -> FP32 matrix-core product (v_mfma_scale_f32_32x32x64_f8f6f4, the QK and
//    PV contraction of the attention kernel) per 32 x 32 x 64 tile, so that a test can bound how
//    far the hardware's sum of exact E4M3 products lies from the exact sum.
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// out[i] = the four E4M3 bytes of the FP32 values with bit patterns first + 4i .. first + 4i + 3
// (i < n_words).
__global__ __launch_bounds__(256) void diag_e4m3_encode(uint32_t first, int64_t n_words, uint32_t* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_words) return;
  const uint32_t b = first + 4u * static_cast<uint32_t>(i);
  out[i] = e4m3x4(__uint_as_float(b), __uint_as_float(b + 1u), __uint_as_float(b + 2u), __uint_as_float(b + 3u));
}

// out[4i + k] = code 4i + k decoded two codes per conversion (e4m3x2_to_f32, as the bias
// correction and the V summaries decode); out[n + 4i + k] = the same code decoded alone
// (e4m3_to_f32, as the K summaries and the thresholds decode), i < n_words.
__global__ __launch_bounds__(256) void diag_e4m3_decode(const uint32_t* codes, int64_t n_words, float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_words) return;
  const uint32_t w = codes[i];
  const f32x2 lo = e4m3x2_to_f32(w, false), hi = e4m3x2_to_f32(w, true);
  *reinterpret_cast<float4*>(out + 4 * i) = make_float4(lo.x, lo.y, hi.x, hi.y);
  *reinterpret_cast<float4*>(out + 4 * n_words + 4 * i) =
      make_float4(e4m3_to_f32(w & 0xFFu), e4m3_to_f32((w >> 8) & 0xFFu), e4m3_to_f32((w >> 16) & 0xFFu),
                  e4m3_to_f32(w >> 24));
}

// One wave per tile t: C[t] (32 x 32 FP32, row-major) = A[t] (32 x 64 E4M3, row-major) times the
// transpose of Bt[t] (32 x 64 E4M3, row-major: row j holds column j of B), with the operand
// layout of the attention kernel: lane l holds row l % 32 of A (of Bt) and the 32 bytes
// [32 (l / 32), +32) of that row; accumulator register r of lane l holds
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__global__ __launch_bounds__(64) void diag_mfma_e4m3(const uint8_t* a, const uint8_t* bt, float* c) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x, row = lane & 31, half = lane >> 5;
  const uint4* pa = reinterpret_cast<const uint4*>(a + t * 2048 + row * 64 + half * 32);
  const uint4* pb = reinterpret_cast<const uint4*>(bt + t * 2048 + row * 64 + half * 32);
  const uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  v8i av, bv;
  av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w; av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
  bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w; bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = 0.0f;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  float* ct = c + t * 1024;
#pragma unroll
  for (int r = 0; r < 16; r++) ct[(8 * (r >> 2) + 4 * half + (r & 3)) * 32 + row] = acc[r];
}

}  // namespace

hipError_t launch_diag_e4m3_encode(uint32_t first, int64_t n_words, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(diag_e4m3_encode, dim3(static_cast<unsigned>((n_words + 255) / 256)), dim3(256), 0, stream,
                     first, n_words, out);
  return hipGetLastError();
}

hipError_t launch_diag_e4m3_decode(const uint32_t* codes, int64_t n_words, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(diag_e4m3_decode, dim3(static_cast<unsigned>((n_words + 255) / 256)), dim3(256), 0, stream,
                     codes, n_words, out);
  return hipGetLastError();
}

hipError_t launch_diag_mfma_e4m3(const uint8_t* a, const uint8_t* bt, float* c, int32_t n_tiles,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(diag_mfma_e4m3, dim3(static_cast<unsigned>(n_tiles)), dim3(64), 0, stream, a, bt, c);
  return hipGetLastError();
}

}  // namespace fp8attn
