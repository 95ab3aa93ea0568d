// QKV preparation kernels (HBM-bound).
//
// TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", section
// "面向注意力的 FP8 Preparation": one E4M3 scale per (batch, head, 64-token Q/K block),
// s = max|X_block| / 448; one scale per (batch, head, channel) for V over all tokens; V is
// written token-contiguous so the PV contraction reads keys contiguously. VC-Attention article
// section 二: V-Smooth subtracts the mean of each 128-row block of the (cluster-permuted) V and
// quantises the residual; the mean is kept as one 16-bit vector per block.
//
// Launch plan on the caller's stream (all row loads are 256-byte rows of the source layout
// [B, N_src, H, 128], so every gather stays coalesced):
//   1. quant_qk      grid (NB, B*H, 2): amax of a 64-row Q or K block -> scale -> codes.
//   2. v_block_stats grid (NB128, B*H): per 128-row block, per channel: amax of V, or (V-Smooth)
//                    the block mean (exact FP64 column sums) and the residual amax.
//   3. v_finalize    grid (B*H): channel amax over blocks -> v_scale and its inverse.
//   4. v_encode      grid (NB, B*H): codes of a 64-row block, transposed through LDS into
//                    [B, H, 128, N64].
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

// Source row index of layout position i for head bh, or -1 (padding, beyond N, or an
// out-of-range permutation entry, which is treated as padding).
__device__ __forceinline__ int64_t gather_src(const int32_t* perm, int per_head, int64_t bh,
                                              int64_t N, int64_t Nsrc, int64_t i) {
  if (i >= N) return -1;
  if (perm == nullptr) return i;
  const int64_t s = per_head ? perm[bh * N + i] : perm[i];
  return (s >= 0 && s < Nsrc) ? s : -1;
}

// Byte offset-free pointer to the 128-channel bf16 row (b, src, h) of the source layout.
__device__ __forceinline__ const uint16_t* src_row(const uint16_t* base, int64_t b, int64_t src,
                                                   int64_t h, int64_t Nsrc, int64_t H) {
  return base + ((b * Nsrc + src) * H + h) * kHeadDim;
}

struct Bf16x8 {
  float v[8];
};

__device__ __forceinline__ Bf16x8 load8(const uint16_t* p) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  Bf16x8 r;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    r.v[2 * j] = __uint_as_float(w[j] << 16);
    r.v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
  return r;
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// 1. Q / K block quantisation. Thread t handles channels 8*(t%16) .. +7 of rows t/16 + 16*p.
__global__ __launch_bounds__(256) void quant_qk(QuantParams p) {
  __shared__ float red[4];
  const int64_t blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int which = blockIdx.z;  // 0: Q, 1: K
  const int64_t b = bh / p.H, h = bh % p.H;
  const uint16_t* src = which == 0 ? p.q : p.k;
  const int32_t* perm = which == 0 ? p.perm_q : p.perm_kv;
  const int per_head = which == 0 ? 0 : p.perm_kv_per_head;
  uint8_t* codes = which == 0 ? p.q8 : p.k8;
  float* scales = which == 0 ? p.q_scale : p.k_scale;

  const int chunk = threadIdx.x & 15;
  const int row0 = threadIdx.x >> 4;
  Bf16x8 x[4];
  float amax = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int64_t i = blk * kBlock + row0 + 16 * pass;
    const int64_t s = gather_src(perm, per_head, bh, p.N, p.Nsrc, i);
    if (s >= 0) {
      x[pass] = load8(src_row(src, b, s, h, p.Nsrc, p.H) + chunk * 8);
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) x[pass].v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(x[pass].v[j]));
  }
  amax = block_max_256(amax, red);
  const float inv = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
  if (threadIdx.x == 0) scales[bh * p.NB + blk] = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int64_t i = blk * kBlock + row0 + 16 * pass;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = x[pass].v[j] * inv;
    uint2 out;
    out.x = e4m3x4(y[0], y[1], y[2], y[3]);
    out.y = e4m3x4(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2*>(codes + (bh * p.N64 + i) * kHeadDim + chunk * 8) = out;
  }
}

// 2. Per 128-row block statistics of V. Thread t: channels 8*(t%16)..+7, rows t/16 + 16*p.
__global__ __launch_bounds__(256) void v_block_stats(QuantParams p) {
  __shared__ double dsum[16][kHeadDim];  // [row group][channel]
  __shared__ float fmax_[16][kHeadDim];
  __shared__ float mhat_s[kHeadDim];
  __shared__ int n_valid_s;
  const int64_t j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int chunk = threadIdx.x & 15;
  const int rg = threadIdx.x >> 4;
  if (threadIdx.x == 0) n_valid_s = 0;
  __syncthreads();

  Bf16x8 x[8];
  bool valid[8];
  int my_valid = 0;  // rows counted once, by the chunk-0 thread of each row
#pragma unroll
  for (int pass = 0; pass < 8; pass++) {
    const int64_t i = j * kVBlock + rg + 16 * pass;
    const int64_t s = gather_src(p.perm_kv, p.perm_kv_per_head, bh, p.N, p.Nsrc, i);
    valid[pass] = s >= 0;
    my_valid += (chunk == 0 && valid[pass]) ? 1 : 0;
    if (valid[pass]) {
      x[pass] = load8(src_row(p.v, b, s, h, p.Nsrc, p.H) + chunk * 8);
    } else {
#pragma unroll
      for (int q = 0; q < 8; q++) x[pass].v[q] = 0.0f;
    }
  }

  float m[8];
#pragma unroll
  for (int q = 0; q < 8; q++) m[q] = 0.0f;
  if (p.vsmooth) {
    // Column sums in FP64: exact for <= 128 bf16 terms, so the summation order is irrelevant.
    double s[8];
#pragma unroll
    for (int q = 0; q < 8; q++) s[q] = 0.0;
#pragma unroll
    for (int pass = 0; pass < 8; pass++)
#pragma unroll
      for (int q = 0; q < 8; q++) s[q] += static_cast<double>(x[pass].v[q]);
#pragma unroll
    for (int q = 0; q < 8; q++) dsum[rg][chunk * 8 + q] = s[q];
    if (my_valid) atomicAdd(&n_valid_s, my_valid);
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
      double tot = 0.0;
      for (int g = 0; g < 16; g++) tot += dsum[g][threadIdx.x];
      const int n_valid = n_valid_s;
      const float mean = n_valid > 0 ? static_cast<float>(tot / static_cast<double>(n_valid)) : 0.0f;
      const uint16_t mb = f32_to_bf16_rne(mean);
      p.v_mean[(bh * p.NB128 + j) * kHeadDim + threadIdx.x] = mb;
      mhat_s[threadIdx.x] = bf16_to_f32(mb);
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 8; pass++)
      if (valid[pass])
#pragma unroll
        for (int q = 0; q < 8; q++) m[q] = fmaxf(m[q], fabsf(x[pass].v[q] - mhat_s[chunk * 8 + q]));
  } else {
#pragma unroll
    for (int pass = 0; pass < 8; pass++)
#pragma unroll
      for (int q = 0; q < 8; q++) m[q] = fmaxf(m[q], fabsf(x[pass].v[q]));
  }
#pragma unroll
  for (int q = 0; q < 8; q++) fmax_[rg][chunk * 8 + q] = m[q];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    float mm = 0.0f;
    for (int g = 0; g < 16; g++) mm = fmaxf(mm, fmax_[g][threadIdx.x]);
    p.ws_partial[(bh * p.NB128 + j) * kHeadDim + threadIdx.x] = mm;
  }
}

// 3. Channel amax over the 128-row blocks -> v_scale and the inverse scale used to encode.
__global__ __launch_bounds__(128) void v_finalize(QuantParams p) {
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  float m = 0.0f;
  for (int64_t j = 0; j < p.NB128; j++) m = fmaxf(m, p.ws_partial[(bh * p.NB128 + j) * kHeadDim + d]);
  p.v_scale[bh * kHeadDim + d] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 0.0f;
  p.ws_inv[bh * kHeadDim + d] = m > 0.0f ? __fdiv_rn(448.0f, m) : 0.0f;
}

// 4. V codes of a 64-row block, transposed to token-contiguous rows of v8t.
__global__ __launch_bounds__(256) void v_encode(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kHeadDim][kBlock + 16];  // [channel][token]
  const int64_t blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int chunk = threadIdx.x & 15;
  const int row0 = threadIdx.x >> 4;
  float inv[8], mhat[8];
#pragma unroll
  for (int q = 0; q < 8; q++) {
    inv[q] = p.ws_inv[bh * kHeadDim + chunk * 8 + q];
    mhat[q] = 0.0f;
  }
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int t = row0 + 16 * pass;
    const int64_t i = blk * kBlock + t;
    const int64_t s = gather_src(p.perm_kv, p.perm_kv_per_head, bh, p.N, p.Nsrc, i);
    uint32_t lo = 0, hi = 0;
    if (s >= 0) {
      const Bf16x8 x = load8(src_row(p.v, b, s, h, p.Nsrc, p.H) + chunk * 8);
      if (p.vsmooth) {
        const uint16_t* mrow = p.v_mean + (bh * p.NB128 + i / kVBlock) * kHeadDim + chunk * 8;
#pragma unroll
        for (int q = 0; q < 8; q++) mhat[q] = bf16_to_f32(mrow[q]);
      }
      float y[8];
#pragma unroll
      for (int q = 0; q < 8; q++) y[q] = (x.v[q] - mhat[q]) * inv[q];
      lo = e4m3x4(y[0], y[1], y[2], y[3]);
      hi = e4m3x4(y[4], y[5], y[6], y[7]);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
      tile[chunk * 8 + q][t] = static_cast<uint8_t>(lo >> (8 * q));
      tile[chunk * 8 + 4 + q][t] = static_cast<uint8_t>(hi >> (8 * q));
    }
  }
  __syncthreads();
  // Thread t writes channel t/2, tokens 32*(t%2) .. +31 (two 16-byte stores).
  const int d = threadIdx.x >> 1;
  const int half = threadIdx.x & 1;
  const uint4* srcp = reinterpret_cast<const uint4*>(&tile[d][32 * half]);
  uint4* dst = reinterpret_cast<uint4*>(p.v8t + (bh * kHeadDim + d) * p.N64 + blk * kBlock + 32 * half);
  dst[0] = srcp[0];
  dst[1] = srcp[1];
}

}  // namespace

hipError_t launch_quantize(const QuantParams& p, hipStream_t stream) {
  const dim3 g_qk(static_cast<unsigned>(p.NB), static_cast<unsigned>(p.B * p.H), 2);
  hipLaunchKernelGGL(quant_qk, g_qk, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v_block_stats, dim3(static_cast<unsigned>(p.NB128), static_cast<unsigned>(p.B * p.H)),
                     dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v_finalize, dim3(static_cast<unsigned>(p.B * p.H)), dim3(kHeadDim), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v_encode, dim3(static_cast<unsigned>(p.NB), static_cast<unsigned>(p.B * p.H)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8attn
