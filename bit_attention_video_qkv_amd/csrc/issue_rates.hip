// issue_rates: measures, on one MI355X, how many shader cycles a SIMD spends per wave64
// instruction of the kinds the attention mainloop issues, alone and mixed with FP8 MFMAs, and
// the cost of one 64-key block of the mainloop's instruction mix with every dependency and
// memory access removed (the issue floor the kernel can approach). Cycles come from s_memtime
// around a loop of independent instructions in every wave of one workgroup per CU; the time of
// the slowest wave of a SIMD divided by the work of all its waves gives cycles per instruction.
// Every store goes to out[2 * (blockIdx.x * waves + wave) + {0, 1}], sized for the launch.
//
// Build: hipcc --offload-arch=gfx950 -O3 issue_rates.hip -o issue_rates (build.py does this).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define FMA(r) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(r) : "v"(c1), "v"(c2));
#define ADD(r, s) asm volatile("v_add_f32 %0, %0, %1" : "+v"(r) : "v"(s));
#define MUL(r) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(r) : "v"(c1));
#define EXP(r) asm volatile("v_exp_f32 %0, %0" : "+v"(r));
#define MAX3(r, a, b) asm volatile("v_maximum3_f32 %0, %0, %1, %2" : "+v"(r) : "v"(a), "v"(b));
#define MAX3L(r, a, b) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(r) : "v"(a), "v"(b));
#define CVT(d, a, b) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "+v"(d) : "v"(a), "v"(b));
#define CVTU8(d, a) asm volatile("v_cvt_pk_u8_f32 %0, %1, 1, %0" : "+v"(d) : "v"(a));
#define SB __builtin_amdgcn_sched_barrier(0);
#define MF(acc) { acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0); SB }
#define MF16(acc) { acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0); SB }

enum Kind {
  kFma, kAdd, kMul, kMax3, kExp, kCvtFp8, kCvtU8, kExpFma, kCvtFma, kMfma, kMfmaFma,
  kBlock, kBlockValuOnly, kBlockPlainSlowOps, kBlockExpCast, kBlockExpCastValuOnly, kBlockExpCastEven,
  kMax3Legacy, kNumKinds
};
static const char* kNames[] = {
    "v_fma_f32",           "v_add_f32",           "v_mul_f32",        "v_maximum3_f32",
    "v_exp_f32",           "v_cvt_pk_fp8_f32",    "v_cvt_pk_u8_f32",  "exp + fma alternating",
    "cvt_pk_fp8 + fma alternating", "mfma 32x32x64 f8",   "mfma + 16 fma each",
    "attention block mix", "block mix, VALU part only", "block mix, exp/cvt replaced by fma",
    "ExpCast block mix", "ExpCast mix, VALU part only", "ExpCast mix, MFMAs spread evenly",
    "v_max3_f32"};
// per wave and iteration: VALU instructions, MFMAs
static const int kValu[] = {32, 32, 32, 16, 32, 16, 16, 32, 16, 0, 64, 136, 136, 136, 88, 88, 88, 16};
static const int kMfmas[] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 4, 4, 8, 0, 8, 9, 0, 9, 0};

template <int KIND, int WPS>
__global__ __launch_bounds__(256 * WPS) void probe(unsigned long long* out, int iters, float c1, float c2) {
  __shared__ int pad[24576];  // 96 KB: one workgroup per CU
  const int wave = threadIdx.x >> 6;
  float x[32], l[4];
#pragma unroll
  for (int i = 0; i < 32; i++) x[i] = 1e-3f * static_cast<float>(threadIdx.x + i);
#pragma unroll
  for (int i = 0; i < 4; i++) l[i] = 0.0f;
  float m0 = 0.0f, m1 = 0.0f;
  int p[16];
#pragma unroll
  for (int i = 0; i < 16; i++) p[i] = i;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; i++) { a[i] = 0x38383838 + i; b[i] = 0x30303030 + i; }
  v16f acc[4];
#pragma unroll
  for (int k = 0; k < 4; k++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[k][i] = 0.0f;
  v4f racc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (threadIdx.x == 1u << 20) pad[0] = 1;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; it++) {
    SB
    if constexpr (KIND == kFma) {
#pragma unroll
      for (int i = 0; i < 32; i++) FMA(x[i])
    } else if constexpr (KIND == kAdd) {
#pragma unroll
      for (int i = 0; i < 32; i++) ADD(x[i], x[(i + 7) & 31])
    } else if constexpr (KIND == kMul) {
#pragma unroll
      for (int i = 0; i < 32; i++) MUL(x[i])
    } else if constexpr (KIND == kMax3) {
#pragma unroll
      for (int i = 0; i < 16; i++) MAX3(x[i], x[16 + i], x[(i + 7) & 31])
    } else if constexpr (KIND == kMax3Legacy) {
#pragma unroll
      for (int i = 0; i < 16; i++) MAX3L(x[i], x[16 + i], x[(i + 7) & 31])
    } else if constexpr (KIND == kExp) {
#pragma unroll
      for (int i = 0; i < 32; i++) EXP(x[i])
    } else if constexpr (KIND == kCvtFp8) {
#pragma unroll
      for (int i = 0; i < 16; i++) CVT(p[i], x[2 * i], x[2 * i + 1])
    } else if constexpr (KIND == kCvtU8) {
#pragma unroll
      for (int i = 0; i < 16; i++) CVTU8(p[i], x[i])
    } else if constexpr (KIND == kExpFma) {
#pragma unroll
      for (int i = 0; i < 16; i++) { EXP(x[i]) FMA(x[16 + i]) }
    } else if constexpr (KIND == kCvtFma) {
#pragma unroll
      for (int i = 0; i < 8; i++) { CVT(p[i], x[2 * i], x[2 * i + 1]) FMA(x[16 + i]) }
    } else if constexpr (KIND == kMfma) {
#pragma unroll
      for (int k = 0; k < 4; k++) MF(acc[k])
    } else if constexpr (KIND == kMfmaFma) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        MF(acc[k])
#pragma unroll
        for (int i = 0; i < 16; i++) FMA(x[i])
        SB
      }
    } else if constexpr (KIND == kBlockExpCast || KIND == kBlockExpCastValuOnly) {
      // one 64-key block of the ExpCast mainloop per wave: 8 MFMAs 32x32x64 and the row-sum
      // MFMA 16x16x128; 16 max3, 32 fma + 32 cvt_pk_u8 (the codes), 8 bookkeeping fma, in the
      // kernel's region order (PV with the row max and the first key half's codes, QK of the
      // first half with the second half's codes, QK of the second half, the row sum)
      constexpr bool kM = KIND == kBlockExpCast;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        if constexpr (kM) MF(acc[k])
        MAX3(m0, x[8 * k], x[8 * k + 1]) MAX3(m1, x[8 * k + 2], x[8 * k + 3])
        MAX3(m0, x[8 * k + 4], x[8 * k + 5]) MAX3(m1, x[8 * k + 6], x[8 * k + 7])
#pragma unroll
        for (int q = 0; q < 4; q++) { FMA(x[4 * k + q]) CVTU8(p[(4 * k + q) & 15], x[4 * k + q]) }
        SB
      }
#pragma unroll
      for (int k = 0; k < 2; k++) {
        if constexpr (kM) MF(acc[k])
#pragma unroll
        for (int q = 0; q < 8; q++) { FMA(x[16 + 8 * k + q]) CVTU8(p[(8 * k + q) & 15], x[16 + 8 * k + q]) }
        SB
      }
#pragma unroll
      for (int k = 0; k < 2; k++) {
        if constexpr (kM) MF(acc[2 + k])
#pragma unroll
        for (int q = 0; q < 4; q++) FMA(l[q])
        SB
      }
      if constexpr (kM) MF16(racc)
    } else if constexpr (KIND == kBlockExpCastEven) {
      // the same instructions with the nine MFMAs spread evenly over the VALU work
#pragma unroll
      for (int k = 0; k < 9; k++) {
        if (k < 8) { MF(acc[k & 3]) } else { MF16(racc) }
        if (k < 4) {
          MAX3(m0, x[8 * k], x[8 * k + 1]) MAX3(m1, x[8 * k + 2], x[8 * k + 3])
          MAX3(m0, x[8 * k + 4], x[8 * k + 5]) MAX3(m1, x[8 * k + 6], x[8 * k + 7])
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int i = 4 * k + q;
          if (i < 32) { FMA(x[i]) CVTU8(p[i & 15], x[i]) }
        }
        if (k >= 7) {
#pragma unroll
          for (int q = 0; q < 4; q++) FMA(l[q])
        }
        SB
      }
    } else {
      // one 64-key block of the mainloop per wave (32 keys per lane): 8 MFMAs; 16 max3, 32 fma,
      // 32 exp, 16 cvt_pk_fp8, 30 add and 10 bookkeeping fma, in the kernel's region order
      constexpr bool kM = KIND != kBlockValuOnly;
      constexpr bool kSlow = KIND != kBlockPlainSlowOps;
#pragma unroll
      for (int k = 0; k < 4; k++) {  // region 1: PV MFMAs, row max, first key half's fma + exp
        if constexpr (kM) MF(acc[k])
        MAX3(m0, x[8 * k], x[8 * k + 1]) MAX3(m1, x[8 * k + 2], x[8 * k + 3])
        MAX3(m0, x[8 * k + 4], x[8 * k + 5]) MAX3(m1, x[8 * k + 6], x[8 * k + 7])
#pragma unroll
        for (int q = 0; q < 4; q++) {
          FMA(x[4 * k + q])
          if constexpr (kSlow) { EXP(x[4 * k + q]) } else { FMA(x[4 * k + q]) }
        }
        SB
      }
#pragma unroll
      for (int k = 0; k < 2; k++) {  // region 2: QK MFMAs, first half's sums and converts, second half
        if constexpr (kM) MF(acc[k])
#pragma unroll
        for (int q = 0; q < 7; q++) ADD(l[q & 3], x[8 * k + q])
#pragma unroll
        for (int q = 0; q < 4; q++) { if constexpr (kSlow) { CVT(p[4 * k + q], x[8 * k + 2 * q], x[8 * k + 2 * q + 1]) } else { FMA(x[q]) } }
#pragma unroll
        for (int q = 0; q < 8; q++) {
          FMA(x[16 + 8 * k + q])
          if constexpr (kSlow) { EXP(x[16 + 8 * k + q]) } else { FMA(x[16 + 8 * k + q]) }
        }
        SB
      }
#pragma unroll
      for (int k = 0; k < 2; k++) {  // region 3: QK MFMAs, second half's sums and converts
        if constexpr (kM) MF(acc[2 + k])
#pragma unroll
        for (int q = 0; q < 8; q++) ADD(l[q & 3], x[16 + 8 * k + q])
#pragma unroll
        for (int q = 0; q < 4; q++) { if constexpr (kSlow) { CVT(p[4 * k + q], x[16 + 8 * k + 2 * q], x[16 + 8 * k + 2 * q + 1]) } else { FMA(x[q]) } }
#pragma unroll
        for (int q = 0; q < 5; q++) FMA(l[q & 3])
        SB
      }
    }
    SB
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = m0 + m1;
#pragma unroll
  for (int i = 0; i < 32; i++) s += x[i];
#pragma unroll
  for (int i = 0; i < 4; i++) s += l[i] + racc[i];
#pragma unroll
  for (int i = 0; i < 16; i++) s += static_cast<float>(p[i]);
#pragma unroll
  for (int k = 0; k < 4; k++) s += acc[k][0] + acc[k][15];
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + wave;
    out[2 * w] = t1 - t0;
    out[2 * w + 1] = s == 12345.0f ? 1ull : 0ull;  // keeps the work alive
  }
}

// The ExpCast block with the kernel's data dependencies (and no memory operations): the QK
// MFMAs write the scores that the next block's row max and codes read, the codes write the P
// words that the next block's PV MFMAs and this block's row-sum MFMA read. SINGLE: one score
// tile, so the next block's QK of key half t issues after this block's codes of half t (the
// kernel's register reuse). DOUBLE: two score tiles, so the next block's QK issues at the start
// of the block, beside the PV MFMAs, and the scores are ready when the next block starts.
__device__ __forceinline__ v16f mf32(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v4f mf16(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

template <bool DOUBLE>
struct DepState {
  v8i ka[2], kb[2], qa, qb, va, sel, pop;  // distinct K operands per key half
  v16f acc[4], sc[DOUBLE ? 2 : 1][2];
  v4f racc;
  float m;
};

// codes of key half t of the scores x into P words 4t..4t+3
__device__ __forceinline__ void dep_codes(v8i& pop, const v16f& x, int t, float c8, float b8) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    uint32_t word = static_cast<uint32_t>(pop[4 * t + w]);
#pragma unroll
    for (int q = 0; q < 4; q++) word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(x[4 * w + q], c8, b8), q, word);
    pop[4 * t + w] = static_cast<int>(word);
  }
}

template <bool DOUBLE, int CUR>
__device__ __forceinline__ void dep_block(DepState<DOUBLE>& st, float c8, float bb) {
  const v16f z = {};
  constexpr int kNext = DOUBLE ? 1 - CUR : CUR;
  // the operands are opaque per block (as if read from LDS): nothing is hoisted out of the loop
  asm volatile("" : "+v"(st.ka[0]), "+v"(st.kb[0]), "+v"(st.ka[1]), "+v"(st.kb[1]), "+v"(st.qa), "+v"(st.qb), "+v"(st.va));
  if constexpr (DOUBLE) {
    // next block's QK first, beside this block's PV
#pragma unroll
    for (int t = 0; t < 2; t++) {
      st.sc[kNext][t] = mf32(st.ka[t], st.qa, z);
      st.sc[kNext][t] = mf32(st.kb[t], st.qb, st.sc[kNext][t]);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; k++) st.acc[k] = mf32(st.va, st.pop, st.acc[k]);
  const v16f& x0 = st.sc[CUR][0];
  const v16f& x1 = st.sc[CUR][1];
  float mlo = __builtin_elementwise_maximum(x0[0], x0[1]), mhi = __builtin_elementwise_maximum(x0[2], x0[3]);
#pragma unroll
  for (int q = 4; q < 16; q += 4) { mlo = max3f(mlo, x0[q], x0[q + 1]); mhi = max3f(mhi, x0[q + 2], x0[q + 3]); }
#pragma unroll
  for (int q = 0; q < 16; q += 4) { mlo = max3f(mlo, x1[q], x1[q + 1]); mhi = max3f(mhi, x1[q + 2], x1[q + 3]); }
  const float m_new = __builtin_elementwise_maximum(st.m, __builtin_elementwise_maximum(mlo, mhi) * c8);
  const float b8 = __builtin_fmaf(-8.0f, m_new, bb);
  st.m = m_new;
  dep_codes(st.pop, x0, 0, c8, b8);
  if constexpr (!DOUBLE) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
    SB
    st.sc[0][0] = mf32(st.ka[0], st.qa, z);
    st.sc[0][0] = mf32(st.kb[0], st.qb, st.sc[0][0]);
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    SB
  }
  dep_codes(st.pop, x1, 1, c8, b8);
  if constexpr (!DOUBLE) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    }
    SB
    st.sc[0][1] = mf32(st.ka[1], st.qa, z);
    st.sc[0][1] = mf32(st.kb[1], st.qb, st.sc[0][1]);
  }
  st.racc = mf16(st.sel, st.pop, st.racc);
  SB
}

template <bool DOUBLE, int WPS>
__global__ __launch_bounds__(256 * WPS) void probe_dep(unsigned long long* out, int iters, float c8, float bb) {
  __shared__ int pad[24576];  // 96 KB: one workgroup per CU
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  DepState<DOUBLE> st;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    st.ka[0][i] = 0x38383838 + i; st.kb[0][i] = 0x30303030 + i; st.ka[1][i] = 0x38383830 - i; st.kb[1][i] = 0x30303038 - i;
    st.qa[i] = 0x34343434 - i; st.qb[i] = 0x2c2c2c2c + i;
    st.va[i] = 0x38303830 + i; st.sel[i] = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0; st.pop[i] = 0;
  }
  const v16f z = {};
#pragma unroll
  for (int k = 0; k < 4; k++) st.acc[k] = z;
#pragma unroll
  for (int b = 0; b < (DOUBLE ? 2 : 1); b++)
#pragma unroll
    for (int t = 0; t < 2; t++) st.sc[b][t] = mf32(st.ka[t], st.qa, z);
  st.racc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  st.m = -1e30f;
  if (threadIdx.x == 1u << 20) pad[0] = 1;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; it += 2) {
    SB
    dep_block<DOUBLE, 0>(st, c8, bb);
    dep_block<DOUBLE, DOUBLE ? 1 : 0>(st, c8, bb);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = st.m + st.racc[0] + st.racc[3];
#pragma unroll
  for (int k = 0; k < 4; k++) s += st.acc[k][0] + st.acc[k][15];
#pragma unroll
  for (int i = 0; i < 8; i++) s += static_cast<float>(st.pop[i]);
  if (lane == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + wave;
    out[2 * w] = t1 - t0;
    out[2 * w + 1] = s == 12345.0f ? 1ull : 0ull;  // keeps the work alive
  }
}

template <bool DOUBLE, int WPS>
void run_dep(int ncu, unsigned long long* dout) {
  const int iters = 1000, threads = 256 * WPS, nw = ncu * 4 * WPS;
  for (int rep = 0; rep < 2; rep++)
    hipLaunchKernelGGL((probe_dep<DOUBLE, WPS>), dim3(ncu), dim3(threads), 0, 0, dout, iters, 0.01f, 55.65f);
  if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return; }
  std::vector<unsigned long long> h(2 * nw);
  (void)hipMemcpy(h.data(), dout, 16ull * nw, hipMemcpyDeviceToHost);
  std::vector<double> c(nw);
  for (int i = 0; i < nw; i++) c[i] = static_cast<double>(h[2 * i]);
  std::sort(c.begin(), c.end());
  const double per_iter = c[static_cast<size_t>(nw * 0.99)] / iters / WPS;
  printf("%-36s waves/SIMD %d: %8.1f SIMD cycles per wave-iteration (88 VALU + 9 MFMA)\n",
         DOUBLE ? "ExpCast dependent, two score tiles" : "ExpCast dependent, one score tile", WPS, per_iter);
  fflush(stdout);
}

template <int KIND, int WPS>
void run(int ncu, unsigned long long* dout) {
  const int iters = 1000, threads = 256 * WPS, nw = ncu * 4 * WPS;
  for (int rep = 0; rep < 2; rep++)
    hipLaunchKernelGGL((probe<KIND, WPS>), dim3(ncu), dim3(threads), 0, 0, dout, iters, 1.0001f, 0.5f);
  if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return; }
  std::vector<unsigned long long> h(2 * nw);
  (void)hipMemcpy(h.data(), dout, 16ull * nw, hipMemcpyDeviceToHost);
  std::vector<double> c(nw);
  for (int i = 0; i < nw; i++) c[i] = static_cast<double>(h[2 * i]);
  std::sort(c.begin(), c.end());
  const double last = c[static_cast<size_t>(nw * 0.99)];  // a SIMD is done with its last wave
  const double per_iter = last / iters / WPS;             // SIMD cycles per wave-iteration
  const int n = kValu[KIND] + kMfmas[KIND];
  printf("%-36s waves/SIMD %d: %8.1f SIMD cycles per wave-iteration (%d VALU + %d MFMA), %6.2f per instruction\n",
         kNames[KIND], WPS, per_iter, kValu[KIND], kMfmas[KIND], per_iter / n);
  fflush(stdout);
}

template <int WPS>
void run_all(int ncu, unsigned long long* dout) {
  run<kFma, WPS>(ncu, dout);
  run<kAdd, WPS>(ncu, dout);
  run<kMul, WPS>(ncu, dout);
  run<kMax3, WPS>(ncu, dout);
  run<kMax3Legacy, WPS>(ncu, dout);
  run<kExp, WPS>(ncu, dout);
  run<kCvtFp8, WPS>(ncu, dout);
  run<kCvtU8, WPS>(ncu, dout);
  run<kExpFma, WPS>(ncu, dout);
  run<kCvtFma, WPS>(ncu, dout);
  run<kMfma, WPS>(ncu, dout);
  run<kMfmaFma, WPS>(ncu, dout);
  run<kBlock, WPS>(ncu, dout);
  run<kBlockValuOnly, WPS>(ncu, dout);
  run<kBlockPlainSlowOps, WPS>(ncu, dout);
  run<kBlockExpCast, WPS>(ncu, dout);
  run<kBlockExpCastValuOnly, WPS>(ncu, dout);
  run<kBlockExpCastEven, WPS>(ncu, dout);
  if constexpr (WPS < 3) {  // (the two-tile form needs more than a third of the registers)
    run_dep<false, WPS>(ncu, dout);
    run_dep<true, WPS>(ncu, dout);
  }
}

int main() {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  printf("device %s, %d compute units\n", prop.gcnArchName, prop.multiProcessorCount);
  const int ncu = prop.multiProcessorCount;
  unsigned long long* dout = nullptr;
  if (hipMalloc(&dout, 16ull * ncu * 12) != hipSuccess) return 1;  // up to 3 waves per SIMD
  run_all<1>(ncu, dout);
  run_all<2>(ncu, dout);
  run_all<3>(ncu, dout);
  (void)hipFree(dout);
  printf("done\n");
  return 0;
}
