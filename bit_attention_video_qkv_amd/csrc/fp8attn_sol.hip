// Sol routing (TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", sections "Sol Routing"
// and "SM90 CuTe Mainloop"): the sequence is cut into 64-token Q and KV blocks; every KV block
// gets a K summary and a V summary; a threshold theta = mu + tau * sigma per Q block (diag or
// exact estimator) decides, from a route QK of the block-quantised Q with the quantised K
// summaries, which KV blocks take the exact route (full E4M3 QK, online softmax, E4M3 PV) and
// which the summary route (the block as n_j copies of its summary key and value). Sink blocks are
// always exact.
//
// Readings (the page leaves these open):
//  * summaries are block means of the dequantised E4M3 K and V:
//      kbar = fl32(fl32(sum_t decode(K8) * s_k) / n_j)   (the code sum is exact in FP32),
//      vbar likewise with the channel scale, stored as BF16 (in the summary PV's operand order);
//  * the K summaries are quantised like K, per group of 64 summaries (scale = amax / 448);
//  * mu and sigma are the mean and standard deviation of the Q block's route scores over all
//    pairs (valid query, KV block), from second moments: mu = ss * qbar . m,
//    E2 = ss^2 * sum_{d,e} Mq[d,e] Mk[d,e] ("exact") or ss^2 * sum_d Mq[d,d] Mk[d,d] ("diag"),
//    m and Mk the mean and second moment of the summaries, Mq the block's query second moment;
//  * a KV block is exact for Q block u when some valid query of u has a route score >= theta_u;
//  * both routes share one online-softmax state (the page's unified merge). The KV blocks are
//    taken in route groups of 64, groups in KV order, each group's summary blocks before its
//    exact blocks: a summary block moves the running max to max(m, r_ij) and adds
//    n_j exp(r_ij - m') to the row sum and n_j exp(r_ij - m') vbar_j to the accumulator; an exact
//    block then takes the ordinary FP8 step against that running max. Only the running max the
//    exact blocks' P codes are taken against depends on the order; the summary contributions
//    are plain sums. So sol_route accumulates them in a state of its own and writes, per row and
//    group, the running max of the summary scores over the groups so far (gmax); the exact
//    route (fp8attn_attn.hip) folds gmax into its running max before each group's exact blocks
//    and adds the two accumulators in its epilogue, each rescaled to the common maximum.
//
// Kernels (launch order):
//   sol_summaries  grid (NBp, B*H)         K and V summaries
//   sol_kquant     grid (NBg, B*H)         quantised K summaries
//   sol_kmoments   grid (B*H) or (B*H, 16) mean and second moment of the summaries (FP64)
//   sol_theta      grid (NB, B*H)          threshold per Q block
//   sol_route      grid (ceil(NB/2), B*H), 4 waves: per group of 64 summaries staged in LDS (the
//                  groups in KV order), the route QK (E4M3 MFMA), the exact-block mask, the
//                  summary contributions (BF16 MFMA) and the running summary maximum
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16(const bf16x8& a, const bf16x8& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// V summaries are stored in the order the summary PV reads them: for (b*h, group g, tile t,
// k-step s, channel tile dt), 64 lanes x 8 BF16 values, lane 32h + l32 holding channel
// 32dt + l32 and summaries 32t + 16s + {4h + 0..3, 8 + 4h + 0..3} (element e: summary
// 32t + 16s + 8(e/4) + 4h + e%4), so each operand is one 16-byte load per lane.
__device__ __forceinline__ int64_t vsum_index(const SolParams& p, int64_t bh, int64_t j, int d) {
  const int64_t g = j >> 6;
  const int js = static_cast<int>(j & 63), t = js >> 5, s = (js >> 4) & 1, rem = js & 15;
  const int h = (rem >> 2) & 1, e = 4 * (rem >> 3) + (rem & 3);
  const int dt = d >> 5, lane = 32 * h + (d & 31);
  return ((((bh * p.NBg + g) * 2 + t) * 2 + s) * 4 + dt) * 512 + lane * 8 + e;
}

// 1. Summaries of KV block j (grid over the padded count NBp: padding summaries get a zero V
// summary, which the summary PV multiplies by p = 0). Threads 0..127: K channel d; 128..255: V
// channel d. Rows and positions past N hold code 0 (the quantisation contract), so all 64 are
// summed.
__global__ __launch_bounds__(256) void sol_summaries(SolParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kt[64][kHeadDim + 16];
  const int64_t j = blockIdx.x, bh = blockIdx.y;
  if (j >= p.NB) {
    if (threadIdx.x >= kHeadDim) p.vsumT[vsum_index(p, bh, j, threadIdx.x - kHeadDim)] = 0;
    return;
  }
  // the K tile (64 rows x 128 bytes) through LDS with 16-byte loads
  const uint4* ksrc = reinterpret_cast<const uint4*>(p.k8 + (bh * p.N64 + 64 * j) * kHeadDim);
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int L = c * 256 + threadIdx.x;  // 512 chunks of 16 bytes
    *reinterpret_cast<uint4*>(&kt[L >> 3][(L & 7) * 16]) = ksrc[L];
  }
  __syncthreads();
  const int n = static_cast<int>(min<int64_t>(64, p.N - 64 * j));
  if (threadIdx.x < kHeadDim) {
    const int d = threadIdx.x;
    float s = 0.0f;
#pragma unroll 16
    for (int r = 0; r < 64; r++) s += e4m3_to_f32(kt[r][d]);
    const float prod = s * p.k_scale[bh * p.NB + j];
    p.ksum[(bh * p.NB + j) * kHeadDim + d] = __fdiv_rn(prod, static_cast<float>(n));
  } else {
    const int d = threadIdx.x - kHeadDim;
    const uint4* vp = reinterpret_cast<const uint4*>(p.v8t + (bh * kHeadDim + d) * p.N64 + 64 * j);
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const uint4 w = vp[c];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const f32x2 lo = e4m3x2_to_f32(ws[q], false), hi = e4m3x2_to_f32(ws[q], true);
        s += lo.x;
        s += lo.y;
        s += hi.x;
        s += hi.y;
      }
    }
    const float prod = s * p.v_scale[bh * kHeadDim + d];
    p.vsumT[vsum_index(p, bh, j, d)] = f32_to_bf16_rne(__fdiv_rn(prod, static_cast<float>(n)));
  }
}

// 2. Quantised K summaries: group g = summaries 64g .. 64g+63 (rows >= NB are zero). Thread t:
// channels 8*(t%16)..+7 of rows t/16 + 16*pass.
__global__ __launch_bounds__(256) void sol_kquant(SolParams p) {
  __shared__ float red[4];
  const int64_t g = blockIdx.x, bh = blockIdx.y;
  const int chunk = threadIdx.x & 15, row0 = threadIdx.x >> 4;
  float x[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int64_t j = 64 * g + row0 + 16 * pass;
    if (j < p.NB) {
      const float4* src = reinterpret_cast<const float4*>(p.ksum + (bh * p.NB + j) * kHeadDim + chunk * 8);
      const float4 a = src[0], b = src[1];
      x[pass][0] = a.x; x[pass][1] = a.y; x[pass][2] = a.z; x[pass][3] = a.w;
      x[pass][4] = b.x; x[pass][5] = b.y; x[pass][6] = b.z; x[pass][7] = b.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; q++) x[pass][q] = 0.0f;
    }
#pragma unroll
    for (int q = 0; q < 8; q++) amax = fmaxf(amax, fabsf(x[pass][q]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
  if (threadIdx.x == 0) p.kq_scale[bh * p.NBg + g] = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int64_t j = 64 * g + row0 + 16 * pass;
    float y[8];
#pragma unroll
    for (int q = 0; q < 8; q++) y[q] = x[pass][q] * inv;
    uint2 out;
    out.x = e4m3x4(y[0], y[1], y[2], y[3]);
    out.y = e4m3x4(y[4], y[5], y[6], y[7]);
    *reinterpret_cast<uint2*>(p.kq8 + (bh * p.NBp + j) * kHeadDim + chunk * 8) = out;
  }
}

// 3. Mean and second moment of the summaries (FP64, ascending j). FULL (the exact estimator):
// grid (B*H, 16), workgroup y computes rows 8y..8y+7 of Mk (thread t: row 8y + t/32, columns
// 4*(t%32)..+3); otherwise (the diag estimator, which reads only the diagonal): grid (B*H),
// thread d computes Mk[d][d]. The thread that owns row d's first columns also sums the mean of
// channel d. Each thread holds the next batch of summaries in registers while it folds the
// current one in, so that many loads are in flight while the sums stay in order.
template <bool FULL>
__global__ __launch_bounds__(256) void sol_kmoments(SolParams p) {
  constexpr int kBatch = FULL ? 16 : 32;
  const int64_t bh = blockIdx.x;
  const int d = FULL ? static_cast<int>(blockIdx.y) * 8 + static_cast<int>(threadIdx.x >> 5)
                     : static_cast<int>(threadIdx.x);
  const int e0 = FULL ? static_cast<int>(threadIdx.x & 31) * 4 : d;
  const float* ks = p.ksum + bh * p.NB * kHeadDim;
  double acc[4] = {0.0, 0.0, 0.0, 0.0}, msum = 0.0;
  auto load = [&](int64_t j, float& a, float4& b) {
    a = ks[j * kHeadDim + d];
    if constexpr (FULL) b = *reinterpret_cast<const float4*>(ks + j * kHeadDim + e0);
  };
  auto fold = [&](float a, const float4& b) {
    const double ad = static_cast<double>(a);
    msum += ad;
    if constexpr (FULL) {
      acc[0] += ad * static_cast<double>(b.x);
      acc[1] += ad * static_cast<double>(b.y);
      acc[2] += ad * static_cast<double>(b.z);
      acc[3] += ad * static_cast<double>(b.w);
    } else {
      acc[0] += ad * ad;
    }
  };
  const int64_t n_full = p.NB / kBatch * kBatch;
  float a_cur[kBatch], a_nxt[kBatch];
  float4 b_cur[kBatch], b_nxt[kBatch];
  if (n_full > 0) {
#pragma unroll
    for (int u = 0; u < kBatch; u++) load(u, a_cur[u], b_cur[u]);
  }
  for (int64_t j = 0; j < n_full; j += kBatch) {
    if (j + kBatch < n_full) {
#pragma unroll
      for (int u = 0; u < kBatch; u++) load(j + kBatch + u, a_nxt[u], b_nxt[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; u++) fold(a_cur[u], b_cur[u]);
#pragma unroll
    for (int u = 0; u < kBatch; u++) {
      a_cur[u] = a_nxt[u];
      b_cur[u] = b_nxt[u];
    }
  }
  for (int64_t j = n_full; j < p.NB; j++) {
    float a;
    float4 b;
    load(j, a, b);
    fold(a, b);
  }
  const double inv_nb = 1.0 / static_cast<double>(p.NB);
  if constexpr (FULL) {
#pragma unroll
    for (int q = 0; q < 4; q++) p.Mk[(bh * kHeadDim + d) * kHeadDim + e0 + q] = acc[q] * inv_nb;
  } else {
    p.Mk[(bh * kHeadDim + d) * kHeadDim + d] = acc[0] * inv_nb;
  }
  if (!FULL || (threadIdx.x & 31) == 0) p.mk[bh * kHeadDim + d] = msum * inv_nb;
}

__device__ __forceinline__ double block_sum_128(double v, double* red) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = red[0] + red[1];
  __syncthreads();
  return r;
}

// 4. Threshold of Q block u. Thread e: channel e. The query codes c_i sit in LDS (the exact
// estimator: decoded, exact in FP32, for its M_k products; the diag estimator: the bytes, which
// keeps a workgroup's LDS at 8 KB); q_i = s_q * c_i. Rows past N hold code 0.
template <bool EXACT>
__global__ __launch_bounds__(128) void sol_theta(SolParams p) {
  __shared__ float c[EXACT ? 64 : 1][kHeadDim + 1];
  __shared__ __attribute__((aligned(16))) uint8_t cb[EXACT ? 1 : 64][kHeadDim];
  __shared__ double red[2];
  const int64_t u = blockIdx.x, bh = blockIdx.y;
  const int e = threadIdx.x;
  const int nq = static_cast<int>(min<int64_t>(64, p.N - 64 * u));
  // (issued before the block's codes, so that their latencies overlap)
  const double sq = p.q_scale[bh * p.NB + u];
  const double mk_e = p.mk[bh * kHeadDim + e];
  const double mk_ee = EXACT ? 0.0 : p.Mk[(bh * kHeadDim + e) * kHeadDim + e];
  const uint4* qb = reinterpret_cast<const uint4*>(p.q8 + (bh * p.N64 + 64 * u) * kHeadDim);
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int L = k * 128 + e;  // 512 chunks of 16 bytes: row L / 8, bytes 16 * (L % 8) ..
    const int i = L >> 3, d0 = (L & 7) * 16;
    const uint4 w = qb[L];
    if constexpr (EXACT) {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 16; q++) c[i][d0 + q] = e4m3_to_f32((ws[q >> 2] >> (8 * (q & 3))) & 0xFFu);
    } else {
      *reinterpret_cast<uint4*>(&cb[i][d0]) = w;
    }
  }
  __syncthreads();
  auto code = [&](int i, int d) -> float {
    if constexpr (EXACT) return c[i][d];
    else return e4m3_to_f32(cb[i][d]);
  };
  // over all 64 rows (rows past nq hold 0). Both sums are exact in any order: a decoded code is
  // a multiple of 2^-9 below 2^9, so 64 of them sum exactly in FP32 (24 bits); its square (at
  // most 8 significant bits) is exact in FP32, and 64 squares sum exactly in FP64.
  float csum = 0.0f;
  double csq = 0.0;
#pragma unroll 16
  for (int i = 0; i < 64; i++) {
    const float v = code(i, e);
    csum += v;
    csq += static_cast<double>(v * v);
  }
  // mu = ss * sq * mean_i c_i . m
  const double mu = block_sum_128(static_cast<double>(csum) / nq * mk_e, red) * sq * p.softmax_scale;
  double part;
  if constexpr (!EXACT) {
    part = csq / nq * mk_ee;
  } else {
    // sum_i c_i[e] (Mk c_i)[e] / nq, with (Mk c_i)[e] = sum_d Mk[d][e] c_i[d] (Mk symmetric)
    float y[64];
#pragma unroll
    for (int i = 0; i < 64; i++) y[i] = 0.0f;
    const double* mrow = p.Mk + bh * kHeadDim * kHeadDim + e;
    for (int d = 0; d < kHeadDim; d++) {
      const float m = static_cast<float>(mrow[d * kHeadDim]);
#pragma unroll
      for (int i = 0; i < 64; i++) y[i] = __builtin_fmaf(m, code(i, d), y[i]);
    }
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 64; i++) acc += static_cast<double>(code(i, e)) * y[i];
    part = acc / nq;
  }
  const double e2 = block_sum_128(part, red) * sq * sq * p.softmax_scale * p.softmax_scale;
  if (e == 0) {
    const double var = e2 - mu * mu;
    p.theta[bh * p.NB + u] = static_cast<float>(mu + p.tau * sqrt(var > 0.0 ? var : 0.0));
  }
}

__device__ __forceinline__ void load_q_operand(const SolParams& p, int64_t bh, int64_t qrow, int lh, v8i (&qop)[2]) {
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const uint4* g = reinterpret_cast<const uint4*>(p.q8 + (bh * p.N64 + qrow) * kHeadDim + 64 * c + 32 * lh);
    const uint4 a = g[0], b = g[1];  // rows past N are code 0 (row < N64)
    qop[c][0] = a.x; qop[c][1] = a.y; qop[c][2] = a.z; qop[c][3] = a.w;
    qop[c][4] = b.x; qop[c][5] = b.y; qop[c][6] = b.z; qop[c][7] = b.w;
  }
}

// LDS slot of one group of 64 summaries: the quantised K summaries (64 rows of 128 bytes, the
// 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 7), so that 16 lanes reading 16 rows
// touch every bank once) and the V summaries in operand order (16 blocks of 64 lanes x 16 bytes).
constexpr int kSlotK = 64 * kHeadDim;          // 8 KB
constexpr int kSlotBytes = kSlotK + 64 * kHeadDim * 2;  // + 16 KB
constexpr int kCopiesPerThread = kSlotBytes / 16 / 256;  // 6

__device__ __forceinline__ int kq_swz(int row) { return (row >> 1) & 7; }

// 5. Route of two Q blocks (workgroup of four waves; waves 2b and 2b+1 hold the 64 queries of Q
// block 2x + b). Per group of 64 summaries, staged in LDS (double-buffered direct copies):
//   route scores S^T = Kq Q^T on the E4M3 matrix cores (lane (query l32, half h) register r of
//   tile t holds summary 32t + 8(r/4) + 4h + r%4); the group's mask word = OR over the Q block's
//   valid queries of (score >= theta), plus the sinks;
//   the summary route over the non-exact summaries: online softmax of (score * log2 e +
//   log2 n_j) and PV with the V summaries on the BF16 matrix cores (O^T = Vbar^T P^T; a lane's
//   P values of tile t, registers 8s..8s+7, are the B operand of k-step (t, s)).
// The per-summary bookkeeping (mask bits, selection) stays in vector registers: the scalar unit
// issues for a SIMD only every fourth cycle, so per-summary scalar work would bound the kernel.
typedef const __attribute__((address_space(4))) float ConstF32;

// OR over the 64 lanes: DPP within each row of 16 lanes, then across row pairs and halves.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x124, 0xF, 0xF, false));  // rotate 4
  v |= static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x128, 0xF, 0xF, false));  // rotate 8
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] | a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] | b[1];
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void sol_route(SolParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kSlotBytes];
  __shared__ uint64_t word_s[4];
  const int64_t bh = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lh = lane >> 5, l32 = lane & 31;
  const int64_t u = 2 * static_cast<int64_t>(blockIdx.x) + (wave >> 1);  // this wave's Q block
  const bool ublock = u < p.NB;                                          // (uniform per wave)
  const int64_t qrow = 64 * u + 32 * (wave & 1) + l32;
  const bool qvalid = ublock && qrow < p.N;
  const float theta_u = ublock ? p.theta[bh * p.NB + u] : 0.0f;
  const float theta = qvalid ? theta_u : INFINITY;  // rows past N never make a block exact
  const float sq = ublock ? p.q_scale[bh * p.NB + u] : 0.0f;
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  constexpr float kLazy = 8.0f;
  // every KV block holds 64 tokens except the last one
  const float lg_last = __log2f(static_cast<float>(p.N - 64 * (p.NB - 1)));
  // the group scales are read-only here: scalar loads, which leave the copies' counter alone
  ConstF32* kqs = (ConstF32*)(p.kq_scale + bh * p.NBg);

  // copies of group g into slot g & 1: thread t issues chunks L = r * 256 + t (r < 6); the first
  // 512 chunks are the K summary tile (swizzled), the next 1024 the V summary tile (contiguous)
  const uint8_t* kq_base = p.kq8 + bh * p.NBp * kHeadDim;
  const uint8_t* vs_base = reinterpret_cast<const uint8_t*>(p.vsumT) + bh * p.NBg * (64 * kHeadDim * 2);
  auto stage = [&](int64_t g, int sl) {
    const uint32_t l0 = lds_addr_of(lds + sl * kSlotBytes);
#pragma unroll
    for (int r = 0; r < kCopiesPerThread; r++) {
      const int L = r * 256 + static_cast<int>(threadIdx.x);
      const uint32_t ldst = l0 + (r * 256 + wave * 64) * 16;
      if (r < 2) {
        const int row = L >> 3, pc = L & 7, c = pc ^ kq_swz(row);
        copy16_to_lds(kq_base + g * 64 * kHeadDim, static_cast<uint32_t>(row * kHeadDim + c * 16), ldst);
      } else {
        copy16_to_lds(vs_base + g * (64 * kHeadDim * 2), static_cast<uint32_t>((L - 512) * 16), ldst);
      }
    }
  };

  v8i qop[2];
  load_q_operand(p, bh, ublock ? qrow : 0, lh, qop);
  v16f oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[dt][r] = 0.0f;
  float m_run = -INFINITY;  // log2 units
  float l_part = 0.0f;
  // running max of the summary route scores over the groups visited so far (log2 units)
  float g_run = -INFINITY;
  float* gmax_row = p.gmax + bh * p.NBg * p.N64 + (ublock ? qrow : 0);

  // the groups in KV order (the exact route takes each group's summary maximum in that order)
  auto group_at = [&](int64_t gi) -> int64_t { return p.reverse ? p.NBg - 1 - gi : gi; };
  stage(group_at(0), 0);
  for (int64_t gi = 0; gi < p.NBg; gi++) {
    const int64_t g = group_at(gi);
    wait_vmcnt<0>();
    // group g has landed in every wave's view, and every wave is done with the other slot
    barrier_nofence();
    if (gi + 1 < p.NBg) stage(group_at(gi + 1), static_cast<int>((gi + 1) & 1));
    const uint8_t* ks = lds + (gi & 1) * kSlotBytes;
    const uint8_t* vsl = ks + kSlotK;
    const int64_t left = p.NB - 64 * g;  // summaries from this group on
    const uint64_t valid = left >= 64 ? ~0ull : (1ull << left) - 1ull;

    // the route scores and the mask run at a raised wave priority, the summary route at the
    // normal one, so that the waves of a SIMD take turns by phase (measured faster)
    __builtin_amdgcn_s_setprio(1);
    // route scores
    const float cs = sq * kqs[g] * p.softmax_scale;
    float x[2][16];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = 32 * t + l32;
      const int sw = kq_swz(row);
      v8i kop[2];
#pragma unroll
      for (int c = 0; c < 2; c++) {
        const int c0 = 4 * c + 2 * lh;
        const uint4 a = *reinterpret_cast<const uint4*>(ks + row * kHeadDim + ((c0 ^ sw) * 16));
        const uint4 b = *reinterpret_cast<const uint4*>(ks + row * kHeadDim + (((c0 + 1) ^ sw) * 16));
        kop[c][0] = a.x; kop[c][1] = a.y; kop[c][2] = a.z; kop[c][3] = a.w;
        kop[c][4] = b.x; kop[c][5] = b.y; kop[c][6] = b.z; kop[c][7] = b.w;
      }
      v16f z;
#pragma unroll
      for (int r = 0; r < 16; r++) z[r] = 0.0f;
      v16f acc = mfma_f8(kop[0], qop[0], z);
      acc = mfma_f8(kop[1], qop[1], acc);
#pragma unroll
      for (int r = 0; r < 16; r++) x[t][r] = acc[r] * cs;
    }
    // mask word of this wave's 32 queries: each lane packs its hits at the summaries' bit
    // positions, then an OR over the wave (the two half-waves hold different summaries)
    uint32_t wt[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      uint32_t b = 0u;
#pragma unroll
      for (int r = 0; r < 16; r++) b |= x[t][r] >= theta ? 1u << (8 * (r >> 2) + (r & 3)) : 0u;
      wt[t] = wave_or(b << (4 * lh));
    }
    // (readfirstlane returns a signed int: widen through uint32_t, not by sign extension)
    uint64_t word = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wt[1]))) << 32) |
                    static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wt[0]));
    if (lane == 0) word_s[wave] = word;
    wait_lgkm0();
    barrier_nofence();
    const int pw = wave & 2;  // first wave of this Q block's pair
    word = (word_s[pw] | word_s[pw + 1]) & valid;
    const int64_t sink_end = min<int64_t>(static_cast<int64_t>(p.sink_blocks), p.NB) - 64 * g;
    if (sink_end > 0) word |= sink_end >= 64 ? ~0ull : ((1ull << sink_end) - 1ull);
    if (ublock && (wave & 1) == 0 && lane == 0) p.mask[(bh * p.NB + u) * p.W + g] = word;

    __builtin_amdgcn_s_setprio(0);
    // summary route over the group's non-exact summaries
    const uint64_t sbits = valid & ~word;
    if (ublock && sbits != 0ull) {
      if (sbits != ~0ull) {  // exact and padding summaries drop out
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const uint32_t sv = static_cast<uint32_t>(sbits >> (32 * t)) >> (4 * lh);  // this lane's bits
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int pos = 8 * (r >> 2) + (r & 3);
            const uint32_t keep = static_cast<uint32_t>(static_cast<int32_t>(sv << (31 - pos)) >> 31);
            x[t][r] = __uint_as_float((__float_as_uint(x[t][r]) & keep) | (0xFF800000u & ~keep));
          }
        }
      }
      // the group's largest summary score (before the block-length correction below)
      float gm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) gm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(gm, x[t][r]), x[t][r + 1]);
      {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(gm), __float_as_uint(gm), false, false);
        gm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      g_run = fmaxf(g_run, gm * kLog2e);
      if (left <= 64) {  // the last KV block weighs its token count instead of 64
        const int jl = static_cast<int>(left) - 1;
        const float dx = (lg_last - 6.0f) * kLn2;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            if (32 * t + 8 * (r >> 2) + 4 * lh + (r & 3) == jl) x[t][r] += dx;
      }
      // weight exponents score * log2 e + 6 (gm is finite: the group has a summary-routed block,
      // and it bounds every corrected score from above). The reference point m_run moves only
      // when some row's maximum passes it by more than kLazy, so the accumulators are rescaled a
      // few times per row, not every group; weights stay below 2^kLazy.
      const float ml2 = __builtin_fmaf(gm, kLog2e, 6.0f);
      if (__builtin_amdgcn_ballot_w64(ml2 > m_run + kLazy) != 0ull) {
        const float m_new = fmaxf(m_run, ml2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on a row's first group
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
          for (int r = 0; r < 16; r++) oacc[dt][r] *= alpha;
      }
      const float c6 = 6.0f - m_run;
      float psum = 0.0f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(x[t][r], kLog2e, c6));
          psum += pv;
          pb[t][r >> 3][r & 7] = static_cast<__bf16>(pv);
        }
      l_part += psum;
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
          for (int dt = 0; dt < 4; dt++) {
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(vsl + ((((t * 2 + s2) * 4 + dt) * 64 + lane) * 16));
            oacc[dt] = mfma_bf16(av, pb[t][s2], oacc[dt]);
          }
    }
    if (ublock && lh == 0) gmax_row[g * p.N64] = g_run;
    wait_lgkm0();  // every read of this slot has returned before the next barrier frees it
  }

  // epilogue: the summary route's normalised output and log2 of its weight, in the units of the
  // exact route (S-scaled row sums); the exact route's epilogue merges it with its own
  if (!qvalid) return;
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
  const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  float* orow = p.o_part + (bh * p.N + qrow) * kHeadDim;
  const bool any = m_run > -INFINITY;
  const float inv_l = any ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      const int d0 = 32 * dt + 8 * g4 + 4 * lh;
      float4 o;
      o.x = oacc[dt][4 * g4 + 0] * inv_l;
      o.y = oacc[dt][4 * g4 + 1] * inv_l;
      o.z = oacc[dt][4 * g4 + 2] * inv_l;
      o.w = oacc[dt][4 * g4 + 3] * inv_l;
      *reinterpret_cast<float4*>(orow + d0) = o;
    }
  if (lh == 0) p.lse[bh * p.N + qrow] = any ? m_run + __log2f(l_tot) + p.log2S : -INFINITY;
}

}  // namespace

hipError_t launch_sol(const SolParams& p, hipStream_t stream) {
  const unsigned bh = static_cast<unsigned>(p.B * p.H);
  hipLaunchKernelGGL(sol_summaries, dim3(static_cast<unsigned>(p.NBp), bh), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sol_kquant, dim3(static_cast<unsigned>(p.NBg), bh), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.estimator == 0) hipLaunchKernelGGL(sol_kmoments<false>, dim3(bh), dim3(kHeadDim), 0, stream, p);
  else hipLaunchKernelGGL(sol_kmoments<true>, dim3(bh, kHeadDim / 8), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.estimator == 0) hipLaunchKernelGGL(sol_theta<false>, dim3(static_cast<unsigned>(p.NB), bh), dim3(128), 0, stream, p);
  else hipLaunchKernelGGL(sol_theta<true>, dim3(static_cast<unsigned>(p.NB), bh), dim3(128), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sol_route, dim3(static_cast<unsigned>((p.NB + 1) / 2), bh), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8attn
