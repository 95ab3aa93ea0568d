// V-Smooth value clustering -> token permutation (VC-Attention article, section 二, first step:
// a light clustering of the value tokens on a few representative channels, after which tokens
// of one cluster are made contiguous so that each 128-row block of the permuted V is
// homogeneous; clusters need not be balanced, and the permutation is computed once and reused).
//
// Readings where the article is silent (the same reading as the library's documentation):
//   * features: the n_feat channels with the largest variance over the head's tokens (ties to
//     the lower channel), used in ascending channel order;
//   * k-means with n_clusters centroids initialised at tokens floor((2c+1) N / (2 n_clusters)),
//     `iters` Lloyd rounds (assign, then update) and a final assignment; squared L2 distance
//     in FP64, ties to the lower cluster id; an empty cluster keeps its centroid;
//   * perm = the head's tokens stably sorted by cluster id.
//
// Work is split into chunks of tokens (many workgroups per head): kChunk tokens for the channel
// statistics and the gather, kStepChunk for the assignment and the scatter. Partial results are
// combined in ascending chunk order, and a cluster's sums inside a chunk in token order, so every
// result is deterministic. The features are bf16 values: sums of them in FP64 are exact for any
// realistic value range (fewer than 2^21 tokens of 8-bit mantissas spanning under 24 binades),
// which makes the means and centroids independent of the summation order. Distances are formed
// with separately rounded products (never fused).
//
// Kernels per head (b, h), grids (chunks, B*H) unless noted:
//   vc_colsum   channel sums per chunk                     vc_sqdev  centred sums of squares
//   vc_select   (B*H): variances, feature choice, initial centroids
//   vc_gather   the selected features of every token (FP32)
//   vc_step     (step chunks) assignment (+ per-chunk cluster sums, or the final per-chunk and
//               per-sub-chunk counts)
//   vc_update   (B*H): centroids from the chunk sums
//   vc_index    (n_clusters, B*H): the scatter index (per cluster, the tokens before each
//               256-token sub-chunk, and the total)
//   vc_scatter  (step chunks) stable scatter into perm; the fused preparation skips it, and the
//               V block statistics of the quantisation place the tokens from the index
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

constexpr int kChunk = 2048;     // tokens per chunk of the channel statistics and the gather
constexpr int kStepChunk = 512;  // tokens per chunk of the assignment and the scatter (2 per thread)

// fl(a * b), rounded on its own: an FMA with an exact zero addend rounds the exact product once,
// and the compiler neither drops it nor fuses it with the add that follows (as it would fuse a
// plain product), so no scheduling barrier is needed.
__device__ __forceinline__ double dmul_rounded(double a, double b) { return __builtin_fma(a, b, 0.0); }

__device__ __forceinline__ float vval(const ClusterParams& p, int64_t bh, int64_t t, int d) {
  const int64_t b = bh / p.H, h = bh % p.H;
  return bf16_to_f32(p.v[((b * p.N + t) * p.H + h) * kHeadDim + d]);
}

// 1. channel sums of the chunk (FP64, exact): two token halves of 128 channel threads.
__global__ __launch_bounds__(256) void vc_colsum(ClusterParams p) {
  __shared__ double red[kHeadDim];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int d = threadIdx.x & 127, half = threadIdx.x >> 7;
  const int64_t t0 = c * kChunk, t1 = min<int64_t>(p.N, t0 + kChunk);
  double acc = 0.0;
#pragma unroll 8
  for (int64_t t = t0 + half; t < t1; t += 2) acc += static_cast<double>(vval(p, bh, t, d));
  if (half == 1) red[d] = acc;
  __syncthreads();
  if (half == 0) p.ws_part1[(bh * p.n_chunks + c) * kHeadDim + d] = acc + red[d];
}

// 2. centred sums of squares of the chunk around the head's channel mean.
__global__ __launch_bounds__(256) void vc_sqdev(ClusterParams p) {
  __shared__ double red[kHeadDim];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int d = threadIdx.x & 127, half = threadIdx.x >> 7;
  double s = 0.0;
  for (int64_t k = 0; k < p.n_chunks; k++) s += p.ws_part1[(bh * p.n_chunks + k) * kHeadDim + d];
  const double mean = s / static_cast<double>(p.N);
  const int64_t t0 = c * kChunk, t1 = min<int64_t>(p.N, t0 + kChunk);
  double acc = 0.0;
#pragma unroll 8
  for (int64_t t = t0 + half; t < t1; t += 2) {
    const double x = static_cast<double>(vval(p, bh, t, d)) - mean;
    acc += dmul_rounded(x, x);
  }
  if (half == 1) red[d] = acc;
  __syncthreads();
  if (half == 0) p.ws_part2[(bh * p.n_chunks + c) * kHeadDim + d] = acc + red[d];
}

// 3. variances -> the n_feat largest (the lower channel first on ties), ascending; initial
// centroids.
__global__ __launch_bounds__(kHeadDim) void vc_select(ClusterParams p) {
  __shared__ double var[kHeadDim];
  __shared__ int feat[kMaxFeatures];
  __shared__ bool taken[kHeadDim];
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  double s = 0.0;
  for (int64_t k = 0; k < p.n_chunks; k++) s += p.ws_part2[(bh * p.n_chunks + k) * kHeadDim + d];
  var[d] = s / static_cast<double>(p.N);
  __syncthreads();
  // channel d is chosen when fewer than n_feat channels rank above it (a larger variance, or an
  // equal one at a lower channel); the chosen ones take their places in ascending channel order
  int rank = 0;
  const double vd = var[d];
  for (int c = 0; c < kHeadDim; c++) {
    const double vc = var[c];
    rank += (vc > vd || (vc == vd && c < d)) ? 1 : 0;
  }
  taken[d] = rank < p.n_feat;
  __syncthreads();
  if (taken[d]) {
    int pos = 0;
    for (int c = 0; c < d; c++) pos += taken[c] ? 1 : 0;
    feat[pos] = d;
    p.ws_featsel[bh * kMaxFeatures + pos] = d;
  }
  __syncthreads();
  for (int i = d; i < p.n_clusters * p.n_feat; i += kHeadDim) {
    const int c = i / p.n_feat, f = i % p.n_feat;
    const int64_t t0 = (static_cast<int64_t>(2 * c + 1) * p.N) / (2 * p.n_clusters);
    p.ws_cent[(bh * kMaxClusters + c) * kMaxFeatures + f] = static_cast<double>(vval(p, bh, t0, feat[f]));
  }
}

// 4. the selected features of the chunk's tokens, FP32 [N, n_feat] per head.
__global__ __launch_bounds__(256) void vc_gather(ClusterParams p) {
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int64_t t0 = c * kChunk, t1 = min<int64_t>(p.N, t0 + kChunk);
  const int F = p.n_feat;
  for (int64_t i = t0 * F + threadIdx.x; i < t1 * F; i += 256) {
    const int64_t t = i / F;
    const int f = static_cast<int>(i % F);
    p.ws_feat[bh * p.N * F + i] = vval(p, bh, t, p.ws_featsel[bh * kMaxFeatures + f]);
  }
}

// 5. assignment of a step chunk's tokens (thread i: tokens i and i + 256 of the chunk), the
// clusters visited in ascending order with each centroid read once per thread. With sums: the
// chunk's feature sums and count per cluster, each by one thread that walks the chunk's tokens in
// order (labels and features staged in LDS), so a cluster's sums accumulate in token order.
// Final step (sums = 0): the chunk's count per cluster, the labels output, the count per cluster
// of each 256-token sub-chunk and, for the fused preparation, the labels as bytes.
// KF: the feature count when fixed at compile time (8, the default), else 0 (n_feat, up to 16).
template <int KF>
__global__ __launch_bounds__(256) void vc_step(ClusterParams p, int sums) {
  constexpr int kSubs = kStepChunk / kClusterSub;
  constexpr int kFM = KF ? KF : kMaxFeatures;  // feature slots
  static_assert(kStepChunk == 2 * 256 && kStepChunk % kClusterSub == 0, "two tokens per thread");
  __shared__ double cent[kMaxClusters * kMaxFeatures];
  __shared__ float feat_s[kStepChunk][kFM + 1];  // (+1: column walks stay conflict-free)
  __shared__ __attribute__((aligned(16))) int lab_s[kStepChunk];
  __shared__ int cnt_s[kMaxClusters];
  __shared__ int scnt_s[kSubs][kMaxClusters];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int K = p.n_clusters, F = KF ? KF : p.n_feat;
  const int tid = threadIdx.x;
  for (int i = tid; i < K * kMaxFeatures; i += 256) cent[i] = p.ws_cent[bh * kMaxClusters * kMaxFeatures + i];
  if (tid < kMaxClusters) cnt_s[tid] = 0;
  if (tid < kSubs * kMaxClusters) scnt_s[tid / kMaxClusters][tid % kMaxClusters] = 0;
  const int64_t t0 = c * kStepChunk;
  const float* fv = p.ws_feat + bh * p.N * F;
  // the thread's two tokens' features: every load is unconditional (addresses clamped into the
  // head's features; a token past N reads the last one, and its label is dropped), so all are in
  // flight before any is used; the features beyond n_feat are multiplied to zero
  float fx[2][kFM];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int64_t t = t0 + tid + 256 * k;
    const int64_t tc = t < p.N ? t : p.N - 1;
#pragma unroll
    for (int f = 0; f < kFM; f++) {
      if constexpr (KF != 0) fx[k][f] = fv[tc * F + f];
      else fx[k][f] = fv[tc * F + (f < F ? f : F - 1)] * (f < F ? 1.0f : 0.0f);
    }
  }
  if (sums) {
#pragma unroll
    for (int k = 0; k < 2; k++)
#pragma unroll
      for (int f = 0; f < kFM; f++) feat_s[tid + 256 * k][f] = fx[k][f];
  }
  __syncthreads();
  // squared distances with separately rounded products, features in ascending order; the first
  // cluster of the smallest distance wins
  int best[2] = {0, 0};
  double bd[2] = {INFINITY, INFINITY};
  for (int cl = 0; cl < K; cl++) {
    double cv[kFM];
#pragma unroll
    for (int f = 0; f < kFM; f++) cv[f] = f < F ? cent[cl * kMaxFeatures + f] : 0.0;
#pragma unroll
    for (int k = 0; k < 2; k++) {
      // (a feature beyond n_feat adds +0 to the sum, which starts at +0: no effect)
      double dist = 0.0;
#pragma unroll
      for (int f = 0; f < kFM; f++) {
        const double diff = static_cast<double>(fx[k][f]) - cv[f];
        dist += dmul_rounded(diff, diff);
      }
      if (dist < bd[k]) {
        bd[k] = dist;
        best[k] = cl;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int lt = tid + 256 * k;
    const int64_t t = t0 + lt;
    const int lab = t < p.N ? best[k] : -1;
    lab_s[lt] = lab;
    if (lab < 0) continue;
    p.ws_labels[bh * p.N + t] = lab;
    if (!sums) {
      atomicAdd(&cnt_s[lab], 1);  // integer counts: order-free
      atomicAdd(&scnt_s[lt / kClusterSub][lab], 1);
      if (p.labels) p.labels[bh * p.N + t] = lab;
      if (p.ws_lab8) p.ws_lab8[bh * p.lab_stride + t] = static_cast<uint8_t>(lab);
    }
  }
  __syncthreads();
  if (!sums) {
    if (tid < K) p.ws_ccount[(bh * p.n_schunks + c) * kMaxClusters + tid] = cnt_s[tid];
    for (int i = tid; i < kSubs * K; i += 256) {
      const int cl = i / kSubs;
      const int64_t sub = c * kSubs + i % kSubs;
      if (sub < p.n_sub) p.ws_scount[(bh * kMaxClusters + cl) * p.n_sub + sub] = scnt_s[i % kSubs][cl];
    }
    return;
  }
  // one (cluster, feature or count) per thread, the chunk's tokens in order; eight tokens' labels
  // and values are read before their adds, and a token of another cluster adds +0 (the sum
  // starts at +0 and so is never -0, so that leaves it unchanged)
  for (int i = tid; i < K * (F + 1); i += 256) {
    const int cl = i / (F + 1), f = i % (F + 1);
    double acc = 0.0;
    for (int lt = 0; lt < kStepChunk; lt += 8) {
      const int4 la = *reinterpret_cast<const int4*>(&lab_s[lt]);
      const int4 lb = *reinterpret_cast<const int4*>(&lab_s[lt + 4]);
      const int l8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      float v8[8];
#pragma unroll
      for (int u = 0; u < 8; u++) v8[u] = f < F ? feat_s[lt + u][f] : 1.0f;
#pragma unroll
      for (int u = 0; u < 8; u++) acc += l8[u] == cl ? static_cast<double>(v8[u]) : 0.0;
    }
    p.ws_csum[((bh * p.n_schunks + c) * kMaxClusters + cl) * (kMaxFeatures + 1) + f] = acc;
  }
}

// 6. centroids: chunk sums in ascending chunk order; an empty cluster keeps its centroid.
__global__ __launch_bounds__(512) void vc_update(ClusterParams p) {
  const int64_t bh = blockIdx.x;
  const int i = threadIdx.x;
  const int F = p.n_feat;
  if (i >= p.n_clusters * F) return;
  const int cl = i / F, f = i % F;
  double s = 0.0, n = 0.0;
  const int64_t stride = kMaxClusters * (kMaxFeatures + 1);
  const double* col = p.ws_csum + (bh * p.n_schunks * kMaxClusters + cl) * (kMaxFeatures + 1);
  for (int64_t k0 = 0; k0 < p.n_schunks; k0 += 8) {  // eight chunks' loads in flight, adds in order
    double a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int64_t k = k0 + u < p.n_schunks ? k0 + u : p.n_schunks - 1;
      a[u] = col[k * stride + f];
      b[u] = col[k * stride + F];
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (k0 + u < p.n_schunks) {
        s += a[u];
        n += b[u];
      }
    }
  }
  if (n > 0.0) p.ws_cent[(bh * kMaxClusters + cl) * kMaxFeatures + f] = s / n;
}

// 7. stable scatter: positions ordered by (cluster, token). The base of (cluster, step chunk) is
// the tokens of the lower clusters plus this cluster's tokens before the chunk (the scatter
// index: cluster totals and the prefix at the chunk's first sub-chunk); inside the chunk, thread
// i's two consecutive tokens come after those of threads < i.
__global__ __launch_bounds__(256) void vc_scatter(ClusterParams p) {
  constexpr int kSubs = kStepChunk / kClusterSub;
  __shared__ int base[kMaxClusters];
  __shared__ int scan[kMaxClusters][257];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int K = p.n_clusters, tid = threadIdx.x;
  if (tid < K) {
    int before = 0;
    for (int cl = 0; cl < tid; cl++) before += p.ws_ctot[bh * kMaxClusters + cl];
    base[tid] = before + p.ws_sbase[(bh * kMaxClusters + tid) * (p.n_sub + 1) + c * kSubs];
  }
  const int64_t tb = c * kStepChunk + 2 * static_cast<int64_t>(tid);
  int lab[2];
  int my[kMaxClusters];
  for (int cl = 0; cl < K; cl++) my[cl] = 0;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int64_t t = tb + k;
    lab[k] = t < p.N ? p.ws_labels[bh * p.N + t] : -1;
    for (int cl = 0; cl < K; cl++) my[cl] += lab[k] == cl ? 1 : 0;
  }
  for (int cl = 0; cl < K; cl++) scan[cl][tid] = my[cl];
  __syncthreads();
  if (tid < K) {  // exclusive prefix over the threads, per cluster
    int run = 0;
    for (int i = 0; i < 256; i++) {
      const int v = scan[tid][i];
      scan[tid][i] = run;
      run += v;
    }
  }
  __syncthreads();
  int pos[kMaxClusters];
  for (int cl = 0; cl < K; cl++) pos[cl] = base[cl] + scan[cl][tid];
  int32_t* out = p.perm + bh * p.N;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    if (lab[k] < 0) continue;
    out[pos[lab[k]]++] = static_cast<int32_t>(tb + k);
  }
}

// 7'. scatter index, grid (n_clusters, B*H): the tokens of cluster c before each sub-chunk
// (exclusive prefix over the sub-chunks in ascending order, 256 at a time: wave scans, then the
// four waves in order) and the cluster's total.
__global__ __launch_bounds__(256) void vc_index(ClusterParams p) {
  __shared__ int wsum[4];
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* cnt = p.ws_scount + (bh * kMaxClusters + c) * p.n_sub;
  int32_t* sb = p.ws_sbase + (bh * kMaxClusters + c) * (p.n_sub + 1);
  int carry = 0;
  for (int64_t s0 = 0; s0 < p.n_sub; s0 += 256) {
    const int64_t s = s0 + tid;
    const int v = s < p.n_sub ? cnt[s] : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      incl += lane >= d ? y : 0;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    if (s < p.n_sub) sb[s] = carry + before + incl - v;
    carry += total;
    __syncthreads();  // (wsum is rewritten by the next pass)
  }
  if (tid == 0) {
    sb[p.n_sub] = carry;
    p.ws_ctot[bh * kMaxClusters + c] = carry;
  }
}

}  // namespace

hipError_t launch_cluster(const ClusterParams& p, hipStream_t stream) {
  const unsigned bh = static_cast<unsigned>(p.B * p.H), nc = static_cast<unsigned>(p.n_chunks);
  const dim3 g(nc, bh), gs(static_cast<unsigned>(p.n_schunks), bh);
  hipLaunchKernelGGL(vc_colsum, g, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(vc_sqdev, g, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(vc_select, dim3(bh), dim3(kHeadDim), 0, stream, p);
  hipLaunchKernelGGL(vc_gather, g, dim3(256), 0, stream, p);
  auto step = [&](int sums) {
    if (p.n_feat == 8) hipLaunchKernelGGL(vc_step<8>, gs, dim3(256), 0, stream, p, sums);
    else hipLaunchKernelGGL(vc_step<0>, gs, dim3(256), 0, stream, p, sums);
  };
  for (int it = 0; it < p.iters; it++) {
    step(1);
    hipLaunchKernelGGL(vc_update, dim3(bh), dim3(512), 0, stream, p);
  }
  step(0);
  hipLaunchKernelGGL(vc_index, dim3(static_cast<unsigned>(p.n_clusters), bh), dim3(256), 0, stream, p);
  // the fused preparation places the tokens in the V block statistics instead
  if (!p.ws_lab8) hipLaunchKernelGGL(vc_scatter, gs, dim3(256), 0, stream, p);
  return hipGetLastError();
}

int64_t cluster_chunks(int64_t N) { return (N + kChunk - 1) / kChunk; }
int64_t cluster_step_chunks(int64_t N) { return (N + kStepChunk - 1) / kStepChunk; }

}  // namespace fp8attn
