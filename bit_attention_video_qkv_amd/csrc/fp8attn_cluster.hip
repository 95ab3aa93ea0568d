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
// One 1024-thread workgroup per (b, h). Every reduction runs in a fixed order, so the result is
// deterministic; sums are FP64 (the features are bf16 values, exact in FP32).
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

constexpr int kThreads = 1024;

// Fixed-order tree sum of one double per thread over the workgroup; every thread gets the total.
__device__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void vsmooth_cluster(ClusterParams p) {
  __shared__ double red[kThreads];
  __shared__ double stat[kHeadDim];
  __shared__ double cent[kMaxClusters * kMaxFeatures];
  __shared__ int feat[kMaxFeatures];
  __shared__ int counts[kMaxClusters][kThreads / 8 + 1];  // per cluster, per 8-thread group

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int64_t N = p.N;
  const int K = p.n_clusters, F = p.n_feat;
  auto vval = [&](int64_t t, int d) -> float {
    return bf16_to_f32(p.v[((b * N + t) * p.H + h) * kHeadDim + d]);
  };

  // ---- channel variance: mean, then the centred sum of squares (8 token groups x 128 ch) ----
  const int g = tid / kHeadDim, d = tid % kHeadDim;
  for (int pass = 0; pass < 2; pass++) {
    double acc = 0.0;
    const double mean = pass ? stat[d] : 0.0;
    for (int64_t t = g; t < N; t += kThreads / kHeadDim) {
      const double x = static_cast<double>(vval(t, d));
      acc += pass ? (x - mean) * (x - mean) : x;
    }
    red[tid] = acc;
    __syncthreads();
    if (tid < kHeadDim) {
      double s = 0.0;
      for (int gg = 0; gg < kThreads / kHeadDim; gg++) s += red[gg * kHeadDim + tid];
      stat[tid] = s / static_cast<double>(N);  // mean, then variance
    }
    __syncthreads();
  }
  // ---- feature choice: the F largest variances (first channel on ties), ascending order ----
  if (tid == 0) {
    bool taken[kHeadDim];
    for (int c = 0; c < kHeadDim; c++) taken[c] = false;
    for (int f = 0; f < F; f++) {
      int best = -1;
      for (int c = 0; c < kHeadDim; c++)
        if (!taken[c] && (best < 0 || stat[c] > stat[best])) best = c;
      taken[best] = true;
      feat[f] = best;
    }
    for (int i = 1; i < F; i++)  // insertion sort, ascending
      for (int j = i; j > 0 && feat[j - 1] > feat[j]; j--) {
        const int tmp = feat[j];
        feat[j] = feat[j - 1];
        feat[j - 1] = tmp;
      }
  }
  __syncthreads();

  // ---- gather the features of every token (FP32, exact) ----
  float* fv = p.ws_feat + bh * N * F;
  for (int64_t t = tid; t < N; t += kThreads)
    for (int f = 0; f < F; f++) fv[t * F + f] = vval(t, feat[f]);
  int32_t* lab = p.ws_labels + bh * N;
  __syncthreads();  // the gathered features are read by other threads of the workgroup below

  if (tid < K * F) {
    const int c = tid / F, f = tid % F;
    const int64_t t0 = (static_cast<int64_t>(2 * c + 1) * N) / (2 * K);
    cent[tid] = static_cast<double>(fv[t0 * F + f]);
  }
  __syncthreads();

  // each thread owns one contiguous chunk of tokens (this also makes the final scatter stable)
  const int64_t chunk = (N + kThreads - 1) / kThreads;
  const int64_t t_begin = min(N, tid * chunk), t_end = min(N, t_begin + chunk);

  auto assign = [&]() {
    for (int64_t t = t_begin; t < t_end; t++) {
      int best = 0;
      double bd = INFINITY;
      for (int c = 0; c < K; c++) {
        double dist = 0.0;
        for (int f = 0; f < F; f++) {
          const double diff = static_cast<double>(fv[t * F + f]) - cent[c * F + f];
          dist += diff * diff;
        }
        if (dist < bd) {
          bd = dist;
          best = c;
        }
      }
      lab[t] = best;
    }
  };

  for (int it = 0; it < p.iters; it++) {
    assign();
    __syncthreads();
    for (int c = 0; c < K; c++) {
      double cnt = 0.0;
      for (int64_t t = t_begin; t < t_end; t++) cnt += lab[t] == c ? 1.0 : 0.0;
      const double total = block_sum(cnt, red);
      for (int f = 0; f < F; f++) {
        double s = 0.0;
        for (int64_t t = t_begin; t < t_end; t++)
          if (lab[t] == c) s += static_cast<double>(fv[t * F + f]);
        const double sum = block_sum(s, red);
        if (tid == 0 && total > 0.0) cent[c * F + f] = sum / total;
      }
    }
    __syncthreads();
  }
  assign();
  __syncthreads();

  // ---- stable counting sort by cluster id. Counts per 8-thread group keep the LDS small; the
  // eight threads of a group then place their chunks in thread order. ----
  const int grp = tid / 8, lane8 = tid % 8;
  int my_cnt[kMaxClusters];
  for (int c = 0; c < K; c++) my_cnt[c] = 0;
  for (int64_t t = t_begin; t < t_end; t++) my_cnt[lab[t]]++;
  // group totals (lane 0 of each group sums its group in thread order)
  for (int c = 0; c < K; c++) {
    red[tid] = static_cast<double>(my_cnt[c]);
    __syncthreads();
    if (lane8 == 0) {
      int s = 0;
      for (int l = 0; l < 8; l++) s += static_cast<int>(red[tid + l]);
      counts[c][grp] = s;
    }
    __syncthreads();
  }
  // exclusive prefix over (cluster, group) in that order: one thread per cluster scans its row,
  // then the cluster bases are chained
  if (tid < K) {
    int run = 0;
    for (int gg = 0; gg < kThreads / 8; gg++) {
      const int v = counts[tid][gg];
      counts[tid][gg] = run;
      run += v;
    }
    counts[tid][kThreads / 8] = run;  // cluster total
  }
  __syncthreads();
  if (tid == 0) {
    int base = 0;
    for (int c = 0; c < K; c++) {
      const int tot = counts[c][kThreads / 8];
      counts[c][kThreads / 8] = base;
      base += tot;
    }
  }
  __syncthreads();
  int pos[kMaxClusters];
  for (int c = 0; c < K; c++) {
    // offset of this thread inside its group: counts of the earlier lanes of the group
    red[tid] = static_cast<double>(my_cnt[c]);
    __syncthreads();
    int before = 0;
    for (int l = 0; l < lane8; l++) before += static_cast<int>(red[grp * 8 + l]);
    pos[c] = counts[c][kThreads / 8] + counts[c][grp] + before;
    __syncthreads();
  }
  int32_t* out = p.perm + bh * N;
  for (int64_t t = t_begin; t < t_end; t++) out[pos[lab[t]]++] = static_cast<int32_t>(t);
  if (p.labels)
    for (int64_t t = t_begin; t < t_end; t++) p.labels[bh * N + t] = lab[t];
}

}  // namespace

hipError_t launch_cluster(const ClusterParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(vsmooth_cluster, dim3(static_cast<unsigned>(p.B * p.H)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fp8attn
