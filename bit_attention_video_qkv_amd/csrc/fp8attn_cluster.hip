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
// Work is split into chunks of kChunk tokens (many workgroups per head); partial results are
// combined in ascending chunk order, so every result is deterministic. The features are bf16
// values: sums of them in FP64 are exact for any realistic value range (fewer than 2^21 tokens
// of 8-bit mantissas spanning under 24 binades), which makes the means and centroids independent
// of the summation order. Distances are formed with separately rounded products (never fused).
//
// Kernels per head (b, h), grids (chunks, B*H) unless noted:
//   vc_colsum   channel sums per chunk                     vc_sqdev  centred sums of squares
//   vc_select   (B*H): variances, feature choice, initial centroids
//   vc_gather   the selected features of every token (FP32)
//   vc_step     assignment (+ per-chunk cluster sums, or the final per-chunk counts)
//   vc_update   (B*H): centroids from the chunk sums          vc_scatter  stable scatter
//   vc_index    (n_clusters, B*H): instead of vc_scatter, the scatter index from which the V block
//               statistics of the quantisation place the tokens themselves
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

constexpr int kChunk = 2048;  // tokens per chunk
constexpr int kTpt = kChunk / 256;  // tokens per thread in vc_step / vc_scatter (contiguous)

__device__ __forceinline__ double dmul_rounded(double a, double b) {
  double p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

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

// 3. variances -> the n_feat largest (first channel on ties), ascending; initial centroids.
__global__ __launch_bounds__(kHeadDim) void vc_select(ClusterParams p) {
  __shared__ double var[kHeadDim];
  __shared__ int feat[kMaxFeatures];
  __shared__ bool taken[kHeadDim];
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  double s = 0.0;
  for (int64_t k = 0; k < p.n_chunks; k++) s += p.ws_part2[(bh * p.n_chunks + k) * kHeadDim + d];
  var[d] = s / static_cast<double>(p.N);
  taken[d] = false;
  __syncthreads();
  if (d == 0) {
    for (int f = 0; f < p.n_feat; f++) {
      int best = -1;
      for (int c = 0; c < kHeadDim; c++)
        if (!taken[c] && (best < 0 || var[c] > var[best])) best = c;
      taken[best] = true;
      feat[f] = best;
    }
    for (int i = 1; i < p.n_feat; i++)  // insertion sort, ascending
      for (int j = i; j > 0 && feat[j - 1] > feat[j]; j--) {
        const int tmp = feat[j];
        feat[j] = feat[j - 1];
        feat[j - 1] = tmp;
      }
    for (int f = 0; f < p.n_feat; f++) p.ws_featsel[bh * kMaxFeatures + f] = feat[f];
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

// 5. assignment of the chunk's tokens (thread i: tokens t0 + kTpt*i .. +kTpt-1). With sums: per
// cluster, the chunk's feature sums and count (wave butterflies, then the 4 waves in order).
// Final step (sums = 0): the chunk's count per cluster, the labels output and, for the scatter
// index, the count per cluster of each 256-token sub-chunk (threads 32 s .. 32 s + 31 hold the
// tokens of sub-chunk s of the chunk).
__global__ __launch_bounds__(256) void vc_step(ClusterParams p, int sums) {
  constexpr int kSubs = kChunk / kClusterSub;
  static_assert(kChunk % kClusterSub == 0 && kClusterSub % kTpt == 0, "sub-chunks of whole threads");
  __shared__ double cent[kMaxClusters * kMaxFeatures];
  __shared__ double wred[4][kMaxFeatures + 1];
  __shared__ int cnt_s[kMaxClusters];
  __shared__ int scnt_s[kSubs][kMaxClusters];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int K = p.n_clusters, F = p.n_feat;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < K * kMaxFeatures; i += 256) cent[i] = p.ws_cent[bh * kMaxClusters * kMaxFeatures + i];
  if (tid < kMaxClusters) cnt_s[tid] = 0;
  if (tid < kSubs * kMaxClusters) scnt_s[tid / kMaxClusters][tid % kMaxClusters] = 0;
  __syncthreads();
  const int64_t tb = c * kChunk + static_cast<int64_t>(tid) * kTpt;
  const float* fv = p.ws_feat + bh * p.N * F;
  // the thread's tokens' features, loaded once (zero beyond n_feat and past N)
  float fx[kTpt][kMaxFeatures];
#pragma unroll
  for (int k = 0; k < kTpt; k++)
#pragma unroll
    for (int f = 0; f < kMaxFeatures; f++) fx[k][f] = (tb + k < p.N && f < F) ? fv[(tb + k) * F + f] : 0.0f;
  int lab[kTpt];
#pragma unroll
  for (int k = 0; k < kTpt; k++) {
    const int64_t t = tb + k;
    lab[k] = -1;
    if (t >= p.N) continue;
    int best = 0;
    double bd = INFINITY;
    for (int cl = 0; cl < K; cl++) {
      double dist = 0.0;
#pragma unroll
      for (int f = 0; f < kMaxFeatures; f++) {
        if (f < F) {
          const double diff = static_cast<double>(fx[k][f]) - cent[cl * kMaxFeatures + f];
          dist += dmul_rounded(diff, diff);
        }
      }
      if (dist < bd) {
        bd = dist;
        best = cl;
      }
    }
    lab[k] = best;
    p.ws_labels[bh * p.N + t] = best;
  }
  if (!sums) {
    const int sub = tid / (kClusterSub / kTpt);
#pragma unroll
    for (int k = 0; k < kTpt; k++) {
      if (lab[k] < 0) continue;
      atomicAdd(&cnt_s[lab[k]], 1);  // integer counts: order-free
      if (p.labels) p.labels[bh * p.N + tb + k] = lab[k];
      if (p.ws_scount) {
        atomicAdd(&scnt_s[sub][lab[k]], 1);
        p.ws_lab8[bh * p.lab_stride + tb + k] = static_cast<uint8_t>(lab[k]);
      }
    }
    __syncthreads();
    if (tid < K) p.ws_ccount[(bh * p.n_chunks + c) * kMaxClusters + tid] = cnt_s[tid];
    if (p.ws_scount) {
      for (int i = tid; i < kSubs * K; i += 256) {
        const int cl = i / kSubs;
        const int64_t s = c * kSubs + i % kSubs;
        if (s < p.n_sub) p.ws_scount[(bh * kMaxClusters + cl) * p.n_sub + s] = scnt_s[i % kSubs][cl];
      }
    }
    return;
  }
  for (int cl = 0; cl < K; cl++) {
    double part[kMaxFeatures + 1];
#pragma unroll
    for (int f = 0; f <= kMaxFeatures; f++) part[f] = 0.0;
#pragma unroll
    for (int k = 0; k < kTpt; k++) {
      if (lab[k] != cl) continue;
#pragma unroll
      for (int f = 0; f < kMaxFeatures; f++) part[f] += static_cast<double>(fx[k][f]);
      part[kMaxFeatures] += 1.0;
    }
#pragma unroll
    for (int f = 0; f <= kMaxFeatures; f++) {
      if (f < F || f == kMaxFeatures) {
        double x = part[f];
        for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
        if (lane == 0) wred[wave][f == kMaxFeatures ? F : f] = x;
      }
    }
    __syncthreads();
    if (tid <= F) {
      const double tot = ((wred[0][tid] + wred[1][tid]) + wred[2][tid]) + wred[3][tid];
      p.ws_csum[((bh * p.n_chunks + c) * kMaxClusters + cl) * (kMaxFeatures + 1) + tid] = tot;
    }
    __syncthreads();
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
  for (int64_t k = 0; k < p.n_chunks; k++) {
    const double* row = p.ws_csum + ((bh * p.n_chunks + k) * kMaxClusters + cl) * (kMaxFeatures + 1);
    s += row[f];
    n += row[F];
  }
  if (n > 0.0) p.ws_cent[(bh * kMaxClusters + cl) * kMaxFeatures + f] = s / n;
}

// 7. stable scatter: positions ordered by (cluster, token). Base of (cluster, chunk) = tokens of
// lower clusters + tokens of this cluster in earlier chunks; inside the chunk, thread i's
// contiguous tokens come after those of threads < i.
__global__ __launch_bounds__(256) void vc_scatter(ClusterParams p) {
  __shared__ int base[kMaxClusters];
  __shared__ int scan[kMaxClusters][257];
  const int64_t c = blockIdx.x, bh = blockIdx.y;
  const int K = p.n_clusters, tid = threadIdx.x;
  if (tid < K) {
    int before = 0;
    for (int cl = 0; cl < tid; cl++)
      for (int64_t k = 0; k < p.n_chunks; k++) before += p.ws_ccount[(bh * p.n_chunks + k) * kMaxClusters + cl];
    for (int64_t k = 0; k < c; k++) before += p.ws_ccount[(bh * p.n_chunks + k) * kMaxClusters + tid];
    base[tid] = before;
  }
  const int64_t tb = c * kChunk + static_cast<int64_t>(tid) * kTpt;
  int lab[kTpt];
  int my[kMaxClusters];
  for (int cl = 0; cl < K; cl++) my[cl] = 0;
#pragma unroll
  for (int k = 0; k < kTpt; k++) {
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
  for (int k = 0; k < kTpt; k++) {
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
  const dim3 g(nc, bh);
  hipLaunchKernelGGL(vc_colsum, g, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(vc_sqdev, g, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(vc_select, dim3(bh), dim3(kHeadDim), 0, stream, p);
  hipLaunchKernelGGL(vc_gather, g, dim3(256), 0, stream, p);
  for (int it = 0; it < p.iters; it++) {
    hipLaunchKernelGGL(vc_step, g, dim3(256), 0, stream, p, 1);
    hipLaunchKernelGGL(vc_update, dim3(bh), dim3(512), 0, stream, p);
  }
  hipLaunchKernelGGL(vc_step, g, dim3(256), 0, stream, p, 0);
  if (p.ws_scount) hipLaunchKernelGGL(vc_index, dim3(static_cast<unsigned>(p.n_clusters), bh), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(vc_scatter, g, dim3(256), 0, stream, p);
  return hipGetLastError();
}

int64_t cluster_chunks(int64_t N) { return (N + kChunk - 1) / kChunk; }

}  // namespace fp8attn
