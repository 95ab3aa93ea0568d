// QKV preparation kernels (HBM-bound).
//
// TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", section
// "面向注意力的 FP8 Preparation": one E4M3 scale per (batch, head, 64-token Q/K block),
// s = max|X_block| / 448; one scale per (batch, head, channel) for V over all tokens; V is
// written token-contiguous so the PV contraction reads keys contiguously. VC-Attention article
// section 二: V-Smooth subtracts the mean of each 128-row block of the (cluster-permuted) V and
// quantises the residual; the mean is kept as one 16-bit vector per block. TeleFuser blog,
// MiniMax-H3 section: sequence-mean smoothing subtracts the per-head FP32 token mean from K
// (and V), and the attention adds the V mean back (optionally minus the mean rounding error of
// the quantised V, the bias compensation).
//
// Launch plan on the caller's stream (all row loads are 256-byte rows of the source layout
// [B, N_src, H, 128], so every gather stays coalesced):
//   0. (smoothing)   seq_block_sums grid (NB, B*H, 1 or 2): FP32 column sums of each 64-row
//                    block of K (and V), rows in ascending order; seq_tree_pass (LDS passes of
//                    the pairwise tree over the block sums) and seq_mean_final -> the means
//                    (and v_shift).
//   1. quant_qk      grid (NB, B*H, 2): amax of a 64-row Q or K block -> scale -> codes.
//   2. v_block_stats grid (NB128, B*H): per 128-row block, per channel: amax of V, or (V-Smooth)
//                    the block mean (exact FP64 column sums) and the residual amax.
//   3. v_finalize    grid (B*H, 4): channel amax over blocks -> v_scale and its inverse.
//   4. v_encode      grid (NB, B*H): codes of a 64-row block, transposed through LDS into
//                    [B, H, 128, N64]; with the bias correction also the FP32 column sums of
//                    the rounding error of the block's valid rows.
//   5. (bias correction) the same tree over the error sums -> v_shift = mean_V - mean error.
// V-Smooth preparation of a clustering step (VC-Attention article, section 四: the gather after
// the clustering fused with the block mean and the quantisation): v_block_stats runs first and
// performs the clustering's stable scatter itself (each 128-row block finds its tokens from the
// cluster labels), writing the permutation that the other kernels then gather through.
//
// Every sum of the smoothing path follows one fixed order (in-block ascending, then the tree),
// with explicitly rounded FP32 operations, so the means and v_shift are reproducible bit for bit.
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

// Source row indices of the layout positions pos[k] for head bh, or -1 (padding, beyond N, or
// an out-of-range permutation entry, which is treated as padding). The permutation entries are
// read at clamped indices (N >= 1) with no per-row branch, so that they load together.
template <int R>
__device__ __forceinline__ void gather_srcs(const int32_t* perm, int per_head, int64_t bh, int64_t N, int64_t Nsrc,
                                            const int64_t (&pos)[R], int32_t (&src)[R]) {
  if (perm == nullptr) {  // (uniform)
#pragma unroll
    for (int k = 0; k < R; k++) src[k] = pos[k] < N ? static_cast<int32_t>(pos[k]) : -1;
  } else {
    const int32_t* row = per_head ? perm + bh * N : perm;
    int32_t e[R];
#pragma unroll
    for (int k = 0; k < R; k++) e[k] = row[pos[k] < N ? pos[k] : N - 1];
#pragma unroll
    for (int k = 0; k < R; k++) src[k] = (pos[k] < N && e[k] >= 0 && e[k] < Nsrc) ? e[k] : -1;
  }
}

// Row s of head (b, h) starts at head_base(...) + s * H * 128 elements.
__device__ __forceinline__ const uint16_t* head_base(const uint16_t* base, int64_t b, int64_t h, int64_t Nsrc,
                                                     int64_t H) {
  return base + (b * Nsrc * H + h) * kHeadDim;
}

// The 16 bytes of channels 8 chunk .. + 7 of source row s of a head (hb = head_base, rstride =
// H * 128), zeros for s < 0. The load always issues (row 0, which exists since N_src >= 1,
// stands in for a padding row), so a thread's row loads are in flight together instead of each
// one waiting behind a branch.
__device__ __forceinline__ uint4 load_row16(const uint16_t* hb, int64_t rstride, int32_t s, int chunk) {
  // an opaque all-ones or zero mask: with a plain select the compiler turns the load back into
  // a predicated one, which it then waits for inside its branch
  uint32_t keep = s >= 0 ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(keep));
  const int64_t row = s >= 0 ? s : 0;
  const uint4 raw = *reinterpret_cast<const uint4*>(hb + row * rstride + chunk * 8);
  return make_uint4(raw.x & keep, raw.y & keep, raw.z & keep, raw.w & keep);
}

struct Bf16x8 {
  float v[8];
};

__device__ __forceinline__ Bf16x8 unpack8(const uint4 raw) {
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

// 0a. FP32 column sums of one 64-row block of K (z = 0) or V (z = 1), valid rows in ascending
// order. The block is staged through LDS as bf16 with coalesced 16-byte row loads (thread t:
// channels 8*(t%16)..+7 of rows t/16 + 16*p); thread d < 128 then sums channel d down the rows.
// The valid-row count is written by the K pass.
__global__ __launch_bounds__(256) void seq_block_sums(QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBlock][kHeadDim + 8];
  __shared__ uint32_t valid_bits[2];  // bit r: row r of the block is valid
  if (threadIdx.x < 2) valid_bits[threadIdx.x] = 0u;
  __syncthreads();
  const int64_t blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int z = blockIdx.z;
  const int64_t b = bh / p.H, h = bh % p.H;
  const uint16_t* src = z == 0 ? p.k : p.v;
  const int chunk = threadIdx.x & 15;
  const int row0 = threadIdx.x >> 4;
  int64_t pos[4];
  int32_t s[4];
  uint4 raw[4];
#pragma unroll
  for (int pass = 0; pass < 4; pass++) pos[pass] = blk * kBlock + row0 + 16 * pass;
  gather_srcs(p.perm_kv, p.perm_kv_per_head, bh, p.N, p.Nsrc, pos, s);
  const uint16_t* hb = head_base(src, b, h, p.Nsrc, p.H);
#pragma unroll
  for (int pass = 0; pass < 4; pass++) raw[pass] = load_row16(hb, p.H * kHeadDim, s[pass], chunk);
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int r = row0 + 16 * pass;
    *reinterpret_cast<uint4*>(&tile[r][chunk * 8]) = raw[pass];
    if (chunk == 0 && s[pass] >= 0) atomicOr(&valid_bits[r >> 5], 1u << (r & 31));
  }
  __syncthreads();
  const int d = threadIdx.x;
  if (d < kHeadDim) {
    const uint64_t vm = static_cast<uint64_t>(valid_bits[0]) | (static_cast<uint64_t>(valid_bits[1]) << 32);
    float acc = 0.0f;
#pragma unroll 16
    for (int r = 0; r < kBlock; r++) {
      const float sum = __fadd_rn(acc, bf16_to_f32(tile[r][d]));
      acc = ((vm >> r) & 1u) ? sum : acc;
    }
    const int cnt = __popcll(vm);
    p.ws_bsum[((z * p.B * p.H + bh) * p.NB + blk) * kHeadDim + d] = acc;
    if (z == 0 && d == 0) p.ws_cnt[bh * p.NB + blk] = cnt;
  }
}

// 0b / 5. Pairwise tree over the NB block sums of one (b, h) and channel. The tree is the
// level-by-level halving s[i] = s[2i] + s[2i+1] with an odd last element carried up; on block
// positions it reads: at level l, position k*2^(l+1) adds position k*2^(l+1) + 2^l when that is
// < NB. A node depends only on the blocks below it, so the tree is evaluated in passes: each
// pass reduces aligned groups of kTreeSpan consecutive nodes (spacing `stride` blocks) in LDS,
// in place, until one node is left; seq_mean_final then divides by the valid-row count.
constexpr int kTreeSpan = 256;
constexpr int kTreeCh = 32;

// grid (ceil(nodes / kTreeSpan), B*H*nz, 128 / kTreeCh); tensor z = z_first + y / (B*H).
__global__ __launch_bounds__(256) void seq_tree_pass(QuantParams p, int z_first, int64_t stride,
                                                      int64_t nodes) {
  __shared__ float s[kTreeSpan][kTreeCh + 1];
  const int64_t BH = p.B * p.H;
  const int64_t bh = blockIdx.y % BH;
  const int z = z_first + static_cast<int>(blockIdx.y / BH);
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kTreeSpan;
  const int c0 = blockIdx.z * kTreeCh;
  float* x = p.ws_bsum + (z * BH + bh) * p.NB * kHeadDim + c0;
  const int n_here = static_cast<int>(min<int64_t>(kTreeSpan, nodes - g0));
  for (int w = threadIdx.x; w < n_here * kTreeCh; w += 256) {
    const int i = w / kTreeCh, c = w % kTreeCh;
    s[i][c] = x[(g0 + i) * stride * kHeadDim + c];
  }
  __syncthreads();
  for (int st = 1; st < n_here; st *= 2) {
    for (int w = threadIdx.x; w < (kTreeSpan / (2 * st)) * kTreeCh; w += 256) {
      const int i = (w / kTreeCh) * 2 * st, c = w % kTreeCh;
      if (g0 + i + st < nodes) s[i][c] = __fadd_rn(s[i][c], s[i + st][c]);
    }
    __syncthreads();
  }
  if (threadIdx.x < kTreeCh) x[g0 * stride * kHeadDim + threadIdx.x] = s[0][threadIdx.x];
}

// mean = root / valid rows (0 when there are none). grid (B*H, nz), 128 threads.
//   pass 0: tensor y (0 K, 1 V) -> ws_mean; the V pass also writes v_shift = mean_V unless the
//           bias correction follows.
//   pass 1: the V half holds the error sums -> v_shift = mean_V - mean error.
__global__ __launch_bounds__(kHeadDim) void seq_mean_final(QuantParams p, int pass) {
  __shared__ int cnt_s[2];
  const int64_t bh = blockIdx.x;
  const int z = pass ? 1 : static_cast<int>(blockIdx.y);
  const int d = threadIdx.x;
  int c = 0;
  for (int64_t j = d; j < p.NB; j += kHeadDim) c += p.ws_cnt[bh * p.NB + j];
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((d & 63) == 0) cnt_s[d >> 6] = c;
  __syncthreads();
  const int count = cnt_s[0] + cnt_s[1];
  const float root = p.ws_bsum[(z * p.B * p.H + bh) * p.NB * kHeadDim + d];
  const float m = count > 0 ? __fdiv_rn(root, static_cast<float>(count)) : 0.0f;
  if (pass == 0) {
    p.ws_mean[(z * p.B * p.H + bh) * kHeadDim + d] = m;
    if (z == 1 && !p.v_bias_correction) p.v_shift[bh * kHeadDim + d] = m;
  } else {
    p.v_shift[bh * kHeadDim + d] = __fsub_rn(p.ws_mean[(p.B * p.H + bh) * kHeadDim + d], m);
  }
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
  // K' = fl32(K - mean_K) on valid rows when smoothing is on (padding rows stay zero)
  const bool shift = which == 1 && p.smoothing >= 1;
  float mk[8];
#pragma unroll
  for (int j = 0; j < 8; j++) mk[j] = shift ? p.ws_mean[bh * kHeadDim + chunk * 8 + j] : 0.0f;
  int64_t pos[4];
  int32_t s[4];
  uint4 raw[4];
#pragma unroll
  for (int pass = 0; pass < 4; pass++) pos[pass] = blk * kBlock + row0 + 16 * pass;
  gather_srcs(perm, per_head, bh, p.N, p.Nsrc, pos, s);
  const uint16_t* hb = head_base(src, b, h, p.Nsrc, p.H);
#pragma unroll
  for (int pass = 0; pass < 4; pass++) raw[pass] = load_row16(hb, p.H * kHeadDim, s[pass], chunk);
  Bf16x8 x[4];
  float amax = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    x[pass] = unpack8(raw[pass]);  // padding rows are zeros and stay zeros
    if (shift)
#pragma unroll
      for (int j = 0; j < 8; j++) x[pass].v[j] = s[pass] >= 0 ? __fsub_rn(x[pass].v[j], mk[j]) : 0.0f;
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

// The stable scatter of the V-Smooth clustering for one 128-row block j of the layout: layout
// position off[c] + r holds the token of rank r (in token order) among the tokens of cluster c,
// off[c] = the tokens of the clusters below c. For each cluster whose positions meet the block,
// the ranks ra .. rb - 1 it needs are found by scanning the byte labels from the 256-token
// sub-chunk that holds rank ra (sbase: the cluster's tokens before each sub-chunk), 4096 labels
// per step (16 per thread), ranks by a workgroup prefix count of the matches.
// src_s[r] receives the token of position 128 j + r, or -1 beyond N.
__device__ __forceinline__ void scatter_rows(const QuantParams& p, int64_t bh, int64_t j, int* src_s, int* off_s,
                                             int* wtot_s, int* s0_s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = j * kVBlock, i1 = min<int64_t>(p.N, i0 + kVBlock);
  const int K = p.sc_clusters;
  if (tid < kVBlock) src_s[tid] = -1;
  if (tid == 0) {
    int o = 0;
    for (int c = 0; c < K; c++) {
      off_s[c] = o;
      o += p.sc_ctot[bh * kMaxClusters + c];
    }
    off_s[K] = o;
  }
  __syncthreads();
  const uint8_t* lab = p.sc_labels + bh * p.sc_lab_stride;
  for (int c = 0; c < K; c++) {
    const int64_t oc = off_s[c];
    const int64_t lo = max<int64_t>(i0, oc), hi = min<int64_t>(i1, static_cast<int64_t>(off_s[c + 1]));
    if (lo >= hi) continue;  // (uniform: every thread reads the same offsets)
    const int ra = static_cast<int>(lo - oc), rb = static_cast<int>(hi - oc);
    const int32_t* sb = p.sc_sbase + (bh * kMaxClusters + c) * (p.sc_nsub + 1);
    __syncthreads();  // (s0_s and wtot_s of the previous cluster are read)
    if (tid == 0) *s0_s = static_cast<int>(p.sc_nsub);
    __syncthreads();
    for (int64_t s = tid; s < p.sc_nsub; s += 256)
      if (sb[s] <= ra && ra < sb[s + 1]) *s0_s = static_cast<int>(s);  // (one sub-chunk matches)
    __syncthreads();
    const int64_t s0 = *s0_s;
    int base = s0 < p.sc_nsub ? sb[s0] : rb;
    for (int64_t t0 = s0 * kClusterSub; base < rb && t0 < p.N; t0 += 16 * 256) {
      // this thread's 16 labels (the row is padded to 16 bytes, so a load that starts below N
      // stays inside it)
      const int64_t tb = t0 + 16 * tid;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (tb < p.N) w = *reinterpret_cast<const uint4*>(lab + tb);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      uint32_t mbits = 0;  // bit k: label tb + k is cluster c
#pragma unroll
      for (int k = 0; k < 16; k++)
        mbits |= (tb + k < p.N && ((ww[k >> 2] >> (8 * (k & 3))) & 0xFFu) == static_cast<uint32_t>(c)) ? 1u << k : 0u;
      const int cnt = __popc(mbits);
      int incl = cnt;  // inclusive prefix over the wave's lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        incl += lane >= d ? y : 0;
      }
      if (lane == 63) wtot_s[wave] = incl;
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        before += q < wave ? wtot_s[q] : 0;
        total += wtot_s[q];
      }
      int rank = base + before + incl - cnt;
      while (mbits) {
        const int k = __ffs(mbits) - 1;
        mbits &= mbits - 1u;
        if (rank >= ra && rank < rb) src_s[oc + rank - i0] = static_cast<int>(tb + k);
        rank++;
      }
      base += total;
      __syncthreads();  // (wtot_s is rewritten by the next step)
    }
  }
  __syncthreads();
}

// 2. Per 128-row block statistics of V. Thread t: channels 8*(t%16)..+7, rows t/16 + 16*p.
// (VS: V-Smooth; without it the FP64 column sums and their 16 KB of LDS are not needed, and
// eight workgroups fit a CU instead of six.) SCATTER: the block's tokens come from the fused
// stable scatter of the clustering, and the block writes them to perm_out.
template <bool VS, bool SCATTER>
__global__ __launch_bounds__(256) void v_block_stats(QuantParams p) {
  __shared__ double dsum[VS ? 16 : 1][kHeadDim];  // [row group][channel]
  __shared__ float fmax_[16][kHeadDim];
  __shared__ float mhat_s[kHeadDim];
  __shared__ int n_valid_s;
  __shared__ int src_s[SCATTER ? kVBlock : 1];
  __shared__ int off_s[SCATTER ? kMaxClusters + 1 : 1];
  __shared__ int wtot_s[4], s0_s;
  const int64_t j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int chunk = threadIdx.x & 15;
  const int rg = threadIdx.x >> 4;
  if (threadIdx.x == 0) n_valid_s = 0;
  if constexpr (SCATTER) {
    scatter_rows(p, bh, j, src_s, off_s, wtot_s, &s0_s);  // (ends with a barrier)
    const int64_t i = j * kVBlock + threadIdx.x;
    if (threadIdx.x < kVBlock && i < p.N) p.perm_out[bh * p.N + i] = src_s[threadIdx.x];
  } else {
    __syncthreads();
  }
  // V' = fl32(V - mean_V) on valid rows under smoothing 2 (never together with V-Smooth)
  const bool shift = p.smoothing == 2;
  float mv[8];
#pragma unroll
  for (int q = 0; q < 8; q++) mv[q] = shift ? p.ws_mean[(p.B * p.H + bh) * kHeadDim + chunk * 8 + q] : 0.0f;

  int32_t srow[8];
  uint4 raw[8];
  if constexpr (SCATTER) {
#pragma unroll
    for (int pass = 0; pass < 8; pass++) srow[pass] = src_s[rg + 16 * pass];
  } else {
    int64_t pos[8];
#pragma unroll
    for (int pass = 0; pass < 8; pass++) pos[pass] = j * kVBlock + rg + 16 * pass;
    gather_srcs(p.perm_kv, p.perm_kv_per_head, bh, p.N, p.Nsrc, pos, srow);
  }
  const uint16_t* vhb = head_base(p.v, b, h, p.Nsrc, p.H);
#pragma unroll
  for (int pass = 0; pass < 8; pass++) raw[pass] = load_row16(vhb, p.H * kHeadDim, srow[pass], chunk);
  float m[8];
#pragma unroll
  for (int q = 0; q < 8; q++) m[q] = 0.0f;
  if constexpr (VS) {
    bool valid[8];
    int my_valid = 0;  // rows counted once, by the chunk-0 thread of each row
#pragma unroll
    for (int pass = 0; pass < 8; pass++) {
      valid[pass] = srow[pass] >= 0;
      my_valid += (chunk == 0 && valid[pass]) ? 1 : 0;
    }
    // (no V shift: sequence-mean smoothing of V is rejected together with V-Smooth)
    Bf16x8 x[8];
#pragma unroll
    for (int pass = 0; pass < 8; pass++) x[pass] = unpack8(raw[pass]);  // padding rows are zeros
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
    // each row folded in as it arrives; padding rows are zeros and stay zeros
#pragma unroll
    for (int pass = 0; pass < 8; pass++) {
      const Bf16x8 x = unpack8(raw[pass]);
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const float v = shift ? (srow[pass] >= 0 ? __fsub_rn(x.v[q], mv[q]) : 0.0f) : x.v[q];
        m[q] = fmaxf(m[q], fabsf(v));
      }
    }
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
// grid (B*H, 4): 32 channels per workgroup, 32 threads per channel take every 32nd block (the
// maximum is exact in any order), then one thread per channel combines them.
__global__ __launch_bounds__(1024) void v_finalize(QuantParams p) {
  __shared__ float red[32][33];
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int d = blockIdx.y * 32 + c;
  float m = 0.0f;
#pragma unroll 4
  for (int64_t j = g; j < p.NB128; j += 32) m = fmaxf(m, p.ws_partial[(bh * p.NB128 + j) * kHeadDim + d]);
  red[g][c] = m;
  __syncthreads();
  if (g == 0) {
    for (int k = 1; k < 32; k++) m = fmaxf(m, red[k][c]);
    p.v_scale[bh * kHeadDim + d] = m > 0.0f ? __fdiv_rn(m, 448.0f) : 0.0f;
    p.ws_inv[bh * kHeadDim + d] = m > 0.0f ? __fdiv_rn(448.0f, m) : 0.0f;
  }
}

// fl32(a * b) that is never fused into a following add: hipcc contracts a*b - c into an FMA
// (its __fmul_rn is a plain operator and the fp-contract pragma is not honoured), and the
// rounding error of V' is defined with a separately rounded product.
__device__ __forceinline__ float mul_rounded(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

// 4. V codes of a 64-row block, transposed to token-contiguous rows of v8t. BIAS: also the FP32
// column sums (valid rows, ascending) of err = fl32(fl32(decode(code) * s_v) - V') into the V half
// of ws_bsum, for the bias-corrected v_shift; the input rows are kept in LDS as bf16 and the codes
// are read back from the transpose tile.
template <bool BIAS>
__global__ __launch_bounds__(256) void v_encode(QuantParams p) {
  // [channel][token quad]: word w of channel c holds the codes of tokens 4w .. 4w + 3 (byte u =
  // token 4w + u); an odd number of words per channel, so the 16 channel octets of a wave's
  // stores spread over the banks (two lanes per bank at most).
  // Rows per workgroup: 128, so that each channel's codes fill whole 128-byte lines of v8t; 64
  // with the bias correction, whose error sums are per 64-row block
  constexpr int kRows = BIAS ? kBlock : 2 * kBlock;
  constexpr int kTileWords = kRows / 4 + 1;
  __shared__ uint32_t tile[kHeadDim][kTileWords];
  const int64_t blk = blockIdx.x;  // block of kRows rows
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / p.H, h = bh % p.H;
  const int chunk = threadIdx.x & 15;  // channels 8 chunk .. + 7
  const int row0 = threadIdx.x >> 4;   // tokens 4 row0 .. + 3
  const bool shift = p.smoothing == 2;
  float inv[8], mhat[8];
#pragma unroll
  for (int q = 0; q < 8; q++) {
    inv[q] = p.ws_inv[bh * kHeadDim + chunk * 8 + q];
    mhat[q] = shift ? p.ws_mean[(p.B * p.H + bh) * kHeadDim + chunk * 8 + q] : 0.0f;
  }
  __shared__ __attribute__((aligned(16))) uint16_t vin_s[BIAS ? kBlock : 1][BIAS ? kHeadDim + 8 : 8];
  __shared__ uint32_t valid_bits[2];  // BIAS: bit t = row t of the block is valid
  if constexpr (BIAS) {
    if (threadIdx.x < 2) valid_bits[threadIdx.x] = 0u;
    __syncthreads();
  }
  // every row of the workgroup loaded before the first is used (then the V-Smooth mean)
  constexpr int kHalves = kRows / kBlock;
  int64_t pos[4 * kHalves];  // row 4 hh + pass
  int32_t srow[4 * kHalves];
  uint4 raw[4 * kHalves];
#pragma unroll
  for (int k = 0; k < 4 * kHalves; k++) pos[k] = blk * kRows + kBlock * (k >> 2) + 4 * row0 + (k & 3);
  gather_srcs(p.perm_kv, p.perm_kv_per_head, bh, p.N, p.Nsrc, pos, srow);
  const uint16_t* vhb = head_base(p.v, b, h, p.Nsrc, p.H);
#pragma unroll
  for (int k = 0; k < 4 * kHalves; k++) raw[k] = load_row16(vhb, p.H * kHeadDim, srow[k], chunk);
  // V-Smooth: the block mean of the workgroup's rows (one 128-row V block holds all of them)
  if (p.vsmooth) {
    const uint4 mraw = *reinterpret_cast<const uint4*>(p.v_mean + (bh * p.NB128 + blk * kRows / kVBlock) * kHeadDim + chunk * 8);
    const Bf16x8 m = unpack8(mraw);
#pragma unroll
    for (int q = 0; q < 8; q++) mhat[q] = m.v[q];
  }
#pragma unroll
  for (int hh = 0; hh < kHalves; hh++) {  // 64-row halves
  uint32_t lo4[4], hi4[4];  // per token: the codes of channels 0-3 and 4-7 of the octet
#pragma unroll
  for (int pass = 0; pass < 4; pass++) {
    const int t = kBlock * hh + 4 * row0 + pass;
    const bool valid = srow[4 * hh + pass] >= 0;
    if constexpr (BIAS) *reinterpret_cast<uint4*>(&vin_s[t][chunk * 8]) = raw[4 * hh + pass];
    const Bf16x8 x = unpack8(raw[4 * hh + pass]);
    float r[8], y[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
      r[q] = __fsub_rn(x.v[q], mhat[q]);
      y[q] = r[q] * inv[q];
    }
    // padding rows: code 0
    const uint32_t lo = valid ? e4m3x4(y[0], y[1], y[2], y[3]) : 0u;
    const uint32_t hi = valid ? e4m3x4(y[4], y[5], y[6], y[7]) : 0u;
    if constexpr (BIAS) {
      if (chunk == 0 && valid) atomicOr(&valid_bits[t >> 5], 1u << (t & 31));
    }
    lo4[pass] = lo;
    hi4[pass] = hi;
  }
  // 4 tokens x 4 channels byte transposes: first pairs of tokens interleaved per channel pair,
  // then the two pairs joined (perm(x, y, s): byte i = byte s_i of {y: 0-3, x: 4-7})
  auto transpose4 = [](const uint32_t (&r)[4], uint32_t (&c)[4]) {
    const uint32_t a01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // ch0 t0 t1, ch1 t0 t1
    const uint32_t b01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // ch2, ch3
    const uint32_t a23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
    const uint32_t b23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
    c[0] = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
    c[1] = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
    c[2] = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
    c[3] = __builtin_amdgcn_perm(b23, b01, 0x07060302u);
  };
  uint32_t clo[4], chi[4];
  transpose4(lo4, clo);
  transpose4(hi4, chi);
#pragma unroll
  for (int q = 0; q < 4; q++) {
    tile[chunk * 8 + q][kBlock / 4 * hh + row0] = clo[q];
    tile[chunk * 8 + 4 + q][kBlock / 4 * hh + row0] = chi[q];
  }
  }
  __syncthreads();
  // 16-token chunks of the channels' code rows: chunk q = 256 i + t is chunk q % kCh of channel
  // q / kCh, so the lanes of a wave write whole 128-byte lines of consecutive channels; with 128
  // rows the second half of the last block lies beyond N64 when NB is odd.
  constexpr int kCh = kRows / 16;  // chunks per channel
#pragma unroll
  for (int i = 0; i < kHeadDim * kCh / 256; i++) {
    const int q = 256 * i + threadIdx.x;
    const int d = q / kCh, k = q % kCh;
    const int64_t tok0 = blk * kRows + 16 * k;
    if (tok0 < p.N64) {
      const uint4 w = make_uint4(tile[d][4 * k], tile[d][4 * k + 1], tile[d][4 * k + 2], tile[d][4 * k + 3]);
      *reinterpret_cast<uint4*>(p.v8t + (bh * kHeadDim + d) * p.N64 + tok0) = w;
    }
  }
  if constexpr (BIAS) {
    // The rounding error of channel c, rows in ascending order (the bias correction exists only
    // with V smoothing, so V' = fl32(V - mean_V)): err = fl32(fl32(decode(code) * s_v) - V').
    if (threadIdx.x < kHeadDim) {
      const int c = threadIdx.x;
      const float mv = p.ws_mean[(p.B * p.H + bh) * kHeadDim + c];
      const float svc = p.v_scale[bh * kHeadDim + c];
      const uint64_t vm = static_cast<uint64_t>(valid_bits[0]) | (static_cast<uint64_t>(valid_bits[1]) << 32);
      float acc = 0.0f;
#pragma unroll 2
      for (int t4 = 0; t4 < kBlock; t4 += 4) {
        const uint32_t codes = tile[c][t4 >> 2];
        const f32x2 lo = e4m3x2_to_f32(codes, false), hi = e4m3x2_to_f32(codes, true);
        const float dec[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const float r = __fsub_rn(bf16_to_f32(vin_s[t4 + u][c]), mv);
          const float e = __fsub_rn(mul_rounded(dec[u], svc), r);
          const float sum = __fadd_rn(acc, e);
          acc = ((vm >> (t4 + u)) & 1u) ? sum : acc;
        }
      }
      p.ws_bsum[((p.B * p.H + bh) * p.NB + blk) * kHeadDim + c] = acc;
    }
  }
}

}  // namespace

// Tree passes and the final division for tensors z_first .. z_first + nz - 1.
static hipError_t launch_seq_means(const QuantParams& p, int z_first, int nz, int pass, hipStream_t stream) {
  const unsigned bhz = static_cast<unsigned>(p.B * p.H * nz);
  for (int64_t stride = 1, nodes = p.NB; nodes > 1; stride *= kTreeSpan, nodes = (nodes + kTreeSpan - 1) / kTreeSpan) {
    const dim3 grid(static_cast<unsigned>((nodes + kTreeSpan - 1) / kTreeSpan), bhz, kHeadDim / kTreeCh);
    hipLaunchKernelGGL(seq_tree_pass, grid, dim3(256), 0, stream, p, z_first, stride, nodes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(seq_mean_final, dim3(static_cast<unsigned>(p.B * p.H), static_cast<unsigned>(nz)),
                     dim3(kHeadDim), 0, stream, p, pass);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t stream) {
  const unsigned bh = static_cast<unsigned>(p.B * p.H);
  hipError_t e;
  const dim3 g_stats(static_cast<unsigned>(p.NB128), static_cast<unsigned>(p.B * p.H));
  if (p.sc_labels) {
    // fused stable scatter: the V statistics place the tokens and write the permutation, which
    // the other kernels then read as perm_kv
    hipLaunchKernelGGL((v_block_stats<true, true>), g_stats, dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.smoothing >= 1) {
    hipLaunchKernelGGL(seq_block_sums, dim3(static_cast<unsigned>(p.NB), bh, static_cast<unsigned>(p.smoothing)),
                       dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seq_means(p, 0, p.smoothing, 0, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 g_qk(static_cast<unsigned>(p.NB), static_cast<unsigned>(p.B * p.H), 2);
  hipLaunchKernelGGL(quant_qk, g_qk, dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!p.sc_labels) {
    if (p.vsmooth) hipLaunchKernelGGL((v_block_stats<true, false>), g_stats, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((v_block_stats<false, false>), g_stats, dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(v_finalize, dim3(static_cast<unsigned>(p.B * p.H), kHeadDim / 32), dim3(1024), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g_enc(static_cast<unsigned>(p.NB), bh);
  if (!p.v_bias_correction) {
    hipLaunchKernelGGL(v_encode<false>, dim3(static_cast<unsigned>(p.NB128), bh), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(v_encode<true>, g_enc, dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_seq_means(p, 1, 1, 1, stream);
}

}  // namespace fp8attn
