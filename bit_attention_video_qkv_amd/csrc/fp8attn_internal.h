// Internal launch interfaces of libfp8attn (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8attn {

struct QuantParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm_q;
  const int32_t* perm_kv;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8t;
  float* q_scale;
  float* k_scale;
  float* v_scale;
  uint16_t* v_mean;
  float* ws_partial;  // [B*H, NB128, 128] per-block channel amax
  float* ws_inv;      // [B*H, 128] 448 / channel amax
  // sequence-mean smoothing (0: off, 1: K, 2: K and V) and the V bias correction
  float* v_shift;     // [B*H, 128] output vector added to O, or null
  float* ws_bsum;     // [2, B*H, NB, 128] FP32 block sums (K, V; the V half is reused for the
                      // block sums of the V rounding error)
  int32_t* ws_cnt;    // [B*H, NB] valid rows per 64-row block
  float* ws_mean;     // [2, B*H, 128] sequence means of K and V
  int64_t B, H, Nsrc, N, N64, NB, NB128;
  int perm_kv_per_head;
  int vsmooth;
  int smoothing;
  int v_bias_correction;
  // V-Smooth preparation with the stable scatter fused into the V block statistics (sc_labels
  // non-null): the statistics kernel places the tokens of each 128-row block from the cluster
  // labels and the scatter index of the clustering and writes them to perm_out, which is then
  // perm_kv (per head) of the other kernels
  const uint8_t* sc_labels;  // [B*H, sc_lab_stride] cluster of each source token (a byte)
  const int32_t* sc_sbase;   // [B*H, kMaxClusters, sc_nsub + 1]
  const int32_t* sc_ctot;    // [B*H, kMaxClusters] tokens per cluster
  int32_t* perm_out;         // [B*H, N]
  int64_t sc_nsub, sc_lab_stride;
  int sc_clusters;
};

struct AttnParams {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const uint16_t* v_mean;   // V-Smooth block means (bf16) or null
  const float* v_shift;     // [B*H, 128] added to every output row before BF16, or null
  uint32_t* mu_op;          // V-Smooth: [B*H, ceil(NB128 / 4), 128] x 32 B mean operand records (workspace)
  uint16_t* out;            // bf16 [B, n_out, H, 128]
  const int32_t* out_rows;  // [N] or null
  unsigned long long* underflow;  // [B*H] or null
  const int32_t* tile_len;  // sparse descriptor (device) or null
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t N, N64, NB, NB128, n_out;
  int B, H;
  int tile_tokens;
  int n_qtiles;    // query tiles per (b, h)
  int total_work;  // B * H * n_qtiles
  float logit_scale;  // softmax_scale * log2(e)
  float log2S;
  int reverse;
  // split-KV (dense): splits pieces of split_blocks key blocks; each piece writes its normalised
  // output and log2-sum-exp, which split_merge combines. splits = 1: no split, o_part null.
  int splits;
  int64_t split_blocks;
  float* o_part;  // [splits, B*H, N, 128]; Sol: [B*H, N, 128], the summary route's output
  float* lse;     // [splits, B*H, N]; Sol: [B*H, N], the summary route's log2 weight
  // Sol routing: exact-block mask [B*H, NB, sol_words] of the exact route (the attention then
  // adds the summary contributions in its epilogue), or null; sol_gmax [B*H,
  // sol_groups, N64]: per row, the running max (log2 units) of the summary route scores over the
  // route groups of 64 KV blocks up to and including each group in KV order, which every exact
  // block of that group takes into its running max first
  const uint64_t* sol_mask;
  int64_t sol_words;
  const float* sol_gmax;
  int64_t sol_groups;
  // per-XCD work queues: eight counters (workspace) zeroed before each launch; variants without
  // V-Smooth or underflow counting take their work items from them
  uint32_t* work_ctr;
  int cus;  // compute units of the device (sizes the persistent grid)
};

// Sol routing preparation and summary route (fp8attn_sol.hip).
struct SolParams {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  float* ksum;       // [B*H, NB, 128] K summaries (FP32)
  uint16_t* vsumT;   // V summaries (bf16, B*H*NBp*128 values) in the summary PV's operand order
  uint8_t* kq8;      // [B*H, NBp, 128] quantised K summaries
  float* kq_scale;   // [B*H, NBg]
  double* mk;        // [B*H, 128] mean of the summaries
  double* Mk;        // [B*H, 128, 128] second moment of the summaries
  float* theta;      // [B*H, NB]
  uint64_t* mask;    // [B*H, NB, W]
  float* o_part;     // piece 1 of the merge buffers: [B*H, N, 128]
  float* lse;        // [B*H, N]
  float* gmax;       // [B*H, NBg, N64] running max of the summary scores over the groups (log2)
  int64_t N, N64, NB, NBg, NBp, W;
  int B, H;
  float softmax_scale;
  float log2S;
  double tau;
  int estimator;
  int sink_blocks;
  int reverse;       // KV order: groups are visited in it
};

// Summaries, quantised K summaries, moments, thresholds, then the route (mask + summary route).
hipError_t launch_sol(const SolParams& p, hipStream_t stream);

hipError_t launch_quantize(const QuantParams& p, hipStream_t stream);

// Diagnostics (fp8attn_diag.hip): the quantiser's E4M3 encoder on consecutive FP32 bit patterns,
// and one E4M3 matrix-core product per 32 x 32 x 64 tile.
hipError_t launch_diag_e4m3_encode(uint32_t first, int64_t n_words, uint32_t* out, hipStream_t stream);
hipError_t launch_diag_e4m3_decode(const uint32_t* codes, int64_t n_words, float* out, hipStream_t stream);
hipError_t launch_diag_mfma_e4m3(const uint8_t* a, const uint8_t* bt, float* c, int32_t n_tiles,
                                 hipStream_t stream);

constexpr int kMaxClusters = 32;  // V-Smooth clustering limits (registers and LDS of the kernel)
constexpr int kMaxFeatures = 16;

struct ClusterParams {
  const uint16_t* v;   // bf16 [B, N, H, 128]
  int32_t* perm;       // [B, H, N]
  int32_t* labels;     // [B, H, N] or null
  float* ws_feat;      // [B*H, N, n_feat]
  int32_t* ws_labels;  // [B*H, N]
  double* ws_part1;    // [B*H, n_chunks, 128] channel sums per chunk
  double* ws_part2;    // [B*H, n_chunks, 128] centred sums of squares per chunk
  int32_t* ws_featsel; // [B*H, kMaxFeatures]
  double* ws_cent;     // [B*H, kMaxClusters, kMaxFeatures]
  double* ws_csum;     // [B*H, n_schunks, kMaxClusters, kMaxFeatures + 1] (sums, count at n_feat)
  int32_t* ws_ccount;  // [B*H, n_schunks, kMaxClusters]
  // scatter index: the tokens of each cluster per 256-token sub-chunk (final assignment), their
  // exclusive prefix over the sub-chunks and their total; and, for the preparation that fuses
  // the stable scatter into the V block statistics, the labels as bytes (else null, and
  // vc_scatter writes perm)
  uint8_t* ws_lab8;    // [B*H, lab_stride] (lab_stride = N rounded up to 16) or null
  int32_t* ws_scount;  // [B*H, kMaxClusters, n_sub]
  int32_t* ws_sbase;   // [B*H, kMaxClusters, n_sub + 1]
  int32_t* ws_ctot;    // [B*H, kMaxClusters]
  int64_t N, n_chunks, n_schunks, n_sub, lab_stride;
  int B, H;
  int n_clusters, n_feat, iters;
};

constexpr int kClusterSub = 256;  // tokens per sub-chunk of the scatter index

int64_t cluster_chunks(int64_t N);       // token chunks of the channel statistics and the gather
int64_t cluster_step_chunks(int64_t N);  // token chunks of the assignment and the scatter
hipError_t launch_cluster(const ClusterParams& p, hipStream_t stream);

enum AttnVariant : int {
  kVarExpCast = 1,
  kVarVSmooth = 2,
  kVarSparse = 4,
  kVarStats = 8,
  kVarSol = 16,
};

// Launches the attention forward for the variant bits; p.n_qtiles / p.total_work are filled in.
hipError_t launch_attention(AttnParams p, int variant, hipStream_t stream);

}  // namespace fp8attn
