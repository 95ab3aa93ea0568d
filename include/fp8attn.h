/*
 * fp8attn.h — C ABI of libfp8attn, block-scaled FP8 (OCP E4M3) attention forward for MI355X
 * (gfx950).
 *
 * Operations and the passages that define them:
 *  - QKV preparation: TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", section
 *    "面向注意力的 FP8 Preparation" (equations s_q, s_k, s_v; V in token-contiguous storage);
 *    FPSAttention write-up, section 3.1 (Q/K per block, V per channel).
 *  - Attention mainloop: same blog, section "SM90 CuTe Mainloop" (E4M3 QK, online softmax,
 *    P cast to E4M3, E4M3 PV, V channel scale after all PV, BF16 out); "FP8 P-Cast Precision
 *    in Attention: Sink-Induced Collapse and the Optimality of S=2^8", sections 二/三 (KV
 *    iteration order, static P scale S).
 *  - Sliding-tile sparsity: FPSAttention write-up, sections 2.2 (neighbourhood W(u)) and 3.1.
 *  - V-Smooth and ExpCast: VC-Attention article, sections 二 and 三.
 *
 * Conventions shared by every entry point:
 *  - Device pointers are caller-owned device memory; no call allocates device memory or
 *    synchronises. The only global state is write-once per device and held in atomics: the
 *    result of the gfx950 check and the device address of fp8attn_forward_noalloc's scratch
 *    array (a module array the loader places on each device). Every entry point is
 *    thread-safe; calls of fp8attn_forward_noalloc that overlap on one device race on its
 *    scratch.
 *  - Work is enqueued on the caller's `stream`; outputs are valid when the stream reaches it.
 *  - Argument checks are synchronous and happen before any launch: on error nothing is
 *    enqueued and FP8ATTN_EINVAL / FP8ATTN_EUNSUPPORTED is returned. A failed launch returns
 *    FP8ATTN_EHIP. No call ever falls back to another implementation.
 *  - Shapes: B batch, N tokens in the layout order, H heads, D = 128 channels.
 *    NB = ceil(N / 64), N64 = 64 * NB, NB128 = ceil(N / 128).
 *  - Indices and offsets are 64-bit inside the library; B*H*N64*128 may exceed 2^31. The
 *    attention entry points (fp8attn_forward, fp8attn_forward_noalloc, fp8attn_sol_forward)
 *    address one head's channel-major V with 32-bit offsets and take N64 <= 2^25 (33,554,432
 *    tokens per head); a larger N returns FP8ATTN_EUNSUPPORTED.
 */
#ifndef FP8ATTN_H_
#define FP8ATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8attn_status {
  FP8ATTN_OK = 0,
  FP8ATTN_EINVAL = 1,        /* bad argument, shape or pointer */
  FP8ATTN_EUNSUPPORTED = 2,  /* valid but not supported (D != 128, device not gfx950, ...) */
  FP8ATTN_EHIP = 3,          /* a HIP call or launch failed */
  FP8ATTN_ESCRATCH = 4       /* fp8attn_forward_noalloc: the shape needs more than its scratch */
} fp8attn_status;

typedef enum fp8attn_kv_order {
  FP8ATTN_KV_FORWARD = 0,  /* key blocks visited 0 .. NB-1 */
  FP8ATTN_KV_REVERSE = 1   /* key blocks visited NB-1 .. 0 (sink block last) */
} fp8attn_kv_order;

/* Split-KV piece count for fp8attn_fwd_opts.kv_splits: 0 or 1 = one piece, 2..MAX = requested
 * count, AUTO = chosen from the shape and the device's compute-unit count. */
#define FP8ATTN_KV_SPLITS_AUTO (-1)
#define FP8ATTN_KV_SPLITS_MAX 16

typedef enum fp8attn_pcast {
  FP8ATTN_PCAST_RNE = 0,     /* P8 = E4M3_RNE(S * exp(x - m)) */
  FP8ATTN_PCAST_EXPCAST = 1  /* P8 byte = clamp(rint(8 z + 56 - 0.35), 0, 126), z = log2(S p) */
} fp8attn_pcast;

/* ------------------------------------------------------------------------------------------
 * fp8attn_quantize_qkv — QKV preparation.
 *
 * Q and K: one FP32 scale per (b, h, 64-token block) of the layout order,
 *   scale = fl32(amax / 448), code = E4M3_RNE(fl32(x * fl32(448 / amax))), amax = max |x|
 *   over the block's valid tokens; an all-zero block has scale 0 and codes 0.
 * V: one FP32 scale per (b, h, channel) over all valid tokens, same rule; codes written
 *   token-contiguous.
 * Gathers: perm_q[i] / perm_kv[...] is the source token of layout position i, or -1 for a
 *   padding position (zero vector, excluded from every amax and mean). K and V share perm_kv.
 * V-Smooth (vsmooth = 1): per 128-row block j of the permuted V', mu_j = mean of the valid
 *   rows (FP64 sum / count, rounded to FP32 then BF16 = v_mean), R = fl32(V' - mu_hat_j), and
 *   R is quantised per channel in place of V (v_scale then holds the residual scales).
 * Sequence-mean smoothing (TeleFuser blog "FP8 Sol-Attn", MiniMax-H3 section: subtract the
 *   per-head token mean of K and V in FP32 before quantisation, add the V mean back to the
 *   output): smoothing = 1 shifts K, 2 shifts K and V. mean = FP32 sum of each 64-row block's
 *   valid rows in ascending order, the block sums combined by a pairwise tree (level by level
 *   s[i] = s[2i] + s[2i+1], an odd last one carried), divided by the valid-row count (0 if none);
 *   K' = fl32(K - mean_K), V' = fl32(V - mean_V) are then quantised as above. smoothing = 2
 *   writes v_shift = mean_V, or with v_bias_correction = 1 (the section's compensation of the
 *   mean bias that rounding V' to E4M3 leaves) fl32(mean_V - e), e = the same mean taken over
 *   fl32(fl32(decode(code) * v_scale) - V'). Pass v_shift to fp8attn_forward.
 *
 * Arguments (device pointers unless noted):
 *   args      host pointer; B, N_src, N, H, D (= 128), perm_q [N] or NULL (identity; then
 *             N == N_src), perm_kv [N] (perm_kv_per_head = 0) or [B*H*N] (= 1) or NULL,
 *             vsmooth 0/1, smoothing 0/1/2 (2 excludes vsmooth), v_bias_correction 0/1
 *             (needs smoothing 2), v_shift FP32 [B, H, D] output, 16-byte aligned, required
 *             when smoothing = 2 (ignored otherwise).
 *   q, k, v   bf16 [B, N_src, H, D] (row-major, 16-byte aligned).
 *   q8, k8    E4M3 [B, H, N64, D]; rows >= N are written as code 0.
 *   v8t       E4M3 [B, H, D, N64]; columns >= N and padding positions are code 0.
 *   q_scale, k_scale   FP32 [B, H, NB].      v_scale   FP32 [B, H, D].
 *   v_mean    bf16 [B, H, NB128, D] (16-byte aligned) when vsmooth, else ignored (may be NULL).
 *   workspace device scratch of at least fp8attn_quantize_workspace_bytes(...) bytes,
 *             16-byte aligned; its contents are overwritten. The size covers every option.
 * Errors: EINVAL on null/misaligned pointers, non-positive sizes, N != N_src without
 *   perm_q, too-small workspace, smoothing outside 0..2, smoothing 2 with vsmooth, bias
 *   correction without smoothing 2; EUNSUPPORTED on D != 128 or a device other than gfx950.
 * ------------------------------------------------------------------------------------------ */
typedef struct fp8attn_quant_args {
  int32_t B, N_src, N, H, D;
  const int32_t* perm_q;
  const int32_t* perm_kv;
  int32_t perm_kv_per_head;
  int32_t vsmooth;
  int32_t smoothing;
  int32_t v_bias_correction;
  float* v_shift;
} fp8attn_quant_args;

size_t fp8attn_quantize_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D,
                                        int32_t vsmooth);

fp8attn_status fp8attn_quantize_qkv(const fp8attn_quant_args* args, const void* q,
                                    const void* k, const void* v, uint8_t* q8, uint8_t* k8,
                                    uint8_t* v8t, float* q_scale, float* k_scale,
                                    float* v_scale, uint16_t* v_mean, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Sliding-tile (STA) block-sparse descriptor (FPSAttention 2.2 / 3.1). The layout is
 * tile-major: n_tiles tiles of tile_tokens positions (a multiple of 64), the valid tokens of a
 * tile first, padding last. Query tile u attends to the key tiles
 * col_idx[row_ptr[u] .. row_ptr[u+1]), listed in ascending order. All arrays are DEVICE
 * pointers. N must equal n_tiles * tile_tokens.
 * ------------------------------------------------------------------------------------------ */
typedef struct fp8attn_sparse {
  int32_t tile_tokens;
  int32_t n_tiles;
  const int32_t* tile_len;  /* [n_tiles] valid tokens per tile, 1 .. tile_tokens */
  const int32_t* row_ptr;   /* [n_tiles + 1] */
  const int32_t* col_idx;   /* [row_ptr[n_tiles]] */
} fp8attn_sparse;

/* ------------------------------------------------------------------------------------------
 * fp8attn_vsmooth_cluster — V-Smooth token permutation (VC-Attention article, section 二, first
 * step: a light clustering of the value tokens on a few representative channels; tokens of a
 * cluster are made contiguous so that each 128-row block of the permuted V is homogeneous; the
 * permutation is computed once and reused across steps). Per (b, h):
 *   features = the n_feat channels of V with the largest variance over the head's tokens (ties
 *   to the lower channel), in ascending channel order; k-means with n_clusters centroids
 *   initialised at tokens floor((2c+1) N / (2 n_clusters)), iters Lloyd rounds and a final
 *   assignment, squared L2 distance in FP64 with ties to the lower cluster id (an empty cluster
 *   keeps its centroid); perm = the head's tokens stably sorted by cluster id. The result is
 *   deterministic. Pass perm as perm_kv (perm_kv_per_head = 1) to fp8attn_quantize_qkv.
 * Arguments (device pointers): v bf16 [B, N, H, D] (D = 128); perm int32 [B, H, N] (out);
 *   labels int32 [B, H, N] (out, cluster id of each source token) or NULL; workspace of at
 *   least fp8attn_vsmooth_cluster_workspace_bytes(...) bytes, 16-byte aligned, overwritten.
 * Errors: EINVAL on null/misaligned pointers, non-positive sizes, n_clusters outside [1, 32],
 *   n_feat outside [1, 16], iters outside [0, 1000], B*H > 65535 or a too-small workspace;
 *   EUNSUPPORTED on D != 128 or a device other than gfx950.
 * ------------------------------------------------------------------------------------------ */
size_t fp8attn_vsmooth_cluster_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D,
                                               int32_t n_feat);
fp8attn_status fp8attn_vsmooth_cluster(int32_t B, int32_t N, int32_t H, int32_t D, const void* v,
                                       int32_t n_clusters, int32_t n_feat, int32_t iters,
                                       int32_t* perm, int32_t* labels, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8attn_vsmooth_prepare — the V-Smooth preparation of a clustering step in one call, with the
 * clustering's stable scatter fused into the gather, block mean and residual quantisation
 * (VC-Attention article, section 四 and Fig. 7: the gather after the clustering, the block
 * mean, the scale and the quantisation fused, so the permuted tensors never pass through HBM;
 * section 二: the permutation is then reused across the steps of a window).
 * Computes exactly what fp8attn_vsmooth_cluster followed by fp8attn_quantize_qkv with
 * perm_kv = perm (perm_kv_per_head = 1) computes, bit for bit, but no kernel writes the
 * permutation before the quantisation: the V block statistics place each 128-row block's
 * tokens from the cluster labels (position off[c] + r holds the token of rank r among the
 * tokens of cluster c) and write perm as they go, for the other kernels and for the reuse
 * steps, which call fp8attn_quantize_qkv with it.
 * Arguments: args as for fp8attn_quantize_qkv with perm_kv = NULL, vsmooth = 1 and
 *   N == N_src (perm_q, smoothing 0/1 allowed); q, k, v, q8 .. v_mean as there; n_clusters,
 *   n_feat, iters, perm (out, int32 [B, H, N]) and labels (out or NULL) as for
 *   fp8attn_vsmooth_cluster; workspace of at least fp8attn_vsmooth_prepare_workspace_bytes(...)
 *   bytes, 16-byte aligned, overwritten.
 * Errors: those of the two calls it replaces; EINVAL also on perm_kv != NULL, vsmooth != 1 or
 *   N != N_src.
 * ------------------------------------------------------------------------------------------ */
size_t fp8attn_vsmooth_prepare_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D,
                                               int32_t n_feat);
fp8attn_status fp8attn_vsmooth_prepare(const fp8attn_quant_args* args, const void* q,
                                       const void* k, const void* v, int32_t n_clusters,
                                       int32_t n_feat, int32_t iters, int32_t* perm,
                                       int32_t* labels, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                       float* q_scale, float* k_scale, float* v_scale,
                                       uint16_t* v_mean, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8attn_sta_build — HOST helper that lays a raster latent grid (T, Hg, W) out in tiles
 * (tt, th, tw) (the grid is padded up to whole tiles; tiles numbered in raster order over the
 * tile grid; inside a tile valid tokens first in raster order, then padding) and lists, for
 * each tile, the tiles within Chebyshev radius (rt, rh, rw) in tile coordinates.
 * All pointers are HOST pointers: perm [n_tiles * tile] (source token or -1), tile_len
 * [n_tiles], row_ptr [n_tiles + 1], col_idx [capacity]; *nnz receives the entry count.
 * Returns EINVAL on bad sizes or when capacity < nnz (then *nnz still holds the need).
 * ------------------------------------------------------------------------------------------ */
fp8attn_status fp8attn_sta_build(int32_t T, int32_t Hg, int32_t W, int32_t tt, int32_t th,
                                 int32_t tw, int32_t rt, int32_t rh, int32_t rw, int32_t* perm,
                                 int32_t* tile_len, int32_t* row_ptr, int32_t* col_idx,
                                 int32_t capacity, int32_t* nnz);

/* ------------------------------------------------------------------------------------------
 * fp8attn_forward — attention forward on the output of fp8attn_quantize_qkv.
 *
 * Per query row, key blocks of 64 are visited in `kv_order` (dense) or along the sparse
 * row; per block: x = (q8 . k8) * s_q * s_k * softmax_scale; m' = max(m, max x);
 * p = exp(x - m'); l = exp(m - m') l + sum p; P8 = E4M3(S p) (or the ExpCast byte, whose
 * l increment is sum decode(P8) / S); acc = exp(m - m') acc + P8 . V8. Masked keys (>= N or
 * sparse padding) have p = 0. End: O = acc * v_scale / (S l), rounded to BF16.
 * V-Smooth (v_mean != NULL): the block's row sum r restores the mean, O = ((s_r / S) acc +
 * sum r mu_hat_j) / l, j the 128-row V block of each key block.
 * Accuracy: the E4M3 products are exact, but the matrix core sums each group of 8 products
 *   with an error below 2^-11 of the group's largest product; a logit therefore carries an
 *   error below 2^-11 * sum over its 16 groups of the largest |product|, times the scales.
 *   While that error stays below one eighth of a log2 unit (N(0,1)-like rows with logits up to
 *   about 2^8 in log2 units, |x s_q s_k softmax_scale| log2(e)), every P code is the exact
 *   evaluation's code or, at a rounding boundary, its neighbour, and the output agrees with an
 *   exact evaluation element by element. Beyond that range codes can move by several steps;
 *   the output stays finite (the ExpCast byte is clamped at 126, never 0x7F) and rows
 *   dominated by a few keys keep their weights, but element-wise agreement is not claimed.
 * Sequence-mean smoothing (opts->v_shift != NULL): O = acc * v_scale / (S l) + v_shift.
 * Split-KV (TeleFuser blog "FP8 Sol-Attn", long-sequence split-KV: pieces of the KV sequence run
 *   their own online softmax and are merged by log-sum-exp), dense only: with P pieces requested
 *   the key blocks are cut at absolute multiples of L = 2 * ceil(NB / (2 P)) blocks (whole
 *   128-row V blocks), giving ceil(NB / L) pieces; each piece runs the loop above in kv_order
 *   from its own m = -inf and yields o_s (the end formula) and lse_s = log2 of its weight; then
 *   O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max lse_s, + v_shift, BF16.
 *   The result differs from the one-piece result by P-code rounding only (each piece has its
 *   own running max).
 *
 * Arguments (device pointers unless noted):
 *   q8, k8, v8t, q_scale, k_scale, v_scale, v_mean   as written by fp8attn_quantize_qkv
 *             (v_mean non-NULL iff the V was quantised with vsmooth = 1).
 *   opts      host pointer:
 *     softmax_scale  > 0 (1/sqrt(128) for the usual attention);
 *     p_scale        S, 0 < S <= 448 (256 recommended);
 *     kv_order, pcast;
 *     sparse         host pointer to a descriptor (device arrays) or NULL for dense;
 *     out_rows       device int32 [N] destination row of each layout row (-1 = not written)
 *                    or NULL (identity); lets a gathered layout write O in source order;
 *     n_out          number of rows of `out` (N when out_rows is NULL);
 *     underflow      device uint64 [B*H] or NULL; when non-NULL the counts of keys whose
 *                    p > 0 but whose P code is 0 are ADDED to it (RNE mode only; slower);
 *     v_shift        device FP32 [B*H, D] (16-byte aligned) from sequence-mean smoothing, or
 *                    NULL; when given O += v_shift before the BF16 rounding. Not with V-Smooth;
 *     kv_splits      0/1 (no split), 2..FP8ATTN_KV_SPLITS_MAX, or FP8ATTN_KV_SPLITS_AUTO:
 *                    for N >= 16384, with rounds = B*H*ceil(N/128) / (2 * compute units):
 *                    rounds < 1 gives min(8, ceil(1 / rounds)) pieces; 1 <= rounds < 4 with
 *                    the last round at most 35% full gives 3; anything else one piece.
 *                    Dense only (sparse: 0, 1 or AUTO, which then means 1). The pieces'
 *                    partial outputs live in the workspace.
 *   out       bf16 [B, n_out, H, D]; rows a query does not own are left untouched.
 *   workspace device scratch of fp8attn_forward_workspace_bytes(B, N, H, D, vsmooth,
 *             kv_splits) bytes (at least 256), 16-byte aligned, overwritten. It holds the work
 *             queues of the call's workgroups (so two calls that run at the same time need two
 *             workspaces), V-Smooth's mean operands and, with more than one piece, FP32
 *             [pieces, B*H, N, D] partial outputs and [pieces, B*H, N] lse.
 * Errors: EINVAL on bad pointers/sizes, S outside (0, 448], sparse with V-Smooth, sparse
 *   N != n_tiles * tile_tokens or tile_tokens not a multiple of 64, ExpCast with underflow
 *   counting, kv_splits out of range or > 1 with sparse; EUNSUPPORTED on D != 128 or a device
 *   other than gfx950.
 * ------------------------------------------------------------------------------------------ */
typedef struct fp8attn_fwd_opts {
  float softmax_scale;
  float p_scale;
  fp8attn_kv_order kv_order;
  fp8attn_pcast pcast;
  const fp8attn_sparse* sparse;
  const int32_t* out_rows;
  int32_t n_out;
  unsigned long long* underflow;
  const float* v_shift;
  int32_t kv_splits;
} fp8attn_fwd_opts;

/* Workspace of fp8attn_forward for the shape, V-Smooth (0/1) and kv_splits (as in the options;
 * pass 1 for a sparse call): at least 256 bytes; 0 when an argument is invalid. */
size_t fp8attn_forward_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D,
                                       int32_t vsmooth, int32_t kv_splits);

fp8attn_status fp8attn_forward(int32_t B, int32_t N, int32_t H, int32_t D, const uint8_t* q8,
                               const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                               const float* k_scale, const float* v_scale,
                               const uint16_t* v_mean, const fp8attn_fwd_opts* opts,
                               void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8attn_forward_noalloc — fp8attn_forward without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). It computes exactly what fp8attn_forward computes, with the same
 * kernels; its scratch (the work-queue counters and, with V-Smooth, the mean operand records)
 * lives in a static device array of FP8ATTN_NOALLOC_SCRATCH_BYTES that each device holds until
 * the process ends. The call allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine. Every call on a device shares that device's array, and its counters are cleared by a
 * kernel at the start of each call; calls that overlap on one device (two streams, two threads)
 * race on it and must be serialised by the caller.
 * Errors: those of fp8attn_forward; FP8ATTN_ESCRATCH when the call would need more scratch than
 *   the array holds (fp8attn_forward_workspace_bytes above FP8ATTN_NOALLOC_SCRATCH_BYTES, e.g.
 *   any split-KV with more than one piece at realistic sizes, or V-Smooth beyond
 *   B*H*ceil(N/512) = 8191 groups of mean records of 4 KB); nothing is enqueued then.
 * ------------------------------------------------------------------------------------------ */
#define FP8ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

fp8attn_status fp8attn_forward_noalloc(int32_t B, int32_t N, int32_t H, int32_t D,
                                       const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                       const float* q_scale, const float* k_scale,
                                       const float* v_scale, const uint16_t* v_mean,
                                       const fp8attn_fwd_opts* opts, void* out,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8attn_sol_forward — Sol routing attention (TeleFuser blog "FP8 Sol-Attn", sections "Sol
 * Routing" and "SM90 CuTe Mainloop") on the output of fp8attn_quantize_qkv (layout order, no
 * V-Smooth, no gathers needed). 64-token Q and KV blocks (NB = ceil(N / 64)):
 *   summaries   kbar_j = fl32(fl32(sum_t decode(K8) * s_k,j) / n_j), vbar_j likewise with the
 *               V channel scales, rounded to BF16 (n_j valid keys of block j);
 *   route keys  the K summaries quantised like K per group of 64 summaries (amax / 448);
 *   threshold   per Q block u: theta_u = mu + tau * sigma, the mean and standard deviation of
 *               the block's route scores over all (valid query, KV block) pairs from second
 *               moments: mu = ss qbar . m, E2 = ss^2 sum_de Mq[d,e] Mk[d,e] (estimator 1, exact)
 *               or ss^2 sum_d Mq[d,d] Mk[d,d] (estimator 0, diag), sigma^2 = E2 - mu^2; m, Mk:
 *               mean and second moment of the K summaries, Mq: the block's query second moment;
 *   route       r_ij = (q8_i . kq8_j) s_q s_kq softmax_scale on the matrix cores; KV block j is
 *               exact for Q block u if j < sink_blocks or some valid query of u has r_ij >=
 *               theta_u; decisions within the matrix cores' rounding of theta may go either way;
 *   one state   both routes update one running max, row sum and accumulator ("SM90 CuTe
 *               Mainloop", unified online-softmax merge). The KV blocks are taken in route
 *               groups of 64 (groups in kv_order); in a group its summary blocks come first: each
 *               counts as n_j copies of (kbar_j, vbar_j) scored by r_ij, m' = max(m, r_ij), row
 *               sum and accumulator gain n_j exp(r_ij - m') and n_j exp(r_ij - m') vbar_j (on the
 *               BF16 matrix cores); then the group's exact blocks take the fp8attn_forward step
 *               against that running max, in kv_order;
 *   output      acc / l + v_shift, BF16.
 * Arguments (device pointers unless noted):
 *   q8 .. v_scale  as written by fp8attn_quantize_qkv (vsmooth = 0).
 *   opts       host pointer: softmax_scale > 0, p_scale in (0, 448], kv_order, pcast, tau
 *              (finite), estimator 0/1, sink_blocks >= 0, v_shift (FP32 [B*H, D], 16-byte
 *              aligned) or NULL.
 *   out        bf16 [B, N, H, D].
 *   route_mask uint64 [B*H, NB, W] (W = ceil(NB / 64); bit j % 64 of word j / 64 = KV block j
 *              exact for Q block u) or NULL.
 *   workspace  fp8attn_sol_workspace_bytes(B, N, H, D) bytes, 16-byte aligned, overwritten. It
 *              holds the summaries, thresholds, the summary contributions and, per row and route
 *              group, the running maximum of the summary scores, and the work queues of the exact
 *              route (two calls that run at the same time need two workspaces).
 * Errors: EINVAL on bad pointers/sizes/options; EUNSUPPORTED on D != 128 or a device other
 *   than gfx950.
 * ------------------------------------------------------------------------------------------ */
typedef struct fp8attn_sol_opts {
  float softmax_scale;
  float p_scale;
  fp8attn_kv_order kv_order;
  fp8attn_pcast pcast;
  float tau;
  int32_t estimator;
  int32_t sink_blocks;
  const float* v_shift;
} fp8attn_sol_opts;

size_t fp8attn_sol_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D);

fp8attn_status fp8attn_sol_forward(int32_t B, int32_t N, int32_t H, int32_t D, const uint8_t* q8,
                                   const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                                   const float* k_scale, const float* v_scale,
                                   const fp8attn_sol_opts* opts, void* out, uint64_t* route_mask,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Diagnostics: the device arithmetic the parity contract rests on, run exactly as the
 * production kernels run it, for tests that compare it with independent implementations.
 *
 * fp8attn_diag_e4m3_encode — the quantisation kernels' E4M3 encoder (round to nearest even onto
 *   the OCP E4M3 grid; TeleFuser blog "FP8 Sol-Attn", section "面向注意力的 FP8 Preparation",
 *   codes of x * (448 / amax)) applied to the FP32 values whose bit patterns are first_bits,
 *   first_bits + 1, ..., first_bits + n - 1: out[i] is the code of pattern first_bits + i.
 *   out: device uint8 [n], 4-byte aligned. The encoder is specified for |x| <= 448 * (1 + 2^-23),
 *   the range the quantiser feeds it; outside it the codes are whatever the hardware gives.
 *   Errors: EINVAL when n < 0, n is not a multiple of 4, out is null or misaligned, or the range
 *   runs past pattern 2^32 - 1; EUNSUPPORTED on a device other than gfx950.
 *
 * fp8attn_diag_e4m3_decode — the E4M3 decoders of the Sol preparation and the V bias
 *   correction (FPSAttention write-up, section 2.1: the dequantised value of a code is its OCP
 *   E4M3 value times its scale) applied to n codes: out[i] is code i decoded two codes per
 *   conversion, out[n + i] the same code decoded alone. codes: device uint8 [n], 4-byte aligned;
 *   out: device float [2 n], 16-byte aligned. The decoders are specified for the finite codes
 *   (all but 0x7F and 0xFF, which the encoders never write). Errors: EINVAL when n < 0, n is not
 *   a multiple of 4 or above 2^40, or a pointer is null or misaligned; EUNSUPPORTED on a device
 *   other than gfx950.
 *
 * fp8attn_diag_mfma_e4m3 — one matrix-core E4M3 product per tile, as the attention's QK and PV
 *   contractions compute it (TeleFuser blog, section "SM90 CuTe Mainloop": E4M3 operands, FP32
 *   accumulation): for t < n_tiles, C[t] = A[t] * B[t] with A[t] 32 x 64 E4M3 row-major
 *   (2048 bytes), B[t] given as its transpose Bt[t] 32 x 64 E4M3 row-major (row j = column j of
 *   B), C[t] 32 x 32 FP32 row-major, accumulated from zero. Device pointers; a and bt 16-byte
 *   aligned, c 4-byte aligned. Errors: EINVAL on n_tiles < 0 or bad pointers; EUNSUPPORTED on a
 *   device other than gfx950.
 * ------------------------------------------------------------------------------------------ */
fp8attn_status fp8attn_diag_e4m3_encode(uint32_t first_bits, int64_t n, uint8_t* out,
                                        hipStream_t stream);
fp8attn_status fp8attn_diag_e4m3_decode(const uint8_t* codes, int64_t n, float* out,
                                        hipStream_t stream);
fp8attn_status fp8attn_diag_mfma_e4m3(const uint8_t* a, const uint8_t* bt, float* c,
                                      int32_t n_tiles, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* fp8attn_status_string(fp8attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* FP8ATTN_H_ */
