// C ABI of libfp8attn: argument validation, workspace carving and kernel launches.
// The operations are specified in include/fp8attn.h next to each declaration.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "fp8attn.h"
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace {

using fp8attn::kHeadDim;

constexpr size_t kAlign = 256;
// Forward workspace head: the eight per-XCD work-queue counters, padded to kAlign.
constexpr size_t kQueueBytes = 256;
// The attention kernels copy a head's channel-major V tile rows (128 rows of N64 bytes) with
// 32-bit offsets from a per-block base: 127 * N64 + 48 must stay below 2^32.
constexpr int64_t kMaxAttnTokens = int64_t{1} << 25;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
// V-Smooth mean operand records: 32 bytes per channel for each group of four 128-row V blocks
size_t mean_record_bytes(size_t bh, int64_t N) { return bh * cdiv(cdiv(N, 128), 4) * kHeadDim * 32; }

// Per-device result of the gfx950 check (0 unknown, 1 gfx950, 2 other). Written once per device.
std::atomic<int> g_arch_ok[64];

fp8attn_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8ATTN_EHIP;
  if (dev < 0 || dev >= 64) return FP8ATTN_EUNSUPPORTED;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8ATTN_EHIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? FP8ATTN_OK : FP8ATTN_EUNSUPPORTED;
}

fp8attn_status from_hip(hipError_t e) { return e == hipSuccess ? FP8ATTN_OK : FP8ATTN_EHIP; }

// Scratch of fp8attn_forward_noalloc: a file-scope device array (each device holds its own copy
// from module load until the process ends). Host code never passes the array's name to a
// kernel: its device address is looked up once per device, with that device current, and only
// that address is used.
static __device__ __align__(256) uint8_t scratch[FP8ATTN_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_addr[64];

fp8attn_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8ATTN_EHIP;
  if (dev < 0 || dev >= 64) return FP8ATTN_EUNSUPPORTED;
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return FP8ATTN_EHIP;
    g_scratch_addr[dev].store(a, std::memory_order_release);  // (a racing first call stores the same)
  }
  *out = a;
  return FP8ATTN_OK;
}

bool valid_splits_arg(int32_t kv_splits) {
  return kv_splits == FP8ATTN_KV_SPLITS_AUTO || (kv_splits >= 0 && kv_splits <= FP8ATTN_KV_SPLITS_MAX);
}

// Compute units of the current device (cached per device; 256 when it cannot be queried).
std::atomic<int> g_cus[64];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
    g_cus[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

// Split-KV pieces for a dense forward: the key blocks are cut at multiples of
// L = 2 * ceil(NB / (2 * want)) blocks (whole 128-row V blocks); returns ceil(NB / L) and L, or 1
// and NB without a split. Auto (measured on MI355X; only sequences of at least 16384 tokens, as
// shorter ones lose more to each piece's prologue and the merge than they gain), with
// rounds = query tiles / (2 workgroups per CU x CUs):
//   rounds < 1                                   -> ceil(1 / rounds) pieces (at most 8);
//   1 <= rounds < 4, last round at most 35% full -> 3 pieces;
//   otherwise                                    -> 1.
int resolve_splits(int32_t B, int32_t N, int32_t H, int32_t kv_splits, int64_t* split_blocks) {
  const int64_t NB = cdiv(N, 64);
  int64_t want = kv_splits;
  if (kv_splits == FP8ATTN_KV_SPLITS_AUTO) {
    const int64_t base = static_cast<int64_t>(B) * H * cdiv(N, 128);
    const int64_t slots = 2 * static_cast<int64_t>(device_cus());
    const int64_t last = base % slots;  // workgroups of the last, partial round
    want = 1;
    if (NB >= 256) {
      if (base < slots) want = std::min<int64_t>(8, cdiv(slots, base));
      else if (base < 4 * slots && last > 0 && 20 * last <= 7 * slots) want = 3;
    }
  }
  if (want <= 1) {
    *split_blocks = NB;
    return 1;
  }
  const int64_t L = 2 * cdiv(NB, 2 * want);
  *split_blocks = L;
  return static_cast<int>(cdiv(NB, L));
}

}  // namespace

extern "C" {

const char* fp8attn_status_string(fp8attn_status s) {
  switch (s) {
    case FP8ATTN_OK: return "ok";
    case FP8ATTN_EINVAL: return "invalid argument";
    case FP8ATTN_EUNSUPPORTED: return "unsupported shape or device";
    case FP8ATTN_EHIP: return "HIP runtime error";
    case FP8ATTN_ESCRATCH: return "shape needs more scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

size_t fp8attn_quantize_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D, int32_t vsmooth) {
  (void)vsmooth;
  if (B < 1 || N < 1 || H < 1 || D != kHeadDim) return 0;
  const size_t bh = static_cast<size_t>(B) * H;
  // channel amax partials and inverse scales, then the smoothing sums, counts and means (the
  // size covers every option, so one workspace serves all calls of a shape)
  return round_up(bh * cdiv(N, 128) * kHeadDim * sizeof(float)) + round_up(bh * kHeadDim * sizeof(float)) +
         round_up(2 * bh * cdiv(N, 64) * kHeadDim * sizeof(float)) + round_up(bh * cdiv(N, 64) * sizeof(int32_t)) +
         round_up(2 * bh * kHeadDim * sizeof(float));
}

}  // extern "C"

namespace {

// Validates the quantisation arguments and fills the launch parameters (no launch).
fp8attn_status quant_setup(const fp8attn_quant_args* a, const void* q, const void* k, const void* v, uint8_t* q8,
                           uint8_t* k8, uint8_t* v8t, float* q_scale, float* k_scale, float* v_scale,
                           uint16_t* v_mean, void* workspace, size_t workspace_bytes, fp8attn::QuantParams* out) {
  if (!a) return FP8ATTN_EINVAL;
  if (a->B < 1 || a->N < 1 || a->H < 1 || a->N_src < 1 || a->D < 1) return FP8ATTN_EINVAL;
  if (a->D != kHeadDim) return FP8ATTN_EUNSUPPORTED;
  if (static_cast<int64_t>(a->B) * a->H > 65535) return FP8ATTN_EUNSUPPORTED;
  if (!a->perm_q && a->N != a->N_src) return FP8ATTN_EINVAL;
  if (!a->perm_kv && a->N != a->N_src) return FP8ATTN_EINVAL;
  if (a->perm_kv_per_head != 0 && a->perm_kv_per_head != 1) return FP8ATTN_EINVAL;
  if (a->vsmooth != 0 && a->vsmooth != 1) return FP8ATTN_EINVAL;
  if (a->smoothing < 0 || a->smoothing > 2 || (a->smoothing == 2 && a->vsmooth)) return FP8ATTN_EINVAL;
  if (a->v_bias_correction != 0 && a->v_bias_correction != 1) return FP8ATTN_EINVAL;
  if (a->v_bias_correction && a->smoothing != 2) return FP8ATTN_EINVAL;
  if (a->smoothing == 2 && (!a->v_shift || !aligned(a->v_shift, 16))) return FP8ATTN_EINVAL;
  const void* p16[] = {q, k, v, q8, k8, v8t, v_scale, workspace};
  for (const void* ptr : p16)
    if (!ptr || !aligned(ptr, 16)) return FP8ATTN_EINVAL;
  if (!q_scale || !k_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4)) return FP8ATTN_EINVAL;
  if ((a->perm_q && !aligned(a->perm_q, 4)) || (a->perm_kv && !aligned(a->perm_kv, 4))) return FP8ATTN_EINVAL;
  if (a->vsmooth && (!v_mean || !aligned(v_mean, 16))) return FP8ATTN_EINVAL;
  const size_t need = fp8attn_quantize_workspace_bytes(a->B, a->N, a->H, a->D, a->vsmooth);
  if (workspace_bytes < need) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;

  fp8attn::QuantParams& p = *out;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.perm_q = a->perm_q;
  p.perm_kv = a->perm_kv;
  p.q8 = q8;
  p.k8 = k8;
  p.v8t = v8t;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.v_mean = a->vsmooth ? v_mean : nullptr;
  p.B = a->B;
  p.H = a->H;
  p.Nsrc = a->N_src;
  p.N = a->N;
  p.NB = cdiv(a->N, 64);
  p.N64 = p.NB * 64;
  p.NB128 = cdiv(a->N, 128);
  p.perm_kv_per_head = a->perm_kv_per_head;
  p.vsmooth = a->vsmooth;
  p.smoothing = a->smoothing;
  p.v_bias_correction = a->v_bias_correction;
  p.v_shift = a->smoothing == 2 ? a->v_shift : nullptr;
  const size_t bh = static_cast<size_t>(a->B) * a->H;
  char* ws = static_cast<char*>(workspace);
  p.ws_partial = reinterpret_cast<float*>(ws);
  ws += round_up(bh * p.NB128 * kHeadDim * sizeof(float));
  p.ws_inv = reinterpret_cast<float*>(ws);
  ws += round_up(bh * kHeadDim * sizeof(float));
  p.ws_bsum = reinterpret_cast<float*>(ws);
  ws += round_up(2 * bh * p.NB * kHeadDim * sizeof(float));
  p.ws_cnt = reinterpret_cast<int32_t*>(ws);
  ws += round_up(bh * p.NB * sizeof(int32_t));
  p.ws_mean = reinterpret_cast<float*>(ws);
  return FP8ATTN_OK;
}

}  // namespace

extern "C" {

fp8attn_status fp8attn_quantize_qkv(const fp8attn_quant_args* a, const void* q, const void* k,
                                    const void* v, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                    float* q_scale, float* k_scale, float* v_scale,
                                    uint16_t* v_mean, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  fp8attn::QuantParams p;
  const fp8attn_status st = quant_setup(a, q, k, v, q8, k8, v8t, q_scale, k_scale, v_scale, v_mean, workspace,
                                        workspace_bytes, &p);
  if (st != FP8ATTN_OK) return st;
  return from_hip(fp8attn::launch_quantize(p, stream));
}

size_t fp8attn_forward_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D, int32_t vsmooth,
                                       int32_t kv_splits) {
  if (B < 1 || N < 1 || H < 1 || D != kHeadDim || !valid_splits_arg(kv_splits)) return 0;
  const size_t bh = static_cast<size_t>(B) * H;
  size_t n = kQueueBytes;                                                   // work queues
  if (vsmooth) n += round_up(mean_record_bytes(bh, N));                   // mean operand records
  int64_t split_blocks = 0;
  const int splits = resolve_splits(B, N, H, kv_splits, &split_blocks);
  if (splits > 1)
    n += round_up(splits * bh * N * kHeadDim * sizeof(float)) + round_up(splits * bh * N * sizeof(float));
  return n;
}

fp8attn_status fp8attn_forward(int32_t B, int32_t N, int32_t H, int32_t D, const uint8_t* q8,
                               const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                               const float* k_scale, const float* v_scale,
                               const uint16_t* v_mean, const fp8attn_fwd_opts* o, void* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!o || B < 1 || N < 1 || H < 1 || D < 1) return FP8ATTN_EINVAL;
  if (D != kHeadDim) return FP8ATTN_EUNSUPPORTED;
  const int64_t total_bh = static_cast<int64_t>(B) * H;
  if (total_bh > 65535 || cdiv(N, 64) * 64 > kMaxAttnTokens) return FP8ATTN_EUNSUPPORTED;
  const void* p16[] = {q8, k8, v8t, v_scale};
  for (const void* ptr : p16)
    if (!ptr || !aligned(ptr, 16)) return FP8ATTN_EINVAL;
  if (!q_scale || !k_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4)) return FP8ATTN_EINVAL;
  if (!out || !aligned(out, 16)) return FP8ATTN_EINVAL;
  if (!(o->softmax_scale > 0.0f) || !isfinite(o->softmax_scale)) return FP8ATTN_EINVAL;
  if (!(o->p_scale > 0.0f) || !(o->p_scale <= 448.0f)) return FP8ATTN_EINVAL;
  if (o->kv_order != FP8ATTN_KV_FORWARD && o->kv_order != FP8ATTN_KV_REVERSE) return FP8ATTN_EINVAL;
  if (o->pcast != FP8ATTN_PCAST_RNE && o->pcast != FP8ATTN_PCAST_EXPCAST) return FP8ATTN_EINVAL;
  const bool vsmooth = v_mean != nullptr;
  const bool sparse = o->sparse != nullptr;
  if (vsmooth && (sparse || !aligned(v_mean, 16))) return FP8ATTN_EINVAL;
  if (o->underflow && (o->pcast != FP8ATTN_PCAST_RNE || !aligned(o->underflow, 8))) return FP8ATTN_EINVAL;
  if (o->v_shift && (vsmooth || !aligned(o->v_shift, 16))) return FP8ATTN_EINVAL;
  if (o->out_rows ? (o->n_out < 1 || !aligned(o->out_rows, 4)) : (o->n_out != N)) return FP8ATTN_EINVAL;
  if (sparse) {
    const fp8attn_sparse* s = o->sparse;
    if (s->tile_tokens <= 0 || s->tile_tokens % 64 != 0 || s->n_tiles < 1) return FP8ATTN_EINVAL;
    if (static_cast<int64_t>(s->tile_tokens) * s->n_tiles != N) return FP8ATTN_EINVAL;
    if (!s->tile_len || !s->row_ptr || !s->col_idx) return FP8ATTN_EINVAL;
  }
  if (!valid_splits_arg(o->kv_splits)) return FP8ATTN_EINVAL;
  if (sparse && o->kv_splits > 1) return FP8ATTN_EINVAL;
  int64_t split_blocks = 0;
  const int splits = sparse ? 1 : resolve_splits(B, N, H, o->kv_splits, &split_blocks);
  if (total_bh * cdiv(N, 64) * splits > INT32_MAX) return FP8ATTN_EUNSUPPORTED;
  const size_t need = fp8attn_forward_workspace_bytes(B, N, H, D, vsmooth ? 1 : 0, sparse ? 1 : o->kv_splits);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;

  fp8attn::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q8 = q8;
  p.k8 = k8;
  p.v8t = v8t;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.v_mean = v_mean;
  // workspace: [work queues][V-Smooth mean operand records][split-KV pieces]
  p.work_ctr = static_cast<uint32_t*>(workspace);
  p.cus = device_cus();
  p.mu_op = vsmooth ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kQueueBytes) : nullptr;
  p.splits = splits;
  p.split_blocks = splits > 1 ? split_blocks : cdiv(N, 64);
  if (splits > 1) {
    const size_t bh = static_cast<size_t>(total_bh);
    char* ws = static_cast<char*>(workspace) + kQueueBytes + (vsmooth ? round_up(mean_record_bytes(bh, N)) : 0);
    p.o_part = reinterpret_cast<float*>(ws);
    p.lse = reinterpret_cast<float*>(ws + round_up(splits * bh * N * kHeadDim * sizeof(float)));
  }
  p.out = static_cast<uint16_t*>(out);
  p.out_rows = o->out_rows;
  p.underflow = o->underflow;
  p.v_shift = o->v_shift;
  p.N = N;
  p.NB = cdiv(N, 64);
  p.N64 = p.NB * 64;
  p.NB128 = cdiv(N, 128);
  p.n_out = o->n_out;
  p.B = B;
  p.H = H;
  p.logit_scale = static_cast<float>(static_cast<double>(o->softmax_scale) * 1.4426950408889634);
  p.log2S = static_cast<float>(log2(static_cast<double>(o->p_scale)));
  p.reverse = o->kv_order == FP8ATTN_KV_REVERSE ? 1 : 0;
  int variant = 0;
  if (o->pcast == FP8ATTN_PCAST_EXPCAST) variant |= fp8attn::kVarExpCast;
  if (vsmooth) variant |= fp8attn::kVarVSmooth;
  if (o->underflow) variant |= fp8attn::kVarStats;
  if (sparse) {
    variant |= fp8attn::kVarSparse;
    p.tile_tokens = o->sparse->tile_tokens;
    p.tile_len = o->sparse->tile_len;
    p.row_ptr = o->sparse->row_ptr;
    p.col_idx = o->sparse->col_idx;
  }
  return from_hip(fp8attn::launch_attention(p, variant, stream));
}

namespace {

struct SolLayout {
  int64_t NB, NBg, NBp, W;
  size_t queue, ksum, vsumT, kq8, kq_scale, mk, Mk, theta, mask, o_part, lse, gmax, total;
};

SolLayout sol_layout(int32_t B, int32_t N, int32_t H) {
  SolLayout L;
  const size_t bh = static_cast<size_t>(B) * H;
  L.NB = cdiv(N, 64);
  L.NBg = cdiv(L.NB, 64);
  L.NBp = 64 * L.NBg;
  L.W = L.NBg;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes);
    return o;
  };
  L.queue = take(kQueueBytes);  // the exact route's work queues
  L.ksum = take(bh * L.NB * kHeadDim * sizeof(float));
  L.vsumT = take(bh * kHeadDim * L.NBp * sizeof(uint16_t));
  L.kq8 = take(bh * L.NBp * kHeadDim);
  L.kq_scale = take(bh * L.NBg * sizeof(float));
  L.mk = take(bh * kHeadDim * sizeof(double));
  L.Mk = take(bh * kHeadDim * kHeadDim * sizeof(double));
  L.theta = take(bh * L.NB * sizeof(float));
  L.mask = take(bh * L.NB * L.W * sizeof(uint64_t));
  L.o_part = take(bh * N * kHeadDim * sizeof(float));  // the summary route's normalised O
  L.lse = take(bh * N * sizeof(float));                  // and log2 of its weight
  L.gmax = take(bh * L.NBg * L.NB * 64 * sizeof(float));  // per row and group: summary max so far
  L.total = off;
  return L;
}

}  // namespace

size_t fp8attn_sol_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D) {
  if (B < 1 || N < 1 || H < 1 || D != kHeadDim) return 0;
  return sol_layout(B, N, H).total;
}

fp8attn_status fp8attn_sol_forward(int32_t B, int32_t N, int32_t H, int32_t D, const uint8_t* q8,
                                   const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                                   const float* k_scale, const float* v_scale,
                                   const fp8attn_sol_opts* o, void* out, uint64_t* route_mask,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!o || B < 1 || N < 1 || H < 1 || D < 1) return FP8ATTN_EINVAL;
  if (D != kHeadDim) return FP8ATTN_EUNSUPPORTED;
  const int64_t total_bh = static_cast<int64_t>(B) * H;
  if (total_bh > 65535 || total_bh * cdiv(N, 64) > INT32_MAX || cdiv(N, 64) * 64 > kMaxAttnTokens)
    return FP8ATTN_EUNSUPPORTED;
  const void* p16[] = {q8, k8, v8t, v_scale, out, workspace};
  for (const void* ptr : p16)
    if (!ptr || !aligned(ptr, 16)) return FP8ATTN_EINVAL;
  if (!q_scale || !k_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4)) return FP8ATTN_EINVAL;
  if (route_mask && !aligned(route_mask, 8)) return FP8ATTN_EINVAL;
  if (!(o->softmax_scale > 0.0f) || !isfinite(o->softmax_scale)) return FP8ATTN_EINVAL;
  if (!(o->p_scale > 0.0f) || !(o->p_scale <= 448.0f)) return FP8ATTN_EINVAL;
  if (o->kv_order != FP8ATTN_KV_FORWARD && o->kv_order != FP8ATTN_KV_REVERSE) return FP8ATTN_EINVAL;
  if (o->pcast != FP8ATTN_PCAST_RNE && o->pcast != FP8ATTN_PCAST_EXPCAST) return FP8ATTN_EINVAL;
  if (!isfinite(o->tau) || o->estimator < 0 || o->estimator > 1 || o->sink_blocks < 0) return FP8ATTN_EINVAL;
  if (o->v_shift && !aligned(o->v_shift, 16)) return FP8ATTN_EINVAL;
  const SolLayout L = sol_layout(B, N, H);
  if (workspace_bytes < L.total) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;

  char* ws = static_cast<char*>(workspace);
  uint64_t* mask = route_mask ? route_mask : reinterpret_cast<uint64_t*>(ws + L.mask);
  float* o_part = reinterpret_cast<float*>(ws + L.o_part);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  const double log2S = log2(static_cast<double>(o->p_scale));

  fp8attn::SolParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.q8 = q8;
  sp.k8 = k8;
  sp.v8t = v8t;
  sp.q_scale = q_scale;
  sp.k_scale = k_scale;
  sp.v_scale = v_scale;
  sp.ksum = reinterpret_cast<float*>(ws + L.ksum);
  sp.vsumT = reinterpret_cast<uint16_t*>(ws + L.vsumT);
  sp.kq8 = reinterpret_cast<uint8_t*>(ws + L.kq8);
  sp.kq_scale = reinterpret_cast<float*>(ws + L.kq_scale);
  sp.mk = reinterpret_cast<double*>(ws + L.mk);
  sp.Mk = reinterpret_cast<double*>(ws + L.Mk);
  sp.theta = reinterpret_cast<float*>(ws + L.theta);
  sp.mask = mask;
  sp.o_part = o_part;  // the summary route's piece, merged by the exact route's epilogue
  sp.lse = lse;
  sp.N = N;
  sp.NB = L.NB;
  sp.N64 = L.NB * 64;
  sp.NBg = L.NBg;
  sp.NBp = L.NBp;
  sp.W = L.W;
  sp.B = B;
  sp.H = H;
  sp.softmax_scale = o->softmax_scale;
  sp.log2S = static_cast<float>(log2S);
  sp.tau = o->tau;
  sp.estimator = o->estimator;
  sp.sink_blocks = o->sink_blocks;
  sp.reverse = o->kv_order == FP8ATTN_KV_REVERSE ? 1 : 0;
  sp.gmax = reinterpret_cast<float*>(ws + L.gmax);
  hipError_t e = fp8attn::launch_sol(sp, stream);
  if (e != hipSuccess) return FP8ATTN_EHIP;

  fp8attn::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q8 = q8;
  p.k8 = k8;
  p.v8t = v8t;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out = static_cast<uint16_t*>(out);
  p.v_shift = o->v_shift;
  p.N = N;
  p.NB = L.NB;
  p.N64 = L.NB * 64;
  p.NB128 = cdiv(N, 128);
  p.n_out = N;
  p.B = B;
  p.H = H;
  p.logit_scale = static_cast<float>(static_cast<double>(o->softmax_scale) * 1.4426950408889634);
  p.log2S = static_cast<float>(log2S);
  p.reverse = o->kv_order == FP8ATTN_KV_REVERSE ? 1 : 0;
  p.splits = 1;
  p.split_blocks = L.NB;
  p.o_part = o_part;
  p.lse = lse;
  p.sol_mask = mask;
  p.sol_words = L.W;
  p.sol_gmax = sp.gmax;
  p.sol_groups = L.NBg;
  p.work_ctr = reinterpret_cast<uint32_t*>(ws + L.queue);
  p.cus = device_cus();
  int variant = fp8attn::kVarSol;
  if (o->pcast == FP8ATTN_PCAST_EXPCAST) variant |= fp8attn::kVarExpCast;
  return from_hip(fp8attn::launch_attention(p, variant, stream));
}

// Host-side tile layout. Each token's tile follows from its raster coordinates; tokens are
// bucketed per tile in raster order (valid first), then padded with -1; the neighbour list of a
// tile is every tile whose tile coordinates are within the per-axis Chebyshev radius.
fp8attn_status fp8attn_sta_build(int32_t T, int32_t Hg, int32_t W, int32_t tt, int32_t th,
                                 int32_t tw, int32_t rt, int32_t rh, int32_t rw, int32_t* perm,
                                 int32_t* tile_len, int32_t* row_ptr, int32_t* col_idx,
                                 int32_t capacity, int32_t* nnz) {
  if (T < 1 || Hg < 1 || W < 1 || tt < 1 || th < 1 || tw < 1 || rt < 0 || rh < 0 || rw < 0)
    return FP8ATTN_EINVAL;
  if (!perm || !tile_len || !row_ptr || !nnz || capacity < 0 || (capacity > 0 && !col_idx))
    return FP8ATTN_EINVAL;
  const int64_t gt = cdiv(T, tt), gh = cdiv(Hg, th), gw = cdiv(W, tw);
  const int64_t n_tiles = gt * gh * gw, tile = static_cast<int64_t>(tt) * th * tw;
  if (n_tiles * tile > INT32_MAX) return FP8ATTN_EINVAL;
  for (int64_t u = 0; u < n_tiles; u++) tile_len[u] = 0;
  for (int64_t t = 0; t < T; t++)
    for (int64_t y = 0; y < Hg; y++)
      for (int64_t x = 0; x < W; x++) {
        const int64_t u = ((t / tt) * gh + (y / th)) * gw + (x / tw);
        perm[u * tile + tile_len[u]++] = static_cast<int32_t>((t * Hg + y) * W + x);
      }
  for (int64_t u = 0; u < n_tiles; u++)
    for (int64_t i = tile_len[u]; i < tile; i++) perm[u * tile + i] = -1;
  int64_t count = 0;
  for (int64_t u = 0; u < n_tiles; u++) {
    row_ptr[u] = static_cast<int32_t>(count);
    const int64_t ut = u / (gh * gw), uy = (u / gw) % gh, ux = u % gw;
    for (int64_t a = ut - rt; a <= ut + rt; a++)
      for (int64_t c = uy - rh; c <= uy + rh; c++)
        for (int64_t e = ux - rw; e <= ux + rw; e++) {
          if (a < 0 || a >= gt || c < 0 || c >= gh || e < 0 || e >= gw) continue;
          if (count < capacity) col_idx[count] = static_cast<int32_t>((a * gh + c) * gw + e);
          count++;
        }
  }
  row_ptr[n_tiles] = static_cast<int32_t>(count);
  *nnz = static_cast<int32_t>(count);
  return count <= capacity ? FP8ATTN_OK : FP8ATTN_EINVAL;
}


namespace {

struct ClusterLayout {
  size_t feat, labels, part1, part2, featsel, cent, csum, ccount, lab8, scount, sbase, ctot, total;
};

// with_index: also the byte labels of the fused preparation
ClusterLayout cluster_layout(int32_t B, int32_t N, int32_t H, int32_t n_feat, bool with_index = false) {
  ClusterLayout L;
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t nc = static_cast<size_t>(fp8attn::cluster_chunks(N));
  const size_t nsc = static_cast<size_t>(fp8attn::cluster_step_chunks(N));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes);
    return o;
  };
  L.feat = take(bh * N * n_feat * sizeof(float));
  L.labels = take(bh * N * sizeof(int32_t));
  L.part1 = take(bh * nc * kHeadDim * sizeof(double));
  L.part2 = take(bh * nc * kHeadDim * sizeof(double));
  L.featsel = take(bh * fp8attn::kMaxFeatures * sizeof(int32_t));
  L.cent = take(bh * fp8attn::kMaxClusters * fp8attn::kMaxFeatures * sizeof(double));
  L.csum = take(bh * nsc * fp8attn::kMaxClusters * (fp8attn::kMaxFeatures + 1) * sizeof(double));
  L.ccount = take(bh * nsc * fp8attn::kMaxClusters * sizeof(int32_t));
  const size_t ns = static_cast<size_t>(cdiv(N, fp8attn::kClusterSub));
  L.scount = take(bh * fp8attn::kMaxClusters * ns * sizeof(int32_t));
  L.sbase = take(bh * fp8attn::kMaxClusters * (ns + 1) * sizeof(int32_t));
  L.ctot = take(bh * fp8attn::kMaxClusters * sizeof(int32_t));
  L.lab8 = with_index ? take(bh * static_cast<size_t>(cdiv(N, 16) * 16)) : 0;
  L.total = off;
  return L;
}

bool valid_cluster_args(int32_t n_clusters, int32_t n_feat, int32_t iters) {
  return n_clusters >= 1 && n_clusters <= fp8attn::kMaxClusters && n_feat >= 1 && n_feat <= fp8attn::kMaxFeatures &&
         iters >= 0 && iters <= 1000;
}

void cluster_params(fp8attn::ClusterParams* cp, const ClusterLayout& L, void* workspace, int32_t B, int32_t N,
                    int32_t H, const void* v, int32_t n_clusters, int32_t n_feat, int32_t iters, int32_t* perm,
                    int32_t* labels) {
  fp8attn::ClusterParams& p = *cp;
  std::memset(&p, 0, sizeof(p));
  p.v = static_cast<const uint16_t*>(v);
  p.perm = perm;
  p.labels = labels;
  char* ws = static_cast<char*>(workspace);
  p.ws_feat = reinterpret_cast<float*>(ws + L.feat);
  p.ws_labels = reinterpret_cast<int32_t*>(ws + L.labels);
  p.ws_part1 = reinterpret_cast<double*>(ws + L.part1);
  p.ws_part2 = reinterpret_cast<double*>(ws + L.part2);
  p.ws_featsel = reinterpret_cast<int32_t*>(ws + L.featsel);
  p.ws_cent = reinterpret_cast<double*>(ws + L.cent);
  p.ws_csum = reinterpret_cast<double*>(ws + L.csum);
  p.ws_ccount = reinterpret_cast<int32_t*>(ws + L.ccount);
  p.ws_scount = reinterpret_cast<int32_t*>(ws + L.scount);
  p.ws_sbase = reinterpret_cast<int32_t*>(ws + L.sbase);
  p.ws_ctot = reinterpret_cast<int32_t*>(ws + L.ctot);
  p.ws_lab8 = L.lab8 ? reinterpret_cast<uint8_t*>(ws + L.lab8) : nullptr;
  p.n_chunks = fp8attn::cluster_chunks(N);
  p.n_schunks = fp8attn::cluster_step_chunks(N);
  p.n_sub = cdiv(N, fp8attn::kClusterSub);
  p.lab_stride = cdiv(N, 16) * 16;
  p.N = N;
  p.B = B;
  p.H = H;
  p.n_clusters = n_clusters;
  p.n_feat = n_feat;
  p.iters = iters;
}

}  // namespace

size_t fp8attn_vsmooth_cluster_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D, int32_t n_feat) {
  if (B < 1 || N < 1 || H < 1 || D != 128 || n_feat < 1 || n_feat > fp8attn::kMaxFeatures) return 0;
  return cluster_layout(B, N, H, n_feat).total;
}

fp8attn_status fp8attn_vsmooth_cluster(int32_t B, int32_t N, int32_t H, int32_t D, const void* v,
                                       int32_t n_clusters, int32_t n_feat, int32_t iters, int32_t* perm,
                                       int32_t* labels, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  if (B < 1 || N < 1 || H < 1 || D < 1) return FP8ATTN_EINVAL;
  if (D != 128) return FP8ATTN_EUNSUPPORTED;
  if (static_cast<int64_t>(B) * H > 65535) return FP8ATTN_EINVAL;
  if (!valid_cluster_args(n_clusters, n_feat, iters)) return FP8ATTN_EINVAL;
  if (!v || !perm || !aligned(v, 16) || !aligned(perm, 4)) return FP8ATTN_EINVAL;
  if (labels && !aligned(labels, 4)) return FP8ATTN_EINVAL;
  const size_t need = fp8attn_vsmooth_cluster_workspace_bytes(B, N, H, D, n_feat);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;
  fp8attn::ClusterParams p;
  cluster_params(&p, cluster_layout(B, N, H, n_feat), workspace, B, N, H, v, n_clusters, n_feat, iters, perm, labels);
  return from_hip(fp8attn::launch_cluster(p, stream));
}

size_t fp8attn_vsmooth_prepare_workspace_bytes(int32_t B, int32_t N, int32_t H, int32_t D, int32_t n_feat) {
  const size_t qb = fp8attn_quantize_workspace_bytes(B, N, H, D, 1);
  if (qb == 0 || n_feat < 1 || n_feat > fp8attn::kMaxFeatures) return 0;
  return round_up(qb) + cluster_layout(B, N, H, n_feat, true).total;
}

fp8attn_status fp8attn_vsmooth_prepare(const fp8attn_quant_args* a, const void* q, const void* k, const void* v,
                                       int32_t n_clusters, int32_t n_feat, int32_t iters, int32_t* perm,
                                       int32_t* labels, uint8_t* q8, uint8_t* k8, uint8_t* v8t, float* q_scale,
                                       float* k_scale, float* v_scale, uint16_t* v_mean, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (!a) return FP8ATTN_EINVAL;
  if (a->B < 1 || a->N < 1 || a->H < 1 || a->N_src < 1 || a->D < 1) return FP8ATTN_EINVAL;
  if (a->D != kHeadDim) return FP8ATTN_EUNSUPPORTED;
  if (a->perm_kv || a->vsmooth != 1 || a->N != a->N_src) return FP8ATTN_EINVAL;
  if (!valid_cluster_args(n_clusters, n_feat, iters)) return FP8ATTN_EINVAL;
  if (!perm || !aligned(perm, 4) || (labels && !aligned(labels, 4))) return FP8ATTN_EINVAL;
  const size_t need = fp8attn_vsmooth_prepare_workspace_bytes(a->B, a->N, a->H, a->D, n_feat);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FP8ATTN_EINVAL;
  // the quantisation with the permutation being written as its shared K/V gather
  fp8attn_quant_args qa = *a;
  qa.perm_kv = perm;
  qa.perm_kv_per_head = 1;
  const size_t qb = round_up(fp8attn_quantize_workspace_bytes(a->B, a->N, a->H, a->D, 1));
  fp8attn::QuantParams qp;
  const fp8attn_status st =
      quant_setup(&qa, q, k, v, q8, k8, v8t, q_scale, k_scale, v_scale, v_mean, workspace, qb, &qp);
  if (st != FP8ATTN_OK) return st;  // (includes the device check)
  fp8attn::ClusterParams cp;
  cluster_params(&cp, cluster_layout(a->B, a->N, a->H, n_feat, true), static_cast<char*>(workspace) + qb, a->B,
                 a->N, a->H, v, n_clusters, n_feat, iters, perm, labels);
  qp.sc_labels = cp.ws_lab8;
  qp.sc_sbase = cp.ws_sbase;
  qp.sc_ctot = cp.ws_ctot;
  qp.perm_out = perm;
  qp.sc_nsub = cp.n_sub;
  qp.sc_lab_stride = cp.lab_stride;
  qp.sc_clusters = n_clusters;
  const hipError_t e = fp8attn::launch_cluster(cp, stream);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(fp8attn::launch_quantize(qp, stream));
}

fp8attn_status fp8attn_forward_noalloc(int32_t B, int32_t N, int32_t H, int32_t D, const uint8_t* q8,
                                       const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                                       const float* k_scale, const float* v_scale,
                                       const uint16_t* v_mean, const fp8attn_fwd_opts* opts, void* out,
                                       hipStream_t stream) {
  // invalid arguments give a zero size and are reported by fp8attn_forward itself
  const size_t need = opts ? fp8attn_forward_workspace_bytes(B, N, H, D, v_mean != nullptr ? 1 : 0,
                                                             opts->sparse ? 1 : opts->kv_splits)
                           : 0;
  if (need > FP8ATTN_NOALLOC_SCRATCH_BYTES) return FP8ATTN_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const fp8attn_status dev = check_device();
    if (dev != FP8ATTN_OK) return dev;
    const fp8attn_status st = scratch_address(&ws);
    if (st != FP8ATTN_OK) return st;
  }
  return fp8attn_forward(B, N, H, D, q8, k8, v8t, q_scale, k_scale, v_scale, v_mean, opts, out, ws,
                         FP8ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

fp8attn_status fp8attn_diag_e4m3_encode(uint32_t first_bits, int64_t n, uint8_t* out, hipStream_t stream) {
  if (n < 0 || n % 4 != 0 || (n > 0 && (!out || !aligned(out, 4)))) return FP8ATTN_EINVAL;
  if (static_cast<uint64_t>(first_bits) + static_cast<uint64_t>(n) > (1ull << 32)) return FP8ATTN_EINVAL;
  if (n == 0) return FP8ATTN_OK;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;
  return from_hip(fp8attn::launch_diag_e4m3_encode(first_bits, n / 4, reinterpret_cast<uint32_t*>(out), stream));
}

fp8attn_status fp8attn_diag_e4m3_decode(const uint8_t* codes, int64_t n, float* out, hipStream_t stream) {
  if (n < 0 || n % 4 != 0 || n > (int64_t{1} << 40)) return FP8ATTN_EINVAL;
  if (n == 0) return FP8ATTN_OK;
  if (!codes || !out || !aligned(codes, 4) || !aligned(out, 16)) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;
  return from_hip(fp8attn::launch_diag_e4m3_decode(reinterpret_cast<const uint32_t*>(codes), n / 4, out, stream));
}

fp8attn_status fp8attn_diag_mfma_e4m3(const uint8_t* a, const uint8_t* bt, float* c, int32_t n_tiles,
                                      hipStream_t stream) {
  if (n_tiles < 0) return FP8ATTN_EINVAL;
  if (n_tiles == 0) return FP8ATTN_OK;
  if (!a || !bt || !c || !aligned(a, 16) || !aligned(bt, 16) || !aligned(c, 4)) return FP8ATTN_EINVAL;
  const fp8attn_status dev = check_device();
  if (dev != FP8ATTN_OK) return dev;
  return from_hip(fp8attn::launch_diag_mfma_e4m3(a, bt, c, n_tiles, stream));
}

}  // extern "C"
