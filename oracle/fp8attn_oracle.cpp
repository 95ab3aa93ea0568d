// CPU oracle for block-scaled FP8 (OCP E4M3) attention forward.
//
// TEST INFRASTRUCTURE ONLY. This file is the plain, slow reference that the HIP library is
// checked against. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
// load it. It shares no code, header, table or constant with the HIP library.
//
// Sources (the pages; each function names the passage it follows):
//  [TF]  "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力" (TeleFuser blog), sections
//        "面向注意力的 FP8 Preparation" (eq. s_q, s_k, s_v), "SM90 CuTe Mainloop",
//        "设计目标、非目标与备选方案", "输出验证".
//  [FPS] FPSAttention write-up (seekfood.cn), sections 2.1 (FP8 fake-quant), 2.2 (STA
//        neighbourhood W(u)), 3.1 (joint tiling: Q/K per block, V per channel, P per tensor).
//  [VC]  VC-Attention article (yeyulingfeng.com), section 二 (V-Smooth: clustering, block
//        mean mu_j, residual R_j, rank-one restore with the row sum r_ij), section 三 (ExpCast
//        c = round(8z + 56 + beta), beta = -0.35), Fig. 4, Fig. 5.
//  [PC]  "FP8 P-Cast Precision in Attention: Sink-Induced Collapse and the Optimality of
//        S=2^8" (xllm-io review), sections 二/三 (underflow iff p*S < 2^-10, KV order, static S),
//        Table I, MSE table.
//
// Precision: every cast the pages fix is emulated exactly (E4M3 codes, FP32 scales, BF16
// output). Everything the pages leave to the implementation (dot products, exp, row sums,
// accumulators) is carried in FP64, which is the obviously-correct choice for a checker.
// Where a floating value decides an integer code, the value is first rounded to FP32, the
// precision the GPU kernel decides in.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ----------------------------------------------------------------------------------------
// OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent field 0 holds
// subnormals m * 2^-9. S.1111.111 is NaN; there is no infinity. Largest finite value 448
// ([TF] divides amax by 448; [PC] section 三 counts 8 values per binade and puts the
// underflow threshold at 2^-10, half the smallest subnormal).
// ----------------------------------------------------------------------------------------
double e4m3_value(uint8_t code) {
  const int sign = code >> 7;
  const int exp_field = (code >> 3) & 0xF;
  const int mant = code & 0x7;
  if (exp_field == 0xF && mant == 0x7) return std::numeric_limits<double>::quiet_NaN();
  double mag;
  if (exp_field == 0)
    mag = std::ldexp(static_cast<double>(mant), -9);
  else
    mag = std::ldexp(1.0 + mant / 8.0, exp_field - 7);
  return sign ? -mag : mag;
}

// Round-to-nearest-even onto the E4M3 grid, saturating to +-448 (all |x| >= 448 map to the
// largest finite code; under RNE the values in (448, 464] round there anyway). NaN -> 0x7F.
uint8_t e4m3_code(double x) {
  if (std::isnan(x)) return 0x7F;
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  const double a = std::fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  if (a < std::ldexp(1.0, -6)) {
    // subnormal binade: grid step 2^-9; a * 2^9 is exact in double.
    const double q = std::nearbyint(a * 512.0);  // default rounding mode: nearest-even
    return sign | static_cast<uint8_t>(q);       // q == 8 is the smallest normal code 0x08
  }
  int e2;
  std::frexp(a, &e2);  // a = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;      // a in [2^e, 2^(e+1))
  const double q = std::nearbyint((std::ldexp(a, -e) - 1.0) * 8.0);  // exact in double
  int mant = static_cast<int>(q);
  if (mant == 8) {
    mant = 0;
    e += 1;
  }
  return sign | static_cast<uint8_t>(((e + 7) << 3) | mant);
}

// BF16: upper half of an IEEE binary32. Encoding rounds to nearest-even.
double bf16_value(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint16_t bf16_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

float bf16_float(uint16_t bits) { return static_cast<float>(bf16_value(bits)); }

// Block scale per [TF] eq. s_q/s_k/s_v (scale = amax / 448, the dequantisation multiplier)
// written in the multiplicative form of [FPS] 2.1 (codes = FP8(x * s_g), s_g = 448 / amax).
// Operation order, fixed here because it decides codes at rounding boundaries:
//   scale = fl32(amax / 448), inv = fl32(448 / amax), code = E4M3(fl32(x * inv)).
struct BlockScale {
  float scale;
  float inv;
};

BlockScale block_scale(float amax) {
  if (amax == 0.0f) return {0.0f, 0.0f};
  return {amax / 448.0f, 448.0f / amax};
}

uint8_t quant_code(float x, const BlockScale& s) {
  if (s.inv == 0.0f) return 0;
  const float y = x * s.inv;  // one FP32 rounding
  return e4m3_code(static_cast<double>(y));
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

// Sol routing inputs of orc_attention (see orc_sol_prepare for the layouts).
struct OrcSol {
  const uint64_t* mask;     // exact-block bitmask [B, H, NB, W]
  const uint8_t* kq8;       // quantised K summaries [B, H, 64 * NBg, D]
  const float* kq_scale;    // [B, H, NBg]
  const uint16_t* vsum;     // V summaries, bf16 [B, H, NB, D]
};

// ---------------------------------------------------------------------------------------
// Codec entry points (used by the format pins).
// ---------------------------------------------------------------------------------------
void orc_e4m3_encode(const double* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = e4m3_code(x[i]);
}

void orc_e4m3_encode_f32(const float* x, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = e4m3_code(static_cast<double>(x[i]));
}

void orc_e4m3_decode(const uint8_t* c, double* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = e4m3_value(c[i]);
}

void orc_bf16_encode(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = bf16_bits(x[i]);
}

// ---------------------------------------------------------------------------------------
// QKV quantisation.
//  * Q, K: one FP32 scale per (b, h, 64-token block) of the layout order ([TF] eq. s_q, s_k;
//    [FPS] 3.1 "Q/K per block").
//  * V: one FP32 scale per (b, h, channel) over all valid tokens ([TF] eq. s_v; [FPS] 3.1
//    "V per channel"), codes stored token-contiguous ([TF] "second launch ... token-contiguous
//    backing storage").
//  * Optional gathers: perm_q[N] (shared by all heads) and perm_kv (shared [N] or per head
//    [B*H*N]) give the source token of each layout position, -1 for padding (zero vector,
//    excluded from every amax and mean). K and V are permuted jointly ([VC] 二 reorders value
//    tokens; moving keys with their values keeps the attention unchanged).
//  * V-Smooth ([VC] 二): per 128-row block j of the permuted V', mu_j = column mean over the
//    valid rows (stored as one 16-bit vector per block, BF16 here), R = V' - mu_hat_j, and R
//    (not V) is quantised per channel.
//
//  * Sequence-mean smoothing ([TF] MiniMax-H3 section: K' = K - mean_T(K), V' = V - mean_T(V)
//    per head, FP32 statistics; the K shift moves every logit of a query row by the same
//    constant, and mean_T(V) is added back to the output because each softmax row sums to 1):
//    smoothing 1 shifts K, 2 shifts K and V. The mean is seq_mean below; K' = fl32(K - mean) and
//    V' = fl32(V - mean) are quantised by the usual rules. v_shift [B, H, D] receives the vector
//    the attention adds to its output: mean_T(V), or with v_bias_correction (the page's
//    compensation of the residual mean bias that rounding V' to E4M3 leaves) mean_T(V) - e,
//    e = seq_mean of fl32(fl32(decode(code) * s_v) - V') over the valid rows.
//
// Shapes: q, k, v bf16 [B, Nsrc, H, D]; q8, k8 [B, H, N64, D]; v8t [B, H, D, N64];
// q_scale, k_scale [B, H, NB]; v_scale [B, H, D]; v_mean bf16 [B, H, ceil(N/128), D];
// v_shift f32 [B, H, D]. N64 = 64 * NB, NB = ceil(N / 64). Padding rows/columns get code 0.
// Returns 0, or 1 on an argument error.
// ---------------------------------------------------------------------------------------

// Mean over the valid layout rows of one channel, in FP32 ([TF] says the statistics are FP32;
// the summation order is this reading): the valid values of each 64-position block of the
// layout summed in ascending position, the block sums combined by a pairwise tree (level by
// level s[i] = s[2i] + s[2i+1], an odd last element carried up unchanged), the total divided
// by the number of valid rows. x[i * stride] is row i's value.
float seq_mean(const float* x, int64_t stride, const std::vector<char>& valid, int64_t N) {
  const int64_t NB = ceil_div(N, 64);
  std::vector<float> s(NB, 0.0f);
  int64_t count = 0;
  for (int64_t blk = 0; blk < NB; blk++) {
    float acc = 0.0f;
    for (int64_t i = blk * 64; i < std::min<int64_t>(N, blk * 64 + 64); i++)
      if (valid[i]) {
        acc = acc + x[i * stride];
        count++;
      }
    s[blk] = acc;
  }
  int64_t n = NB;
  while (n > 1) {
    for (int64_t i = 0; i < n / 2; i++) s[i] = s[2 * i] + s[2 * i + 1];
    if (n % 2) s[n / 2] = s[n - 1];
    n = (n + 1) / 2;
  }
  return count ? s[0] / static_cast<float>(count) : 0.0f;
}

int orc_quantize(int B, int Nsrc, int N, int H, int D, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const int32_t* perm_q, const int32_t* perm_kv,
                 int perm_kv_per_head, int vsmooth, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                 float* q_scale, float* k_scale, float* v_scale, uint16_t* v_mean,
                 int smoothing, int v_bias_correction, float* v_shift) {
  if (B < 1 || N < 1 || H < 1 || D < 1 || Nsrc < 1) return 1;
  if (!perm_q && N != Nsrc) return 1;
  if (!perm_kv && N != Nsrc) return 1;
  if (vsmooth && !v_mean) return 1;
  if (smoothing < 0 || smoothing > 2 || (smoothing == 2 && (vsmooth || !v_shift))) return 1;
  if (v_bias_correction && smoothing != 2) return 1;
  const int64_t NB = ceil_div(N, 64), N64 = NB * 64, NB128 = ceil_div(N, 128);

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; b++) {
    for (int h = 0; h < H; h++) {
      const int64_t bh = static_cast<int64_t>(b) * H + h;
      auto src_index = [&](const int32_t* perm, bool per_head, int64_t i) -> int64_t {
        if (!perm) return i;
        return per_head ? perm[bh * N + i] : perm[i];
      };
      auto elem = [&](const uint16_t* x, int64_t src, int d) -> float {
        return bf16_float(x[((static_cast<int64_t>(b) * Nsrc + src) * H + h) * D + d]);
      };

      // Q and K: per 64-token block of the layout (K shifted by its sequence mean when
      // smoothing is on).
      for (int t = 0; t < 2; t++) {
        const uint16_t* x = t == 0 ? q : k;
        const int32_t* perm = t == 0 ? perm_q : perm_kv;
        const bool per_head = t == 0 ? false : (perm_kv_per_head != 0);
        uint8_t* codes = t == 0 ? q8 : k8;
        float* scales = t == 0 ? q_scale : k_scale;
        std::vector<float> shift(D, 0.0f);
        if (t == 1 && smoothing >= 1) {
          std::vector<float> kl(static_cast<size_t>(N) * D, 0.0f);
          std::vector<char> kvalid(N, 0);
          for (int64_t i = 0; i < N; i++) {
            const int64_t s = src_index(perm, per_head, i);
            if (s < 0) continue;
            kvalid[i] = 1;
            for (int d = 0; d < D; d++) kl[i * D + d] = elem(x, s, d);
          }
          for (int d = 0; d < D; d++) shift[d] = seq_mean(kl.data() + d, D, kvalid, N);
        }
        auto value = [&](int64_t s, int d) -> float { return elem(x, s, d) - shift[d]; };  // FP32
        for (int64_t blk = 0; blk < NB; blk++) {
          float amax = 0.0f;
          for (int64_t i = blk * 64; i < std::min<int64_t>(N, blk * 64 + 64); i++) {
            const int64_t s = src_index(perm, per_head, i);
            if (s < 0) continue;
            for (int d = 0; d < D; d++) amax = std::max(amax, std::fabs(value(s, d)));
          }
          const BlockScale sc = block_scale(amax);
          scales[bh * NB + blk] = sc.scale;
          for (int64_t i = blk * 64; i < blk * 64 + 64; i++) {
            uint8_t* row = codes + (bh * N64 + i) * D;
            const int64_t s = i < N ? src_index(perm, per_head, i) : -1;
            for (int d = 0; d < D; d++) row[d] = s < 0 ? 0 : quant_code(value(s, d), sc);
          }
        }
      }

      // V (or the V-Smooth residual): gather the layout rows once.
      std::vector<float> vl(static_cast<size_t>(N) * D, 0.0f);
      std::vector<char> valid(N, 0);
      for (int64_t i = 0; i < N; i++) {
        const int64_t s = src_index(perm_kv, perm_kv_per_head != 0, i);
        if (s < 0) continue;
        valid[i] = 1;
        for (int d = 0; d < D; d++) vl[i * D + d] = elem(v, s, d);
      }
      if (vsmooth) {
        for (int64_t j = 0; j < NB128; j++) {
          const int64_t lo = j * 128, hi = std::min<int64_t>(N, lo + 128);
          int64_t count = 0;
          for (int64_t i = lo; i < hi; i++) count += valid[i];
          for (int d = 0; d < D; d++) {
            double sum = 0.0;
            for (int64_t i = lo; i < hi; i++)
              if (valid[i]) sum += vl[i * D + d];
            const float mean = count ? static_cast<float>(sum / static_cast<double>(count)) : 0.0f;
            const uint16_t mbits = bf16_bits(mean);
            v_mean[(bh * NB128 + j) * D + d] = mbits;
            const float mhat = bf16_float(mbits);
            for (int64_t i = lo; i < hi; i++)
              if (valid[i]) vl[i * D + d] = vl[i * D + d] - mhat;  // FP32 subtraction
          }
        }
      }
      std::vector<float> vmean(D, 0.0f);
      if (smoothing == 2) {
        for (int d = 0; d < D; d++) {
          vmean[d] = seq_mean(vl.data() + d, D, valid, N);
          for (int64_t i = 0; i < N; i++)
            if (valid[i]) vl[i * D + d] = vl[i * D + d] - vmean[d];  // FP32 subtraction
        }
      }
      for (int d = 0; d < D; d++) {
        float amax = 0.0f;
        for (int64_t i = 0; i < N; i++)
          if (valid[i]) amax = std::max(amax, std::fabs(vl[i * D + d]));
        const BlockScale sc = block_scale(amax);
        v_scale[bh * D + d] = sc.scale;
        uint8_t* row = v8t + (bh * D + d) * N64;
        for (int64_t i = 0; i < N64; i++)
          row[i] = (i < N && valid[i]) ? quant_code(vl[i * D + d], sc) : 0;
        if (v_shift) {
          float c = vmean[d];
          if (v_bias_correction) {
            std::vector<float> err(N, 0.0f);
            for (int64_t i = 0; i < N; i++)
              if (valid[i]) {
                const float deq = static_cast<float>(e4m3_value(row[i])) * sc.scale;  // FP32 product
                err[i] = deq - vl[i * D + d];                                          // FP32
              }
            c = c - seq_mean(err.data(), 1, valid, N);
          }
          v_shift[bh * D + d] = c;
        }
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------------------
// Sol routing ([TF] "Sol Routing" and "SM90 CuTe Mainloop": 64-token Q/KV blocks, K and V
// summaries per KV block, a threshold theta = mu + tau * sigma per Q block from a diag or exact
// estimator, a route QK of the block-quantised Q with the quantised K summaries, an exact-block
// bitmask, sinks always exact). Readings (where the page is silent):
//  * summaries come from the dequantised E4M3 K and V of the block's n_j valid keys:
//      sK = sum_t decode(K8[t, d])   (exact in FP32: multiples of 2^-9 below 2^15 in magnitude)
//      kbar[j, d] = fl32(fl32(sK * s_k[j]) / n_j);   vbar likewise with s_v[d], stored as BF16;
//  * the K summaries are quantised like K: groups of 64 summaries, scale = fl32(amax / 448),
//    codes E4M3(fl32(kbar * fl32(448 / amax)));
//  * mu and sigma are the mean and standard deviation of the block's route scores over all
//    pairs (valid query i of the block, KV block j), from second moments: with q_i the
//    dequantised queries, qbar their mean, Mq = mean_i q_i q_i^T, and over the summaries
//    m = mean_j kbar_j, Mk = mean_j kbar_j kbar_j^T (FP64, every summary weighted equally):
//      mu = ss * qbar . m,   E2 = ss^2 * sum_{d,e} Mq[d, e] Mk[d, e]   (estimator 1, "exact": the
//      full second moments, which give the exact mean square over the pairs) or
//      E2 = ss^2 * sum_d Mq[d, d] Mk[d, d]   (estimator 0, "diag": per-channel moments only),
//      sigma = sqrt(max(E2 - mu^2, 0)),   theta_u = mu + tau * sigma   (ss = softmax_scale);
//  * route score r_ij = (q8_i . kq8_j) * s_q[u] * kq_scale[j / 64] * softmax_scale; KV block j is
//    exact for Q block u when j < sink_blocks or some valid query i of u has r_ij >= theta_u.
// A device evaluates r_ij on the matrix cores (R17: each group of 8 products truncated, error
// below 2^-11 of the group maxima) and theta in floating point, so a decision within
// b_ij = 2^-11 * sum_g max |q k| * scales + 2^-20 * |r_ij| + 2^-14 * (|mu| + |tau| sqrt(E2))
// of the threshold can go either way: such bits are flagged in amb_mask (the mask holds the exact
// decision).
// Shapes: q8, k8 [B, H, N64, D], v8t [B, H, D, N64]; ksum f32 [B, H, NB, D]; vsum bf16 [B, H, NB,
// D]; kq8 [B, H, 64 * NBg, D] (NBg = ceil(NB / 64)); kq_scale [B, H, NBg]; theta f64 [B, H, NB];
// mask, amb_mask uint64 [B, H, NB, W] (W = ceil(NB / 64); bit j % 64 of word j / 64).
// ---------------------------------------------------------------------------------------
int orc_sol_prepare(int B, int N, int H, int D, const uint8_t* q8, const uint8_t* k8,
                    const uint8_t* v8t, const float* q_scale, const float* k_scale,
                    const float* v_scale, double tau, int estimator, int sink_blocks,
                    double softmax_scale, float* ksum, uint16_t* vsum, uint8_t* kq8,
                    float* kq_scale, double* theta, uint64_t* mask, uint64_t* amb_mask) {
  if (B < 1 || N < 1 || H < 1 || D < 1 || estimator < 0 || estimator > 1 || sink_blocks < 0) return 1;
  const int64_t NB = ceil_div(N, 64), N64 = NB * 64, NBg = ceil_div(NB, 64), W = ceil_div(NB, 64);
  std::vector<double> code_value(256);
  for (int c = 0; c < 256; c++) code_value[c] = e4m3_value(static_cast<uint8_t>(c));

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; b++) {
    for (int h = 0; h < H; h++) {
      const int64_t bh = static_cast<int64_t>(b) * H + h;
      // summaries
      for (int64_t j = 0; j < NB; j++) {
        const int64_t n = std::min<int64_t>(64, N - 64 * j);
        for (int d = 0; d < D; d++) {
          float sk = 0.0f, sv = 0.0f;
          for (int64_t t = 64 * j; t < 64 * j + n; t++) {
            sk += static_cast<float>(code_value[k8[(bh * N64 + t) * D + d]]);
            sv += static_cast<float>(code_value[v8t[(bh * D + d) * N64 + t]]);
          }
          const float kb = (sk * k_scale[bh * NB + j]) / static_cast<float>(n);
          const float vb = (sv * v_scale[bh * D + d]) / static_cast<float>(n);
          ksum[(bh * NB + j) * D + d] = kb;
          vsum[(bh * NB + j) * D + d] = bf16_bits(vb);
        }
      }
      // quantised K summaries (groups of 64 summaries; padding summaries code 0)
      for (int64_t g = 0; g < NBg; g++) {
        float amax = 0.0f;
        for (int64_t j = 64 * g; j < std::min(NB, 64 * g + 64); j++)
          for (int d = 0; d < D; d++) amax = std::max(amax, std::fabs(ksum[(bh * NB + j) * D + d]));
        const BlockScale sc = block_scale(amax);
        kq_scale[bh * NBg + g] = sc.scale;
        for (int64_t j = 64 * g; j < 64 * g + 64; j++)
          for (int d = 0; d < D; d++)
            kq8[(bh * NBg * 64 + j) * D + d] = j < NB ? quant_code(ksum[(bh * NB + j) * D + d], sc) : 0;
      }
      // moments of the summaries
      std::vector<double> mk(D, 0.0), Mk(static_cast<size_t>(D) * D, 0.0);
      for (int d = 0; d < D; d++) {
        for (int64_t j = 0; j < NB; j++) mk[d] += static_cast<double>(ksum[(bh * NB + j) * D + d]);
        mk[d] /= static_cast<double>(NB);
      }
      for (int d = 0; d < D; d++)
        for (int e = 0; e < D; e++) {
          if (estimator == 0 && e != d) continue;
          double acc = 0.0;
          for (int64_t j = 0; j < NB; j++)
            acc += static_cast<double>(ksum[(bh * NB + j) * D + d]) * static_cast<double>(ksum[(bh * NB + j) * D + e]);
          Mk[static_cast<size_t>(d) * D + e] = acc / static_cast<double>(NB);
        }
      // thresholds and the route
      for (int64_t u = 0; u < NB; u++) {
        const int64_t nq = std::min<int64_t>(64, N - 64 * u);
        const double sq = q_scale[bh * NB + u];
        std::vector<double> qbar(D, 0.0), Mq(static_cast<size_t>(D) * D, 0.0);
        for (int64_t i = 64 * u; i < 64 * u + nq; i++) {
          const uint8_t* qr = q8 + (bh * N64 + i) * D;
          for (int d = 0; d < D; d++) {
            const double qd = code_value[qr[d]] * sq;
            qbar[d] += qd;
            for (int e = 0; e < D; e++) {
              if (estimator == 0 && e != d) continue;
              Mq[static_cast<size_t>(d) * D + e] += qd * code_value[qr[e]] * sq;
            }
          }
        }
        double mu = 0.0, e2 = 0.0;
        for (int d = 0; d < D; d++) {
          qbar[d] /= static_cast<double>(nq);
          mu += qbar[d] * mk[d];
          for (int e = 0; e < D; e++) e2 += Mq[static_cast<size_t>(d) * D + e] / static_cast<double>(nq) *
                                            Mk[static_cast<size_t>(d) * D + e];
        }
        mu *= softmax_scale;
        e2 *= softmax_scale * softmax_scale;
        const double th = mu + tau * std::sqrt(std::max(e2 - mu * mu, 0.0));
        const double th_err = std::ldexp(1.0, -14) * (std::fabs(mu) + std::fabs(tau) * std::sqrt(e2));
        theta[bh * NB + u] = th;
        uint64_t* mrow = mask + (bh * NB + u) * W;
        uint64_t* arow = amb_mask + (bh * NB + u) * W;
        for (int64_t w = 0; w < W; w++) mrow[w] = arow[w] = 0;
        for (int64_t j = 0; j < NB; j++) {
          const uint64_t bit = 1ull << (j % 64);
          if (j < sink_blocks) {
            mrow[j / 64] |= bit;
            continue;
          }
          const double sc = sq * static_cast<double>(kq_scale[bh * NBg + j / 64]) * softmax_scale;
          bool any_ge = false, any_amb = false;
          for (int64_t i = 64 * u; i < 64 * u + nq; i++) {
            const uint8_t* qr = q8 + (bh * N64 + i) * D;
            const uint8_t* kr = kq8 + (bh * NBg * 64 + j) * D;
            double dot = 0.0, gsum = 0.0;
            for (int g = 0; g < D; g += 8) {
              double gm = 0.0;
              for (int d = g; d < std::min(D, g + 8); d++) {
                const double pr = code_value[qr[d]] * code_value[kr[d]];
                dot += pr;
                gm = std::max(gm, std::fabs(pr));
              }
              gsum += gm;
            }
            const double r = dot * sc;
            const double bnd = std::ldexp(gsum, -11) * sc + std::ldexp(1.0, -20) * std::fabs(r) + th_err;
            if (r >= th) any_ge = true;
            if (std::fabs(r - th) <= bnd) any_amb = true;
          }
          if (any_ge) mrow[j / 64] |= bit;
          // ambiguous unless some query is clearly above, or every query clearly below
          bool clearly_above = false;
          if (any_amb) {
            for (int64_t i = 64 * u; i < 64 * u + nq && !clearly_above; i++) {
              const uint8_t* qr = q8 + (bh * N64 + i) * D;
              const uint8_t* kr = kq8 + (bh * NBg * 64 + j) * D;
              double dot = 0.0, gsum = 0.0;
              for (int g = 0; g < D; g += 8) {
                double gm = 0.0;
                for (int d = g; d < std::min(D, g + 8); d++) {
                  const double pr = code_value[qr[d]] * code_value[kr[d]];
                  dot += pr;
                  gm = std::max(gm, std::fabs(pr));
                }
                gsum += gm;
              }
              const double r = dot * sc;
              const double bnd = std::ldexp(gsum, -11) * sc + std::ldexp(1.0, -20) * std::fabs(r) + th_err;
              if (r - th > bnd) clearly_above = true;
            }
            if (!clearly_above) arow[j / 64] |= bit;
          }
        }
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------------------
// Attention forward. One routine serves every mode; each output row is independent.
//
// mode 0 EXACT    softmax(QK^T * scale) V in FP64, two passes, no quantisation.
// mode 1 NOQUANT  the streaming (online-softmax) loop of the FP8 path with every cast removed.
// mode 2 PCAST    only P is cast to E4M3 ([PC] "kernel-faithful simulation": Q, K, V kept in
//                 high precision, P8 = E4M3(S * p), output divided by S afterwards).
// mode 3 FP8      the full path on the quantised codes and scales from orc_quantize.
//
// Streaming loop ([TF] "SM90 CuTe Mainloop": exact E4M3 QK -> scale -> online softmax ->
// P to E4M3 -> E4M3 PV with token-contiguous V -> V channel scale after all PV; [PC] 二/三:
// KV block order and the static scale S). Per 64-key block, in the requested order:
//   x_k   = (q . k) * s_q * s_k * softmax_scale
//   m'    = max(m, max_k x_k),  alpha = exp(m - m')   (alpha = 0 while m = -inf)
//   p_k   = exp(x_k - m')
//   code  = E4M3(fl32(S * p_k))                  (RNE; [PC]: underflow iff p*S < 2^-10)
//         | clamp(rint(fl32(8 z + 56 - 0.35)), 0, 126),  z = log2(S * p_k)   (ExpCast, [VC] 三)
//   l     = alpha * l + r,   r = sum_k p_k  (RNE)   or  sum_k decode(code) / S  (ExpCast)
//   acc_d = alpha * acc_d + sum_k decode(code) * V_kd
//   V-Smooth: M_d = alpha * M_d + r * mu_hat_j,d  (j = 128-row V block of this key block)
// End: O_d = acc_d * s_v,d / (S * l), or O_d = ((s_r,d / S) * acc_d + M_d) / l with V-Smooth.
// Masked keys (index >= N, or STA padding) have p = 0 and do not move the max.
//
// KV order: forward visits blocks 0..NB-1, reverse NB-1..0 ([PC] "前向 0→N vs 反向 N→0").
// Sparse (STA, [FPS] 2.2/3.1): the layout is tile-major with tile_tokens per tile; the query
// tile u visits, for each KV tile v listed in col_idx[row_ptr[u] .. row_ptr[u+1]) (ascending),
// that tile's blocks in order; reverse reverses the whole sequence. Positions >= tile_len of a
// tile are padding: masked as keys, not computed as queries.
//
// Inputs by mode:
//   modes 0-2: qd, kd, vd float64 [B, H, N, D] (layout order).
//   mode 3:    q8, k8 [B, H, N64, D], v8t [B, H, D, N64], q_scale, k_scale [B, H, NB],
//              v_scale [B, H, D], v_mean bf16 [B, H, ceil(N/128), D] or null (V-Smooth off).
// rows: the layout query indices to compute (same for every (b, h)), n_rows of them.
// Outputs: out f64 [B, H, n_rows, D]; out_bf16 [B, H, n_rows, D] or null; underflow
// [B, H, n_rows] or null (keys with p > 0 whose P code is 0); row_valid [B, H, n_rows] or null;
// amb_bound [B, H, n_rows, D] or null (modes 2-3); v_shift [B, H, D] or null (mode 3: the
// vector sequence-mean smoothing adds to every output row, see orc_quantize); kv_splits: 1 (or
// 0) streams each row in one piece, > 1 is split-KV (dense rows, modes 1-3, see below).
//
// Ambiguous P codes. The pages fix P8 = E4M3(S p) but not how p is evaluated; an FP32
// evaluation (the kernel's precision) can land on either side of a rounding boundary when S p
// lies within a few FP32 rounding errors of it, and both codes are then correct results. A key
// is ambiguous when |S p - boundary| <= eta * S p with
//   eta = 2^-20 * (|x| + |m'| + |ln S| + 1)        (x, m' in natural-log units),
// a generous bound on the relative error of an FP32 evaluation of exp(x - m' + ln S), plus (FP8
// mode) the error bound of the E4M3 matrix-core contraction on x_k and on the running max (the
// contraction sums each group of 8 consecutive products after truncating them to
// 2^(floor(log2 max|p|) - 14) of the group, an error below 2^-11 * sum_g max_g |p|); for ExpCast
// the same window is applied to 8 z + 55.65 around a half-integer. Only the nearest rounding
// boundary is considered: an ambiguous key may take its code or the one neighbouring code across
// that boundary (one code step), never a code further away. Where the window would span more
// than one code (logits so large that the contraction bound exceeds a code step) no allowance
// covers it, and parity is not claimed element by element there. amb_bound[d] is the largest
// change of output channel d that flipping every ambiguous code of the row can cause:
//   sum_k step_k * e^(m_k - m_final) / (S l) * (|V_kd| + [ExpCast] |O_d|),
// step_k the gap between the two candidate code values, V the dequantised value (V-Smooth: the
// residual part plus, for ExpCast, the block mean), plus the same contraction bound for PV
// (2^-11 * sum over groups of 8 keys of max |P8 V_d|, scaled like acc), plus the change of the
// normalisation the logit error bound allows (2 |O_d| sum_k p_k (dx_k + dm) / l).
// ---------------------------------------------------------------------------------------
int orc_attention(int mode, int B, int N, int H, int D, const double* qd, const double* kd,
                  const double* vd, const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  const uint16_t* v_mean, double softmax_scale, double p_scale, int kv_reverse,
                  int expcast, int tile_tokens, int n_tiles, const int32_t* tile_len,
                  const int32_t* row_ptr, const int32_t* col_idx, const int32_t* rows,
                  int64_t n_rows, double* out, uint16_t* out_bf16, int64_t* underflow,
                  uint8_t* row_valid, double* amb_bound, const float* v_shift, int kv_splits,
                  const OrcSol* sol) {
  if (mode < 0 || mode > 3 || B < 1 || N < 1 || H < 1 || D < 1 || n_rows < 0) return 1;
  if (mode < 3 && (!qd || !kd || !vd)) return 1;
  if (mode == 3 && (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale)) return 1;
  if (!(p_scale > 0.0)) return 1;
  const bool sparse = tile_len != nullptr;
  if (sol && (mode != 3 || sparse || v_mean || kv_splits > 1 || !sol->mask || !sol->kq8 ||
              !sol->kq_scale || !sol->vsum))
    return 1;
  if (sparse && (tile_tokens <= 0 || tile_tokens % 64 != 0 ||
                 static_cast<int64_t>(tile_tokens) * n_tiles != N || !row_ptr || !col_idx))
    return 1;
  const int64_t NB = ceil_div(N, 64), N64 = NB * 64, NB128 = ceil_div(N, 128);
  const bool vsmooth = (mode == 3 && v_mean != nullptr);
  const double S = p_scale;
  const double log2e = 1.0 / std::log(2.0);

  double code_value[256];
  for (int c = 0; c < 256; c++) code_value[c] = e4m3_value(static_cast<uint8_t>(c));

#pragma omp parallel for collapse(3) schedule(dynamic, 4)
  for (int b = 0; b < B; b++) {
    for (int h = 0; h < H; h++) {
      for (int64_t ri = 0; ri < n_rows; ri++) {
        const int64_t bh = static_cast<int64_t>(b) * H + h;
        const int64_t i = rows[ri];
        const int64_t o_idx = bh * n_rows + ri;
        double* o = out + o_idx * D;
        bool computable = (i >= 0 && i < N);
        if (computable && sparse) computable = (i % tile_tokens) < tile_len[i / tile_tokens];
        if (row_valid) row_valid[o_idx] = computable ? 1 : 0;
        if (underflow) underflow[o_idx] = 0;
        if (amb_bound)
          for (int d = 0; d < D; d++) amb_bound[o_idx * D + d] = 0.0;
        if (!computable) {
          for (int d = 0; d < D; d++) o[d] = 0.0;
          if (out_bf16)
            for (int d = 0; d < D; d++) out_bf16[o_idx * D + d] = 0;
          continue;
        }

        // Key validity and the logit of one (query, key) pair.
        auto key_valid = [&](int64_t kk) -> bool {
          if (kk >= N) return false;
          if (sparse) return (kk % tile_tokens) < tile_len[kk / tile_tokens];
          return true;
        };
        auto logit = [&](int64_t kk) -> double {
          double dot = 0.0;
          if (mode == 3) {
            const uint8_t* qr = q8 + (bh * N64 + i) * D;
            const uint8_t* kr = k8 + (bh * N64 + kk) * D;
            for (int d = 0; d < D; d++) dot += code_value[qr[d]] * code_value[kr[d]];
            return dot * static_cast<double>(q_scale[bh * NB + i / 64]) *
                   static_cast<double>(k_scale[bh * NB + kk / 64]) * softmax_scale;
          }
          const double* qr = qd + (bh * N + i) * D;
          const double* kr = kd + (bh * N + kk) * D;
          for (int d = 0; d < D; d++) dot += qr[d] * kr[d];
          return dot * softmax_scale;
        };
        auto value = [&](int64_t kk, int d) -> double {
          if (mode == 3) return code_value[v8t[(bh * D + d) * N64 + kk]];
          return vd[(bh * N + kk) * D + d];
        };

        if (mode == 0) {
          // Two-pass FP64 softmax over every valid key of the row's mask.
          std::vector<int64_t> keys;
          if (sparse) {
            const int64_t u = i / tile_tokens;
            for (int32_t e = row_ptr[u]; e < row_ptr[u + 1]; e++)
              for (int64_t kk = static_cast<int64_t>(col_idx[e]) * tile_tokens;
                   kk < static_cast<int64_t>(col_idx[e] + 1) * tile_tokens; kk++)
                if (key_valid(kk)) keys.push_back(kk);
          } else {
            for (int64_t kk = 0; kk < N; kk++) keys.push_back(kk);
          }
          std::vector<double> x(keys.size());
          double m = -std::numeric_limits<double>::infinity();
          for (size_t t = 0; t < keys.size(); t++) {
            x[t] = logit(keys[t]);
            m = std::max(m, x[t]);
          }
          double l = 0.0;
          std::vector<double> acc(D, 0.0);
          for (size_t t = 0; t < keys.size(); t++) {
            const double p = std::exp(x[t] - m);
            l += p;
            for (int d = 0; d < D; d++) acc[d] += p * value(keys[t], d);
          }
          for (int d = 0; d < D; d++) o[d] = acc[d] / l;
          if (amb_bound)
            for (int d = 0; d < D; d++) amb_bound[o_idx * D + d] = 0.0;
        } else {
          // The sequence of 64-key blocks this query visits.
          std::vector<int64_t> blocks;
          if (sparse) {
            const int64_t u = i / tile_tokens, per_tile = tile_tokens / 64;
            for (int32_t e = row_ptr[u]; e < row_ptr[u + 1]; e++)
              for (int64_t t = 0; t < per_tile; t++) blocks.push_back(col_idx[e] * per_tile + t);
          } else {
            for (int64_t kb = 0; kb < NB; kb++) blocks.push_back(kb);
          }
          if (kv_reverse) std::reverse(blocks.begin(), blocks.end());
          // Sol routing: the row's exact-block bits, and per KV block the route score r_j of the
          // query against the quantised K summary (natural-log units, like the logits) and the
          // bound on the matrix core's contraction error of that score
          const uint64_t* sol_mrow = nullptr;
          std::vector<double> sol_r, sol_rb;
          if (sol) {
            const int64_t u = i / 64, W = ceil_div(NB, 64), NBg = ceil_div(NB, 64);
            sol_mrow = sol->mask + (bh * NB + u) * W;
            sol_r.assign(NB, 0.0);
            sol_rb.assign(NB, 0.0);
            const uint8_t* qr = q8 + (bh * N64 + i) * D;
            for (int64_t j = 0; j < NB; j++) {
              const uint8_t* kr = sol->kq8 + (bh * NBg * 64 + j) * D;
              double dot = 0.0, gsum = 0.0;
              for (int g = 0; g < D; g += 8) {
                double gm = 0.0;
                for (int d = g; d < std::min(D, g + 8); d++) {
                  const double pr = code_value[qr[d]] * code_value[kr[d]];
                  dot += pr;
                  gm = std::max(gm, std::fabs(pr));
                }
                gsum += gm;
              }
              const double sc = static_cast<double>(q_scale[bh * NB + u]) *
                                static_cast<double>(sol->kq_scale[bh * NBg + j / 64]) * softmax_scale;
              sol_r[j] = dot * sc;
              sol_rb[j] = std::ldexp(gsum, -11) * sc;
            }
          }
          auto sol_exact = [&](int64_t j) { return ((sol_mrow[j / 64] >> (j % 64)) & 1ull) != 0; };
          // One streaming pass over a sequence of key blocks: the row's normalised output, its
          // running max and row sum, and the ambiguity bound of that output.
          struct Pass {
            std::vector<double> o, amb;
            double m = 0.0, l = 0.0, lx = 0.0;
            int64_t n_under = 0;
          };
          auto stream = [&](const std::vector<int64_t>& seq) -> Pass {

          double m = -std::numeric_limits<double>::infinity(), l = 0.0;
          // accS: Sol's summary contributions, in dequantised V units (acc holds the exact blocks'
          // S-scaled P codes times V codes); both share the running max m and the row sum l
          std::vector<double> acc(D, 0.0), accM(D, 0.0), accS(D, 0.0);
          int64_t n_under = 0;
          // ambiguity sums per channel, in the running-max units of acc
          std::vector<double> amb_v(amb_bound ? D : 0, 0.0), amb_pv(amb_bound ? D : 0, 0.0);
          double amb_l = 0.0;   // ExpCast: code steps that move the row sum
          double amb_lx = 0.0;  // row-sum change from the logit error bound (sum p * dx)
          // |dequantised value| of key kk in channel d, and (V-Smooth with ExpCast, where a code
          // flip also moves the row sum r) the block mean's magnitude
          auto vabs = [&](int64_t kk, int d) -> double {
            double val = std::fabs(value(kk, d));
            if (mode == 3) val *= static_cast<double>(v_scale[bh * D + d]);
            if (vsmooth && expcast) val += std::fabs(bf16_value(v_mean[(bh * NB128 + kk / 128) * D + d]));
            return val;
          };
          // Bound on the QK contraction error of the kernel's E4M3 MFMA (mode 3): the products
          // of each group of 8 consecutive channels are truncated to 2^(floor(log2 max|p|) - 14)
          // of that group before an FP32 sum, so |error| < 2^-11 * sum_g max_{d in g} |p_d|.
          auto qk_err = [&](int64_t kk) -> double {
            if (mode != 3 || !amb_bound) return 0.0;
            const uint8_t* qr = q8 + (bh * N64 + i) * D;
            const uint8_t* kr = k8 + (bh * N64 + kk) * D;
            double gsum = 0.0;
            for (int g = 0; g < D; g += 8) {
              double gm = 0.0;
              for (int d = g; d < std::min(D, g + 8); d++)
                gm = std::max(gm, std::fabs(code_value[qr[d]] * code_value[kr[d]]));
              gsum += gm;
            }
            return std::ldexp(gsum, -11) * static_cast<double>(q_scale[bh * NB + i / 64]) *
                   static_cast<double>(k_scale[bh * NB + kk / 64]) * softmax_scale;
          };
          double x[64], pv[64], dx[64];
          bool kv_ok[64];
          double dm_run = 0.0;     // error bound of the running max
          for (const int64_t kb : seq) {
            if (sol && !sol_exact(kb)) {
              // Summary block ([TF] "Sol Routing": the block's compressed contribution stays in the
              // same online-softmax state; "SM90 CuTe Mainloop": numerator, denominator and the
              // block length are corrected together, and both routes update one row max, row sum
              // and accumulator). The block counts as n_j copies of (kbar_j, vbar_j) with the route
              // score r_j: m' = max(m, r_j), then l and both accumulators are rescaled by
              // exp(m - m') and gain w = n_j exp(r_j - m') and w vbar_j.
              const double r_j = sol_r[kb], rb = amb_bound ? sol_rb[kb] : 0.0;
              const double n_j = static_cast<double>(std::min<int64_t>(64, N - 64 * kb));
              if (amb_bound && r_j > m) dm_run = std::max(rb, (m > r_j - 4.0 * rb) ? dm_run : 0.0);
              const double m_new = std::max(m, r_j);
              const double alpha = (m == -std::numeric_limits<double>::infinity()) ? 0.0 : std::exp(m - m_new);
              const double w = n_j * std::exp(r_j - m_new);
              for (int d = 0; d < D; d++) {
                acc[d] *= alpha;
                accS[d] = alpha * accS[d] + w * bf16_value(sol->vsum[(bh * NB + kb) * D + d]);
              }
              l = alpha * l + w;
              if (amb_bound) {
                // the device evaluates r_j within rb on the matrix cores, so w within a factor
                // exp(+-rb); its summary product runs on BF16 matrix cores with the weight split
                // into two BF16 parts (relative error below 2^-16). In the S-scaled units of amb_v.
                const double e = S * w * (2.0 * rb + std::ldexp(1.0, -14));
                for (int d = 0; d < D; d++) {
                  amb_v[d] = alpha * amb_v[d] + e * std::fabs(bf16_value(sol->vsum[(bh * NB + kb) * D + d]));
                  amb_pv[d] *= alpha;
                }
                amb_l = alpha * amb_l + e;
                amb_lx *= alpha;
              }
              m = m_new;
              continue;
            }
            double mblk = -std::numeric_limits<double>::infinity();
            for (int t = 0; t < 64; t++) {
              const int64_t kk = kb * 64 + t;
              kv_ok[t] = key_valid(kk);
              dx[t] = 0.0;
              if (kv_ok[t]) {
                x[t] = logit(kk);
                mblk = std::max(mblk, x[t]);
                if (amb_bound) dx[t] = qk_err(kk);
              }
            }
            const double m_new = std::max(m, mblk);
            if (m_new == -std::numeric_limits<double>::infinity()) continue;  // nothing valid yet
            if (amb_bound && mblk > m) {
              // the running max now comes from this block: its error is that of the keys that
              // may hold the maximum within their own error bounds
              double dmb = 0.0;
              for (int t = 0; t < 64; t++)
                if (kv_ok[t] && x[t] + 2.0 * dx[t] >= mblk - 2.0 * dm_run) dmb = std::max(dmb, dx[t]);
              dm_run = std::max(dmb, (m > mblk - 4.0 * dmb) ? dm_run : 0.0);
            }
            const double alpha = (m == -std::numeric_limits<double>::infinity()) ? 0.0
                                                                                 : std::exp(m - m_new);
            double r = 0.0;
            for (double& a : amb_v) a *= alpha;
            for (double& a : amb_pv) a *= alpha;
            amb_l *= alpha;
            amb_lx *= alpha;
            for (int t = 0; t < 64; t++) {
              pv[t] = 0.0;
              if (!kv_ok[t]) continue;
              const double p = std::exp(x[t] - m_new);
              if (mode == 1) {
                pv[t] = p;
                r += p;
              } else if (expcast) {
                const double z = (x[t] - m_new) * log2e + std::log2(S);
                const float tf = static_cast<float>(8.0 * z + 56.0 - 0.35);
                double c = std::nearbyint(static_cast<double>(tf));
                c = std::min(126.0, std::max(0.0, c));
                const uint8_t code = static_cast<uint8_t>(c);
                pv[t] = code_value[code] / (mode == 2 ? S : 1.0);
                r += code_value[code] / S;
                if (code == 0 && p > 0.0) n_under++;
                if (amb_bound) {
                  const double eta = std::ldexp(1.0, -20) *
                                     (std::fabs(x[t]) + std::fabs(m_new) + std::fabs(std::log(S)) + 1.0) +
                                     dx[t] + dm_run;
                  // the nearest half-integer: within the window, rint may give either side
                  const double half = std::floor(static_cast<double>(tf)) + 0.5;
                  if (std::fabs(static_cast<double>(tf) - half) <= 8.0 * log2e * eta) {
                    const double c1 = std::min(126.0, std::max(0.0, half - 0.5));
                    const double c2 = std::min(126.0, std::max(0.0, half + 0.5));
                    const double step = std::fabs(code_value[static_cast<int>(c2)] -
                                                  code_value[static_cast<int>(c1)]);
                    if (step > 0.0) {
                      for (int d = 0; d < D; d++) amb_v[d] += step * vabs(kb * 64 + t, d);
                      amb_l += step;
                    }
                  }
                }
              } else {
                const float sp = static_cast<float>(S * p);
                const uint8_t code = e4m3_code(static_cast<double>(sp));
                pv[t] = code_value[code] / (mode == 2 ? S : 1.0);
                r += p;
                if (code == 0 && p > 0.0) n_under++;
                if (amb_bound && sp > 0.0f) {
                  const double eta = std::ldexp(1.0, -20) *
                                     (std::fabs(x[t]) + std::fabs(m_new) + std::fabs(std::log(S)) + 1.0) +
                                     dx[t] + dm_run;
                  // the nearest rounding boundary (midpoint to the neighbouring code on the
                  // side of S p): within the relative window, either code may result
                  const double cv = code_value[code];
                  const double nb = static_cast<double>(sp) >= cv
                                        ? (code < 0x7E ? code_value[code + 1] : cv)
                                        : (code > 0 ? code_value[code - 1] : cv);
                  const double mid = 0.5 * (cv + nb);
                  if (nb != cv && std::fabs(static_cast<double>(sp) - mid) <= eta * static_cast<double>(sp))
                    for (int d = 0; d < D; d++) amb_v[d] += std::fabs(nb - cv) * vabs(kb * 64 + t, d);
                }
              }
            }
            l = alpha * l + r;
            if (amb_bound && mode == 3)
              for (int t = 0; t < 64; t++)
                if (kv_ok[t]) amb_lx += std::exp(x[t] - m_new) * (dx[t] + dm_run);
            if (amb_bound && mode == 3) {
              // the PV contraction truncates within groups of 8 consecutive keys the same way
              for (int d = 0; d < D; d++)
                for (int g = 0; g < 64; g += 8) {
                  double gm = 0.0;
                  for (int t = g; t < g + 8; t++)
                    if (kv_ok[t]) gm = std::max(gm, std::fabs(pv[t]) * vabs(kb * 64 + t, d));
                  amb_pv[d] += std::ldexp(gm, -11);
                }
            }
            for (int d = 0; d < D; d++) {
              double s = 0.0;
              for (int t = 0; t < 64; t++)
                if (kv_ok[t]) s += pv[t] * value(kb * 64 + t, d);
              acc[d] = alpha * acc[d] + s;
              accS[d] *= alpha;
            }
            if (vsmooth) {
              const int64_t j = kb / 2;
              for (int d = 0; d < D; d++)
                accM[d] = alpha * accM[d] + r * bf16_value(v_mean[(bh * NB128 + j) * D + d]);
            }
            m = m_new;
          }
          Pass ps;
          ps.o.assign(D, 0.0);
          ps.amb.assign(D, 0.0);
          for (int d = 0; d < D; d++) {
            if (mode == 3) {
              const double sv = static_cast<double>(v_scale[bh * D + d]);
              ps.o[d] = vsmooth ? ((sv / S) * acc[d] + accM[d]) / l : acc[d] * sv / (S * l) + accS[d] / l;
            } else {
              ps.o[d] = acc[d] / l;  // mode 2 already divided P by S
            }
          }
          if (amb_bound)
            for (int d = 0; d < D; d++)
              ps.amb[d] = (amb_v[d] + amb_l * std::fabs(ps.o[d]) + amb_pv[d]) / (S * l) +
                          2.0 * std::fabs(ps.o[d]) * amb_lx / l;
          ps.m = m;
          ps.l = l;
          ps.lx = amb_lx / l;
          ps.n_under = n_under;
          return ps;
        };

        // Split-KV ([TF] long-sequence split-KV: the KV sequence is cut into pieces that run
        // their own online softmax, merged by log-sum-exp). Reading: dense rows only; the cuts
        // sit at absolute multiples of L = 2 * ceil(NB / (2 * kv_splits)) blocks (whole 128-row
        // V blocks); each piece keeps the row's KV order; piece s gives o_s, m_s, l_s and
        // O = sum_s w_s o_s / sum_s w_s with w_s = l_s * exp(m_s - max m).
        std::vector<Pass> parts;
        if (sol) {
          // Sol routing ([TF] "Sol Routing" and "SM90 CuTe Mainloop"): one pass, one state. The
          // mainloop takes the KV blocks in route groups of 64 (the K-summary groups its route QK
          // runs on); the non-exact columns of a group's route scores are consumed as summary
          // contributions, then the group's exact tiles run. Reading: groups in KV order, and
          // inside a group first its summary blocks, then its exact blocks, each in KV order.
          std::vector<int64_t> seq;
          const int64_t NBg = ceil_div(NB, 64);
          for (int64_t gi = 0; gi < NBg; gi++) {
            const int64_t g = kv_reverse ? NBg - 1 - gi : gi;
            for (int pass = 0; pass < 2; pass++)
              for (const int64_t kb : blocks)
                if (kb / 64 == g && sol_exact(kb) == (pass == 1)) seq.push_back(kb);
          }
          parts.push_back(stream(seq));
        } else if (kv_splits <= 1 || sparse) {
          parts.push_back(stream(blocks));
        } else {
          const int64_t L = 2 * ceil_div(NB, 2 * static_cast<int64_t>(kv_splits));
          for (int64_t lo = 0; lo < NB; lo += L) {
            std::vector<int64_t> piece;
            for (const int64_t kb : blocks)
              if (kb >= lo && kb < lo + L) piece.push_back(kb);
            parts.push_back(stream(piece));
          }
        }
        if (parts.size() == 1) {
          for (int d = 0; d < D; d++) o[d] = parts[0].o[d];
          if (amb_bound)
            for (int d = 0; d < D; d++) amb_bound[o_idx * D + d] = parts[0].amb[d];
          if (underflow) underflow[o_idx] = parts[0].n_under;
        } else {
          double mmax = -std::numeric_limits<double>::infinity();
          for (const Pass& ps : parts) mmax = std::max(mmax, ps.m);
          std::vector<double> w(parts.size());
          double wsum = 0.0;
          int64_t n_under = 0;
          for (size_t sidx = 0; sidx < parts.size(); sidx++) {
            w[sidx] = parts[sidx].l * std::exp(parts[sidx].m - mmax);
            wsum += w[sidx];
            n_under += parts[sidx].n_under;
          }
          for (int d = 0; d < D; d++) {
            double acc_o = 0.0;
            for (size_t sidx = 0; sidx < parts.size(); sidx++) acc_o += w[sidx] * parts[sidx].o[d];
            o[d] = acc_o / wsum;
          }
          // each piece's bound, plus the change of its weight that its row-sum bound allows
          if (amb_bound)
            for (int d = 0; d < D; d++) {
              double a = 0.0;
              for (size_t sidx = 0; sidx < parts.size(); sidx++)
                a += w[sidx] / wsum *
                     (parts[sidx].amb[d] + 2.0 * parts[sidx].lx * (std::fabs(parts[sidx].o[d]) + std::fabs(o[d])));
              amb_bound[o_idx * D + d] = a;
            }
          if (underflow) underflow[o_idx] = n_under;
        }
          // sequence-mean smoothing ([TF] MiniMax-H3 section): each softmax row sums to 1, so
          // the attention of the shifted V plus mean_T(V) is the attention of V
          if (mode == 3 && v_shift)
            for (int d = 0; d < D; d++) o[d] += static_cast<double>(v_shift[bh * D + d]);
        }
        if (out_bf16)
          for (int d = 0; d < D; d++) out_bf16[o_idx * D + d] = bf16_bits(static_cast<float>(o[d]));
      }
    }
  }
  return 0;
}

// ---------------------------------------------------------------------------------------
// 3D sliding-tile layout ([FPS] 2.2: non-overlapping 3D tiles T_u; the query tile u attends
// to the key tiles v with ||c_u - c_v||_inf within the window; 3.1: the same tile drives the
// quantisation blocks). The raster grid (T, Hg, W) is padded up to whole tiles (tt, th, tw);
// tiles are numbered in raster order over the tile grid; inside a tile the valid tokens come
// first in raster order, then the padding. Per-dimension Chebyshev radius (rt, rh, rw).
// Outputs: perm[n_tiles * tile] source token or -1; tile_len[n_tiles]; row_ptr[n_tiles + 1];
// col_idx[nnz] (ascending per row; caller sizes it n_tiles * n_tiles); *nnz.
// ---------------------------------------------------------------------------------------
int orc_sta_layout(int T, int Hg, int W, int tt, int th, int tw, int rt, int rh, int rw,
                   int32_t* perm, int32_t* tile_len, int32_t* row_ptr, int32_t* col_idx,
                   int32_t* nnz) {
  if (T < 1 || Hg < 1 || W < 1 || tt < 1 || th < 1 || tw < 1 || rt < 0 || rh < 0 || rw < 0)
    return 1;
  const int nt = static_cast<int>(ceil_div(T, tt)), nh = static_cast<int>(ceil_div(Hg, th)),
            nw = static_cast<int>(ceil_div(W, tw));
  const int tile = tt * th * tw, n_tiles = nt * nh * nw;
  for (int a = 0; a < nt; a++)
    for (int c = 0; c < nh; c++)
      for (int e = 0; e < nw; e++) {
        const int u = (a * nh + c) * nw + e;
        int pos = 0;
        for (int t = a * tt; t < a * tt + tt; t++)
          for (int y = c * th; y < c * th + th; y++)
            for (int x = e * tw; x < e * tw + tw; x++)
              if (t < T && y < Hg && x < W) perm[u * tile + pos++] = (t * Hg + y) * W + x;
        tile_len[u] = pos;
        while (pos < tile) perm[u * tile + pos++] = -1;
      }
  int count = 0;
  for (int u = 0; u < n_tiles; u++) {
    row_ptr[u] = count;
    const int ua = u / (nh * nw), uc = (u / nw) % nh, ue = u % nw;
    for (int v = 0; v < n_tiles; v++) {
      const int va = v / (nh * nw), vc = (v / nw) % nh, ve = v % nw;
      if (std::abs(ua - va) <= rt && std::abs(uc - vc) <= rh && std::abs(ue - ve) <= rw)
        col_idx[count++] = v;
    }
  }
  row_ptr[n_tiles] = count;
  *nnz = count;
  return 0;
}

// ---------------------------------------------------------------------------------------
// V-Smooth clustering ([VC] 二 step 1: light online clustering on a few representative
// dimensions; same-cluster tokens made contiguous; clusters need not be balanced).
// Readings where the pages are silent: features = the n_feat channels of V with the largest
// variance over tokens (ties to the lower channel); k-means with n_clusters centroids
// initialised at tokens floor((2c+1) N / (2 n_clusters)); iters Lloyd rounds of (assign,
// update) in FP64 with squared L2 distance summed over the features in ascending channel
// order, ties to the lower cluster id, empty clusters keep their centroid; a final assignment
// with the last centroids; perm = tokens stably sorted by cluster id. Output perm [B, H, N]
// and, if non-null, labels [B, H, N] (cluster id of each source token).
// ---------------------------------------------------------------------------------------
int orc_vsmooth_perm(int B, int N, int H, int D, const uint16_t* v, int n_clusters, int n_feat,
                     int iters, int32_t* perm, int32_t* labels) {
  if (B < 1 || N < 1 || H < 1 || D < 1 || n_clusters < 1 || n_feat < 1 || n_feat > D ||
      iters < 0)
    return 1;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; b++) {
    for (int h = 0; h < H; h++) {
      auto val = [&](int64_t t, int d) -> double {
        return bf16_value(v[((static_cast<int64_t>(b) * N + t) * H + h) * D + d]);
      };
      std::vector<double> var(D);
      for (int d = 0; d < D; d++) {
        double s = 0.0;
        for (int64_t t = 0; t < N; t++) s += val(t, d);
        const double mean = s / N;
        double ss = 0.0;
        for (int64_t t = 0; t < N; t++) ss += (val(t, d) - mean) * (val(t, d) - mean);
        var[d] = ss / N;
      }
      std::vector<int> order(D);
      for (int d = 0; d < D; d++) order[d] = d;
      std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return var[a] > var[c]; });
      std::vector<int> feat(order.begin(), order.begin() + n_feat);
      std::sort(feat.begin(), feat.end());

      std::vector<double> cent(static_cast<size_t>(n_clusters) * n_feat);
      for (int c = 0; c < n_clusters; c++) {
        const int64_t t0 = (static_cast<int64_t>(2 * c + 1) * N) / (2 * n_clusters);
        for (int f = 0; f < n_feat; f++) cent[c * n_feat + f] = val(t0, feat[f]);
      }
      std::vector<int> label(N, 0);
      auto assign = [&]() {
        for (int64_t t = 0; t < N; t++) {
          int best = 0;
          double bd = std::numeric_limits<double>::infinity();
          for (int c = 0; c < n_clusters; c++) {
            double dist = 0.0;
            for (int f = 0; f < n_feat; f++) {
              const double diff = val(t, feat[f]) - cent[c * n_feat + f];
              dist += diff * diff;
            }
            if (dist < bd) {
              bd = dist;
              best = c;
            }
          }
          label[t] = best;
        }
      };
      for (int it = 0; it < iters; it++) {
        assign();
        std::vector<double> sum(static_cast<size_t>(n_clusters) * n_feat, 0.0);
        std::vector<int64_t> cnt(n_clusters, 0);
        for (int64_t t = 0; t < N; t++) {
          cnt[label[t]]++;
          for (int f = 0; f < n_feat; f++) sum[label[t] * n_feat + f] += val(t, feat[f]);
        }
        for (int c = 0; c < n_clusters; c++)
          if (cnt[c] > 0)
            for (int f = 0; f < n_feat; f++)
              cent[c * n_feat + f] = sum[c * n_feat + f] / static_cast<double>(cnt[c]);
      }
      assign();
      std::vector<int32_t> idx(N);
      for (int64_t t = 0; t < N; t++) idx[t] = static_cast<int32_t>(t);
      std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t c) { return label[a] < label[c]; });
      std::memcpy(perm + (static_cast<int64_t>(b) * H + h) * N, idx.data(), sizeof(int32_t) * N);
      if (labels)
        for (int64_t t = 0; t < N; t++) labels[(static_cast<int64_t>(b) * H + h) * N + t] = label[t];
    }
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
