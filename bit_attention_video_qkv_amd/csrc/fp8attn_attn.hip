// FP8 (OCP E4M3) attention forward mainloop for gfx950.
//
// What is computed (TeleFuser blog "FP8 Sol-Attn: H100 视频 DiT 的量化稀疏注意力", section
// "SM90 CuTe Mainloop"; P-cast paper sections 二/三; VC-Attention article sections 二/三):
// E4M3 QK^T with FP32 accumulation, scaled back by s_q * s_k; an online softmax whose running
// max moves once per 64-key block in the requested KV order; P = S * exp(x - m) cast to E4M3
// (or the ExpCast byte); E4M3 PV against token-contiguous V with FP32 accumulation; the V
// channel scale and 1 / (S l) applied after all PV; BF16 output. Optional STA block-sparse KV
// list (FPSAttention 2.2/3.1) and V-Smooth rank-one mean restore.
//
// gfx950 mapping:
//  * Both contractions use v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> FP32, K = 64 per issue).
//  * QK is computed transposed, S^T = K Q^T: each lane then owns one query column and 32 of
//    the block's 64 keys, so the row max needs one cross-half swap and the row sum none until
//    the end. The K tile rows are read in a permuted order so that lane half h owns the keys
//    [32h, 32h+32) of the block; the E4M3 P bytes of a lane are then exactly the B operand of
//    O^T = V^T P^T, whose A operand is 32 contiguous key bytes of a token-contiguous V row.
//  * O^T accumulators give every lane one query, so the softmax rescale is a per-lane scalar.
//  * K and V tiles (8 KB each per 64 keys) are staged in LDS by direct global->LDS loads,
//    double buffered, with XOR-swizzled 16-byte chunks for conflict-free operand reads.
//  * One wave owns 64 queries (two 32-row sub-tiles sharing every K/V operand read); a
//    workgroup has 4 waves (dense) or 2 waves (sparse, so a workgroup never straddles a
//    384-token query tile). Workgroups are mapped XCD-major so each XCD streams one head's K/V.
#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTileBytes = kBlock * kHeadDim;  // 8 KB: one 64-key K tile or V tile

// Physical 16-byte chunk of logical chunk cc in row `row` of the K tile (8 chunks per row).
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | (((row >> 5) & 1) << 2); }
// Same for the V tile (4 chunks per 64-byte channel row).
__device__ __forceinline__ int swz_v(int d) { return (d >> 1) & 3; }

// Key (row of the K tile) that feeds A-operand row i of key sub-tile t: chosen so that the
// S^T accumulator register r of lane half h holds key 32h + 16t + r.
__device__ __forceinline__ int k_row_of(int t, int i) {
  return 32 * ((i >> 2) & 1) + 16 * t + 4 * (i >> 3) + (i & 3);
}

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float xmax(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xsum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ v8i load_op_lds(const uint8_t* base, int off0, int off1) {
  const uint4 a = *reinterpret_cast<const uint4*>(base + off0);
  const uint4 b = *reinterpret_cast<const uint4*>(base + off1);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm_lgkm() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }
// Workgroup barrier without the release/acquire fence of __syncthreads(): that fence makes the
// compiler wait for every outstanding global->LDS copy, including prefetches meant to stay in
// flight across the barrier. Callers order their own LDS traffic with explicit waits; the
// "memory" clobber keeps the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Iteration state over the key blocks of one query tile.
struct KvCursor {
  int e;    // sparse: CSR entry; dense: block counter
  int bt;   // sparse: block within the KV tile
};

// One workgroup owns WAVES * 32 query rows of one (b, h); each wave owns 32 rows.
//
// Schedule. Key block j is consumed in two phases per wave:
//   M(j): PV of block j-1 (V^T P^T on the matrix cores) and QK of block j (K Q^T), on operands
//         already in registers;
//   V(j): online softmax of block j and its P cast (VALU), during which the wave reads the
//         operands of the next pair from LDS.
// LDS "pair" p (buffer p % 3) holds V tile p-1, K tile p, s_k of block p and its valid key
// count (plus, for V-Smooth, the mean factors of V tile p-1's 128-row block). The first group
// of waves stages pair j+2 by direct global->LDS copies right after its prefetch reads in V(j)
// and waits for it at the end of M(j+1), so no LDS read ever follows a copy it does not need.
// With GROUPS == 2 the second half of the waves runs one phase behind the first half; waves w
// and w + WAVES/2 share a SIMD, so one wave's softmax overlaps the other wave's MFMAs. A barrier
// closes every phase.
template <int WAVES, int GROUPS, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd(AttnParams p) {
  constexpr int kRowsPerWg = WAVES * 32;
  constexpr int kLoaders = (WAVES / GROUPS) * 64;
  constexpr int kMetaOff = 2 * kTileBytes;          // s_k (f32), valid keys (i32)
  constexpr int kMeanOff = kMetaOff + 16;           // V-Smooth mean factors, 128 x f32
  constexpr int kPairBytes = kMeanOff + (VSMOOTH ? kHeadDim * 4 : 0);
  constexpr int kBufs = 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBufs][kPairBytes];

  // ---- work item (XCD-major: dispatch round-robins workgroups over the 8 XCDs) ----
  const int per_xcd = (p.total_work + 7) / 8;
  const int work = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (work >= p.total_work) return;
  const int64_t bh = work / p.n_qtiles;
  const int64_t q0 = static_cast<int64_t>(work % p.n_qtiles) * kRowsPerWg;
  const int64_t b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lh = lane >> 5;   // lane half
  const int l32 = lane & 31;
  const int group = (GROUPS == 2 && wave >= WAVES / 2) ? 1 : 0;
  const bool loader = tid < kLoaders;

  // ---- sparse row of this query tile ----
  int e_begin = 0, e_end = 0, q_valid_len = 0;
  if constexpr (SPARSE) {
    const int u = static_cast<int>(q0 / p.tile_tokens);
    e_begin = p.row_ptr[u];
    e_end = p.row_ptr[u + 1];
    q_valid_len = p.tile_len[u];
    if (static_cast<int>(q0 % p.tile_tokens) >= q_valid_len) return;  // all padding rows
  }

  // ---- key-block sequence ----
  auto nblk_of_tile = [&](int e) -> int {
    const int v = p.col_idx[e];
    return min((p.tile_len[v] + kBlock - 1) / kBlock, p.tile_tokens / kBlock);
  };
  int n_iter = 0;
  if constexpr (SPARSE) {
    for (int e = e_begin; e < e_end; e++) n_iter += nblk_of_tile(e);
  } else {
    n_iter = static_cast<int>(p.NB);
  }
  KvCursor lc;  // the loaders' cursor: the next K block to stage
  if constexpr (SPARSE) {
    lc.e = p.reverse ? e_end - 1 : e_begin;
    lc.bt = (p.reverse && e_end > e_begin) ? nblk_of_tile(e_end - 1) - 1 : 0;
  } else {
    lc.e = 0;
    lc.bt = 0;
  }
  auto block_of = [&](const KvCursor& c, int& limit) -> int64_t {
    if constexpr (SPARSE) {
      const int v = p.col_idx[c.e];
      limit = min(kBlock, p.tile_len[v] - c.bt * kBlock);
      return static_cast<int64_t>(v) * (p.tile_tokens / kBlock) + c.bt;
    } else {
      const int64_t kb = p.reverse ? (p.NB - 1 - c.e) : c.e;
      limit = static_cast<int>(min<int64_t>(kBlock, p.N - kb * kBlock));
      return kb;
    }
  };
  auto advance = [&](KvCursor& c) {
    if constexpr (SPARSE) {
      if (!p.reverse) {
        if (++c.bt >= nblk_of_tile(c.e)) {
          c.e++;
          c.bt = 0;
        }
      } else if (--c.bt < 0) {
        c.e--;
        if (c.e >= e_begin) c.bt = nblk_of_tile(c.e) - 1;
      }
    } else {
      c.e++;
    }
  };
  // Dense V-Smooth: key block j closes its 128-row V block when the next block lies elsewhere.
  auto closes_vblock = [&](int j) -> bool {
    if (j + 1 >= n_iter) return true;
    const int64_t kb = p.reverse ? (p.NB - 1 - j) : j;
    const int64_t kn = p.reverse ? (p.NB - 2 - j) : j + 1;
    return (kb >> 1) != (kn >> 1);
  };

  // ---- staging of pair `pidx` (V tile pidx-1, K tile pidx) into buffer `buf` (loaders only) ----
  // Each loader lane copies fixed 16-byte chunks: its byte offsets inside a K tile and inside a
  // V tile are computed once; per pair only the wave-uniform tile base changes.
  constexpr int kRounds = 512 / kLoaders;
  const uint8_t* kbase = p.k8 + bh * p.N64 * kHeadDim;
  const uint8_t* vbase = p.v8t + bh * kHeadDim * p.N64;
  // fixed extent 4 (>= kRounds): an extent that depends on the template parameters makes the
  // host pass of this toolchain drop the kernel launch stubs
  static_assert(kRounds <= 4, "at least 128 loader threads");
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int r = 0; r < kRounds; r++) {
    const int L = r * kLoaders + tid;
    const int row = L >> 3;
    koff[r] = static_cast<uint32_t>(row * kHeadDim + (((L & 7) ^ swz_k(row)) * 16));
    const int d = L >> 2;
    voff[r] = static_cast<uint32_t>(d * p.N64 + (((L & 3) ^ swz_v(d)) * 16));
  }
  int64_t kb_prev = 0;  // K block of the previous pair (= the V tile of this pair)
  auto stage_pair = [&](int pidx, int buf) {
    uint8_t* lk = &lds[buf][0];
    uint8_t* lv = &lds[buf][kTileBytes];
    int64_t kb = 0;
    if (pidx < n_iter) {
      int limit_k;
      kb = block_of(lc, limit_k);
      const uint8_t* kt = kbase + kb * kTileBytes;
#pragma unroll
      for (int r = 0; r < kRounds; r++)
        __builtin_amdgcn_global_load_lds(kt + koff[r],
                                         (__attribute__((address_space(3))) void*)(lk + (r * kLoaders + wave * 64) * 16),
                                         16, 0, 0);
      if (wave == 0 && lane == 0) {
        __builtin_amdgcn_global_load_lds(p.k_scale + bh * p.NB + kb,
                                         (__attribute__((address_space(3))) void*)(&lds[buf][kMetaOff]), 4, 0, 0);
        *reinterpret_cast<int*>(&lds[buf][kMetaOff + 4]) = limit_k;
      }
      advance(lc);
    }
    if (pidx >= 1) {
      const uint8_t* vt = vbase + kb_prev * kBlock;
#pragma unroll
      for (int r = 0; r < kRounds; r++)
        __builtin_amdgcn_global_load_lds(vt + voff[r],
                                         (__attribute__((address_space(3))) void*)(lv + (r * kLoaders + wave * 64) * 16),
                                         16, 0, 0);
      if constexpr (VSMOOTH) {
        if (wave == 0 && lane < 32)
          __builtin_amdgcn_global_load_lds(p.mu_f + (bh * p.NB128 + (kb_prev >> 1)) * kHeadDim + 4 * lane,
                                           (__attribute__((address_space(3))) void*)(&lds[buf][kMeanOff]), 16, 0, 0);
      }
    }
    kb_prev = kb;
  };

  // ---- Q operands (B operand of S^T = K Q^T), straight from HBM ----
  const int64_t qrow = q0 + 32 * wave + l32;  // this lane's query row
  v8i qop[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    if (qrow < p.N64) {
      const uint4* g = reinterpret_cast<const uint4*>(p.q8 + (bh * p.N64 + qrow) * kHeadDim + 64 * c + 32 * lh);
      const uint4 a = g[0], bq = g[1];
      qop[c][0] = a.x; qop[c][1] = a.y; qop[c][2] = a.z; qop[c][3] = a.w;
      qop[c][4] = bq.x; qop[c][5] = bq.y; qop[c][6] = bq.z; qop[c][7] = bq.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) qop[c][j] = 0;
    }
  }
  const int64_t qblk = (q0 + 32 * wave) / kBlock;  // the wave's 32 rows lie in one Q block
  const float s_q = qblk < p.NB ? p.q_scale[bh * p.NB + qblk] : 0.0f;

  // ---- per-wave state ----
  v16f oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[dt][r] = 0.0f;
  v16f sacc[2];
  v8i pop;
#pragma unroll
  for (int w = 0; w < 8; w++) pop[w] = 0;
  float m_run = -INFINITY;  // running max, log2 units
  float l_part = 0.0f;      // this lane's 32-key share of the S-scaled row sum
  float r_cur = 0.0f;       // V-Smooth: S-scaled row sum of the open 128-row V block
  float r_done = 0.0f;      // V-Smooth: closed V block awaiting its mean in the next M phase
  bool mean_due = false;    // V-Smooth: r_done holds a closed block (uniform over the wave)
  float s_k = 0.0f;
  int limit = kBlock;
  unsigned long long n_under = 0;

  // Operands of the next M phase, read from LDS during the V phase before it.
  v8i kop[2][2], vop[4];
  float s_k_next = 0.0f;
  int limit_next = kBlock;
  auto read_pair = [&](int pidx) {
    const uint8_t* base = &lds[pidx % kBufs][0];
    if (pidx >= 1) {
#pragma unroll
      for (int dt = 0; dt < 4; dt++) {
        const int d = 32 * dt + l32;
        const int sw = swz_v(d);
        vop[dt] = load_op_lds(base + kTileBytes, d * kBlock + ((2 * lh) ^ sw) * 16,
                              d * kBlock + ((2 * lh + 1) ^ sw) * 16);
      }
    }
    if (pidx < n_iter) {
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int row = k_row_of(t, l32);
        const int sw = swz_k(row);
#pragma unroll
        for (int c = 0; c < 2; c++) {
          const int c0 = 4 * c + 2 * lh;
          kop[t][c] = load_op_lds(base, row * kHeadDim + (c0 ^ sw) * 16, row * kHeadDim + ((c0 + 1) ^ sw) * 16);
        }
      }
      s_k_next = *reinterpret_cast<const float*>(base + kMetaOff);
      limit_next = *reinterpret_cast<const int*>(base + kMetaOff + 4);
    }
  };

  // M(j): PV of block j-1 and QK of block j on the prefetched operands of pair j.
  auto phase_m = [&](int j) {
    if constexpr (VSMOOTH) {
      if (mean_due) {
        const float* mu = reinterpret_cast<const float*>(&lds[j % kBufs][kMeanOff]);
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const float4 m4 = *reinterpret_cast<const float4*>(mu + 32 * dt + 8 * g + 4 * lh);
            oacc[dt][4 * g + 0] = __builtin_fmaf(r_done, m4.x, oacc[dt][4 * g + 0]);
            oacc[dt][4 * g + 1] = __builtin_fmaf(r_done, m4.y, oacc[dt][4 * g + 1]);
            oacc[dt][4 * g + 2] = __builtin_fmaf(r_done, m4.z, oacc[dt][4 * g + 2]);
            oacc[dt][4 * g + 3] = __builtin_fmaf(r_done, m4.w, oacc[dt][4 * g + 3]);
          }
      }
      r_done = 0.0f;
      mean_due = false;
    }
    if (j >= 1) {
#pragma unroll
      for (int dt = 0; dt < 4; dt++) oacc[dt] = mfma_f8(vop[dt], pop, oacc[dt]);
    }
    if (j < n_iter) {
      s_k = s_k_next;
      limit = limit_next;
#pragma unroll
      for (int t = 0; t < 2; t++) {
        v16f z;
#pragma unroll
        for (int r = 0; r < 16; r++) z[r] = 0.0f;
        sacc[t] = mfma_f8(kop[t][0], qop[0], z);
        sacc[t] = mfma_f8(kop[t][1], qop[1], sacc[t]);
      }
    }
  };

  // V(j): online softmax of block j and its E4M3 P bytes.
  auto phase_v = [&](int j) {
    read_pair(j + 1);
    if (loader && j + 2 <= n_iter) stage_pair(j + 2, (j + 2) % kBufs);
    const float cs = fmaxf(s_q * s_k * p.logit_scale, 1e-30f);  // log2 units per MFMA unit
    float x[32];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) x[16 * t + r] = sacc[t][r];
    if (limit < kBlock) {
#pragma unroll
      for (int q = 0; q < 32; q++)
        if (32 * lh + q >= limit) x[q] = -INFINITY;
    }
    // two chains of three-input maxima
    float mlo = fmaxf(x[0], x[1]), mhi = fmaxf(x[2], x[3]);
#pragma unroll
    for (int q = 4; q < 32; q += 4) {
      mlo = fmaxf(fmaxf(mlo, x[q]), x[q + 1]);
      mhi = fmaxf(fmaxf(mhi, x[q + 2]), x[q + 3]);
    }
    const float mloc = fmaxf(mlo, mhi);
    // every visited block holds a valid key, so the max is finite after the first block; the
    // guard only keeps a fully masked first block from producing NaN
    const float m_cand = fmaxf(m_run, xmax(mloc) * cs);
    const float m_new = m_cand == -INFINITY ? 0.0f : m_cand;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_cand;
    float lsum;
    uint32_t pk[8];
    if constexpr (EXPCAST) {
      const float c8 = 8.0f * cs;
      const float b8 = 8.0f * (p.log2S - m_new) + 55.65f;
      float l4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < 8; w++) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const float tq = __builtin_fmaf(x[4 * w + q], c8, b8);
          const float code = fminf(fmaxf(__builtin_rintf(tq), 0.0f), 126.0f);
          word |= static_cast<uint32_t>(code) << (8 * q);
        }
        pk[w] = word;
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), true);
        l4[w & 3] += (lo[0] + lo[1]) + (hi[0] + hi[1]);
      }
      lsum = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    } else {
      const float bias = p.log2S - m_new;
      float pv[32];
#pragma unroll
      for (int q = 0; q < 32; q++) pv[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[q], cs, bias));
      // tree sum (eight independent chains) keeps the adds off one dependency chain
      float l8[8];
#pragma unroll
      for (int q = 0; q < 8; q++) l8[q] = (pv[q] + pv[q + 8]) + (pv[q + 16] + pv[q + 24]);
      lsum = ((l8[0] + l8[1]) + (l8[2] + l8[3])) + ((l8[4] + l8[5]) + (l8[6] + l8[7]));
#pragma unroll
      for (int w = 0; w < 8; w++) pk[w] = e4m3x4(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
      if constexpr (STATS) {
        if (qrow < p.N) {
#pragma unroll
          for (int q = 0; q < 32; q++)
            n_under += (pv[q] > 0.0f && ((pk[q >> 2] >> (8 * (q & 3))) & 0xFFu) == 0u) ? 1ull : 0ull;
        }
      }
    }
#pragma unroll
    for (int w = 0; w < 8; w++) pop[w] = static_cast<int>(pk[w]);
    l_part = alpha * l_part + lsum;
    if constexpr (VSMOOTH) {
      r_cur = alpha * r_cur + xsum(lsum);
      r_done *= alpha;
      if (closes_vblock(j)) {
        r_done = r_cur;
        r_cur = 0.0f;
        mean_due = true;
      }
    }
    // rescale O only when some row's max moved (alpha == 1 leaves O bit-identical)
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] *= alpha;
    }
  };

  // ---- prologue: pairs 0 and 1 staged, operands of pair 0 in registers ----
  if (loader && n_iter > 0) {
    stage_pair(0, 0);
    stage_pair(1, 1);
  }
  wait_vm();
  __syncthreads();
  read_pair(0);

  // ---- phases. The second group passes one extra barrier first, so its phase k runs beside
  // the first group's phase k + 1 (s_barrier counts arrivals, not program points). ----
  // Hand-offs: a pair staged by the loaders in V(j-1) is complete (copies and the valid-count
  // store) before the barrier that ends M(j); every LDS read of a buffer is consumed by an MFMA
  // (so complete) at least one barrier before the loaders overwrite that buffer.
  if (group == 1) barrier_nofence();
  for (int j = 0; j < n_iter; j++) {
    phase_m(j);
    if (loader) wait_vm_lgkm();  // pair j+1, staged during V(j-1), has landed
    barrier_nofence();
    phase_v(j);
    barrier_nofence();
  }
  phase_m(n_iter);  // PV of the last block
  __syncthreads();
  if (GROUPS == 2 && group == 0) __syncthreads();

  if constexpr (STATS) {
    unsigned long long tot = n_under;
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (lane == 0 && tot) atomicAdd(p.underflow + bh, tot);
  }

  // ---- epilogue: O = acc * g_d / l', BF16, scattered to the destination rows ----
  bool ok = qrow < p.N;
  if constexpr (SPARSE) ok = ok && static_cast<int>(qrow % p.tile_tokens) < q_valid_len;
  const float l_tot = xsum(l_part);
  int64_t dst = qrow;
  if (ok && p.out_rows) dst = p.out_rows[qrow];
  ok = ok && dst >= 0 && dst < p.n_out;
  if (ok) {
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = p.out + ((b * p.n_out + dst) * p.H + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int d0 = 32 * dt + 8 * g + 4 * lh;
        const float4 sv = *reinterpret_cast<const float4*>(p.v_scale + bh * kHeadDim + d0);
        float gs[4] = {sv.x, sv.y, sv.z, sv.w};
        if constexpr (VSMOOTH) {
#pragma unroll
          for (int e = 0; e < 4; e++) gs[e] = gs[e] > 0.0f ? gs[e] : 1.0f;
        }
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * g + 0] * gs[0] * inv_l)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * g + 1] * gs[1] * inv_l)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * g + 2] * gs[2] * inv_l)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(oacc[dt][4 * g + 3] * gs[3] * inv_l)) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = o;
      }
  }
}

// V-Smooth: mu_f[bh, j, d] = float(mean_hat[bh, j, d]) * (s_r[d] > 0 ? 1 / s_r[d] : 1).
__global__ __launch_bounds__(128) void vsmooth_mean_factors(AttnParams p) {
  const int64_t j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int d = threadIdx.x;
  const float sr = p.v_scale[bh * kHeadDim + d];
  const float f = sr > 0.0f ? __fdiv_rn(1.0f, sr) : 1.0f;
  const int64_t idx = (bh * p.NB128 + j) * kHeadDim + d;
  p.mu_f[idx] = bf16_to_f32(p.v_mean[idx]) * f;
}

template <int WAVES, int GROUPS, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS>
hipError_t launch_variant(AttnParams& p, hipStream_t stream) {
  const int rows = WAVES * 32;
  p.n_qtiles = static_cast<int>((p.N + rows - 1) / rows);
  p.total_work = p.B * p.H * p.n_qtiles;
  const unsigned grid = static_cast<unsigned>(((p.total_work + 7) / 8) * 8);
  hipLaunchKernelGGL((attn_fwd<WAVES, GROUPS, SPARSE, EXPCAST, VSMOOTH, STATS>), dim3(grid), dim3(WAVES * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(AttnParams p, int variant, hipStream_t stream) {
  const bool ec = variant & kVarExpCast, vs = variant & kVarVSmooth, sp = variant & kVarSparse,
             st = variant & kVarStats;
  if (vs) {
    hipLaunchKernelGGL(vsmooth_mean_factors, dim3(static_cast<unsigned>(p.NB128), static_cast<unsigned>(p.B * p.H)),
                       dim3(kHeadDim), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Dense: 8 waves of 32 queries in two ping-pong groups. Sparse: a workgroup stays inside one
  // query tile (128 or 64 rows) and runs a single group.
  if (sp && p.tile_tokens % 128 == 0) {
    if (st) return launch_variant<4, 1, true, false, false, true>(p, stream);
    if (ec) return launch_variant<4, 1, true, true, false, false>(p, stream);
    return launch_variant<4, 1, true, false, false, false>(p, stream);
  }
  if (sp) {
    if (st) return launch_variant<2, 1, true, false, false, true>(p, stream);
    if (ec) return launch_variant<2, 1, true, true, false, false>(p, stream);
    return launch_variant<2, 1, true, false, false, false>(p, stream);
  }
  if (vs) {
    if (st) return launch_variant<8, 2, false, false, true, true>(p, stream);
    if (ec) return launch_variant<8, 2, false, true, true, false>(p, stream);
    return launch_variant<8, 2, false, false, true, false>(p, stream);
  }
  if (st) return launch_variant<8, 2, false, false, false, true>(p, stream);
  if (ec) return launch_variant<8, 2, false, true, false, false>(p, stream);
  return launch_variant<8, 2, false, false, false, false>(p, stream);
}

}  // namespace fp8attn
