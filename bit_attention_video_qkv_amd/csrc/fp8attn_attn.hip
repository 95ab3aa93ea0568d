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

// Iteration state over the key blocks of one query tile.
struct KvCursor {
  int e;    // sparse: CSR entry; dense: block counter
  int bt;   // sparse: block within the KV tile
};

template <int WAVES, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS>
__global__ __launch_bounds__(WAVES * 64, 1) void attn_fwd(AttnParams p) {
  constexpr int kThreads = WAVES * 64;
  constexpr int kRowsPerWg = WAVES * 64;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kTileBytes];  // [buf][K | V]

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

  // ---- sparse row of this query tile ----
  int u = 0, e_begin = 0, e_end = 0, q_valid_len = 0;
  if constexpr (SPARSE) {
    u = static_cast<int>(q0 / p.tile_tokens);
    e_begin = p.row_ptr[u];
    e_end = p.row_ptr[u + 1];
    q_valid_len = p.tile_len[u];
    if (static_cast<int>(q0 % p.tile_tokens) >= q_valid_len) return;  // all padding rows
  }

  // Block sequence helpers.
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
  // Cursor at iteration 0 and its advance; returns (block index, valid keys in block).
  KvCursor cur;
  if constexpr (SPARSE) {
    if (!p.reverse) {
      cur.e = e_begin;
      cur.bt = 0;
    } else {
      cur.e = e_end - 1;
      cur.bt = nblk_of_tile(e_end - 1) - 1;
    }
  } else {
    cur.e = 0;
    cur.bt = 0;
  }
  auto block_of = [&](const KvCursor& c, int& limit) -> int64_t {
    if constexpr (SPARSE) {
      const int v = p.col_idx[c.e];
      const int len = p.tile_len[v];
      limit = min(kBlock, len - c.bt * kBlock);
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
      } else {
        if (--c.bt < 0) {
          c.e--;
          if (c.e >= e_begin) c.bt = nblk_of_tile(c.e) - 1;
        }
      }
    } else {
      c.e++;
    }
  };

  // ---- global -> LDS staging of one K tile and one V tile ----
  const uint8_t* kbase = p.k8 + bh * p.N64 * kHeadDim;
  const uint8_t* vbase = p.v8t + bh * kHeadDim * p.N64;
  auto issue_tile_loads = [&](int64_t kb, int buf) {
    uint8_t* lk = &lds[buf][0];
    uint8_t* lv = &lds[buf][kTileBytes];
#pragma unroll
    for (int r = 0; r < 512 / kThreads; r++) {
      const int L = r * kThreads + tid;
      const int row = L >> 3;
      const int cc = (L & 7) ^ swz_k(row);
      const uint8_t* g = kbase + (kb * kBlock + row) * kHeadDim + cc * 16;
      __builtin_amdgcn_global_load_lds(
          g, (__attribute__((address_space(3))) void*)(lk + (r * kThreads + wave * 64) * 16),
          16, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 512 / kThreads; r++) {
      const int L = r * kThreads + tid;
      const int d = L >> 2;
      const int cc = (L & 3) ^ swz_v(d);
      const uint8_t* g = vbase + d * p.N64 + kb * kBlock + cc * 16;
      __builtin_amdgcn_global_load_lds(
          g, (__attribute__((address_space(3))) void*)(lv + (r * kThreads + wave * 64) * 16),
          16, 0, 0);
    }
  };

  // ---- Q operands (B operand of S^T = K Q^T), straight from HBM ----
  const int64_t wrow0 = q0 + 64 * wave;  // first query row of this wave (64-aligned)
  v8i qop[2][2];
#pragma unroll
  for (int s = 0; s < 2; s++) {
    const int64_t row = wrow0 + 32 * s + l32;
#pragma unroll
    for (int c = 0; c < 2; c++) {
      if (row < p.N64) {
        const uint4* g = reinterpret_cast<const uint4*>(p.q8 + (bh * p.N64 + row) * kHeadDim + 64 * c + 32 * lh);
        const uint4 a = g[0], bq = g[1];
        qop[s][c][0] = a.x; qop[s][c][1] = a.y; qop[s][c][2] = a.z; qop[s][c][3] = a.w;
        qop[s][c][4] = bq.x; qop[s][c][5] = bq.y; qop[s][c][6] = bq.z; qop[s][c][7] = bq.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; j++) qop[s][c][j] = 0;
      }
    }
  }
  const int64_t qblk = wrow0 / kBlock;
  const float s_q = qblk < p.NB ? p.q_scale[bh * p.NB + qblk] : 0.0f;

  // ---- accumulators and softmax state ----
  v16f oacc[2][4];
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
      for (int r = 0; r < 16; r++) oacc[s][dt][r] = 0.0f;
  float m_run[2] = {-INFINITY, -INFINITY};  // running max, log2 units
  float l_part[2] = {0.0f, 0.0f};           // this lane's 32-key share of the S-scaled row sum
  float r_pend[2] = {0.0f, 0.0f};           // V-Smooth: pending S-scaled row sum of V block
  unsigned long long n_under = 0;

  if (n_iter > 0) {
    int lim0;
    issue_tile_loads(block_of(cur, lim0), 0);
  }

  for (int it = 0; it < n_iter; it++) {
    int limit;
    const int64_t kb = block_of(cur, limit);
    KvCursor nxt = cur;
    advance(nxt);
    wait_vm();
    __syncthreads();
    if (it + 1 < n_iter) {
      int lim_n;
      issue_tile_loads(block_of(nxt, lim_n), (it + 1) & 1);
    }
    const uint8_t* lk = &lds[it & 1][0];
    const uint8_t* lv = &lds[it & 1][kTileBytes];

    // S^T = K Q^T for both query sub-tiles; K operands read once, used twice.
    v16f sacc[2][2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = k_row_of(t, l32);
      const int sw = swz_k(row);
#pragma unroll
      for (int c = 0; c < 2; c++) {
        const int c0 = 4 * c + 2 * lh;
        const v8i kop = load_op_lds(lk, row * kHeadDim + ((c0) ^ sw) * 16,
                                    row * kHeadDim + ((c0 + 1) ^ sw) * 16);
#pragma unroll
        for (int s = 0; s < 2; s++) {
          if (c == 0) {
            v16f z;
#pragma unroll
            for (int r = 0; r < 16; r++) z[r] = 0.0f;
            sacc[s][t] = mfma_f8(kop, qop[s][0], z);
          } else {
            sacc[s][t] = mfma_f8(kop, qop[s][1], sacc[s][t]);
          }
        }
      }
    }

    const float s_k = p.k_scale[bh * p.NB + kb];
    const float cs = fmaxf(s_q * s_k * p.logit_scale, 1e-30f);  // log2-unit logit per MFMA unit

    // ---- online softmax and P cast per sub-tile ----
    v8i pop[2];
#pragma unroll
    for (int s = 0; s < 2; s++) {
      float x[32];
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) x[16 * t + r] = sacc[s][t][r];
      if (limit < kBlock) {
#pragma unroll
        for (int j = 0; j < 32; j++)
          if (32 * lh + j >= limit) x[j] = -INFINITY;
      }
      float mloc = x[0];
#pragma unroll
      for (int j = 1; j < 32; j++) mloc = fmaxf(mloc, x[j]);
      // every visited block holds a valid key, so m_new is finite after the first block;
      // the guard only keeps a fully masked first block from producing NaN
      const float m_cand = fmaxf(m_run[s], xmax(mloc) * cs);
      const float m_new = m_cand == -INFINITY ? 0.0f : m_cand;
      const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
      m_run[s] = m_cand;
      float lsum = 0.0f;
      uint32_t pk[8];
      if constexpr (EXPCAST) {
        const float c8 = 8.0f * cs;
        const float b8 = 8.0f * (p.log2S - m_new) + 55.65f;
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
          lsum += (lo[0] + lo[1]) + (hi[0] + hi[1]);
        }
      } else {
        const float bias = p.log2S - m_new;
        float pv[32];
#pragma unroll
        for (int j = 0; j < 32; j++) {
          pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], cs, bias));
          lsum += pv[j];
        }
#pragma unroll
        for (int w = 0; w < 8; w++) pk[w] = e4m3x4(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
        if constexpr (STATS) {
          const int64_t row = wrow0 + 32 * s + l32;
          if (row < p.N) {
#pragma unroll
            for (int j = 0; j < 32; j++)
              n_under += (pv[j] > 0.0f && ((pk[j >> 2] >> (8 * (j & 3))) & 0xFFu) == 0u) ? 1ull : 0ull;
          }
        }
      }
#pragma unroll
      for (int w = 0; w < 8; w++) pop[s][w] = static_cast<int>(pk[w]);
      l_part[s] = alpha * l_part[s] + lsum;
      if constexpr (VSMOOTH) r_pend[s] = alpha * r_pend[s] + xsum(lsum);
      // rescale O only when some row's max moved (alpha == 1 leaves O bit-identical)
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
          for (int r = 0; r < 16; r++) oacc[s][dt][r] *= alpha;
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < 4; dt++) {
      const int d = 32 * dt + l32;
      const int sw = swz_v(d);
      const v8i vop = load_op_lds(lv, d * kBlock + ((2 * lh) ^ sw) * 16, d * kBlock + ((2 * lh + 1) ^ sw) * 16);
#pragma unroll
      for (int s = 0; s < 2; s++) oacc[s][dt] = mfma_f8(vop, pop[s], oacc[s][dt]);
    }

    // ---- V-Smooth: add the pending block mean when the 128-row V block changes ----
    if constexpr (VSMOOTH) {
      int lim_x;
      const bool last = (it + 1 >= n_iter);
      const bool flush = last || (block_of(nxt, lim_x) / 2 != kb / 2);
      if (flush) {
        const float* mu = p.mu_f + (bh * p.NB128 + kb / 2) * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
          for (int g = 0; g < 4; g++) {
            const float4 m4 = *reinterpret_cast<const float4*>(mu + 32 * dt + 8 * g + 4 * lh);
#pragma unroll
            for (int s = 0; s < 2; s++) {
              oacc[s][dt][4 * g + 0] = __builtin_fmaf(r_pend[s], m4.x, oacc[s][dt][4 * g + 0]);
              oacc[s][dt][4 * g + 1] = __builtin_fmaf(r_pend[s], m4.y, oacc[s][dt][4 * g + 1]);
              oacc[s][dt][4 * g + 2] = __builtin_fmaf(r_pend[s], m4.z, oacc[s][dt][4 * g + 2]);
              oacc[s][dt][4 * g + 3] = __builtin_fmaf(r_pend[s], m4.w, oacc[s][dt][4 * g + 3]);
            }
          }
        r_pend[0] = 0.0f;
        r_pend[1] = 0.0f;
      }
    }
    cur = nxt;
  }

  if constexpr (STATS) {
    unsigned long long tot = n_under;
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (lane == 0 && tot) atomicAdd(p.underflow + bh, tot);
  }

  // ---- epilogue: O = acc * g_d / l', BF16, scattered to the destination rows ----
#pragma unroll
  for (int s = 0; s < 2; s++) {
    const int64_t row = wrow0 + 32 * s + l32;
    bool ok = row < p.N;
    if constexpr (SPARSE) ok = ok && static_cast<int>(row % p.tile_tokens) < q_valid_len;
    const float l_tot = xsum(l_part[s]);
    int64_t dst = row;
    if (ok && p.out_rows) dst = p.out_rows[row];
    ok = ok && dst >= 0 && dst < p.n_out;
    if (!ok) continue;
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
        o.x = static_cast<uint32_t>(f32_to_bf16_rne(oacc[s][dt][4 * g + 0] * gs[0] * inv_l)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(oacc[s][dt][4 * g + 1] * gs[1] * inv_l)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16_rne(oacc[s][dt][4 * g + 2] * gs[2] * inv_l)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(oacc[s][dt][4 * g + 3] * gs[3] * inv_l)) << 16);
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

template <int WAVES, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS>
hipError_t launch_variant(AttnParams& p, hipStream_t stream) {
  const int rows = WAVES * 64;
  p.n_qtiles = static_cast<int>((p.N + rows - 1) / rows);
  p.total_work = p.B * p.H * p.n_qtiles;
  const unsigned grid = static_cast<unsigned>(((p.total_work + 7) / 8) * 8);
  hipLaunchKernelGGL((attn_fwd<WAVES, SPARSE, EXPCAST, VSMOOTH, STATS>), dim3(grid), dim3(WAVES * 64), 0,
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
  if (sp && p.tile_tokens % 128 == 0) {
    if (st) return launch_variant<2, true, false, false, true>(p, stream);
    if (ec) return launch_variant<2, true, true, false, false>(p, stream);
    return launch_variant<2, true, false, false, false>(p, stream);
  }
  if (sp) {  // tiles of an odd number of 64-token blocks: one wave (64 rows) per workgroup
    if (st) return launch_variant<1, true, false, false, true>(p, stream);
    if (ec) return launch_variant<1, true, true, false, false>(p, stream);
    return launch_variant<1, true, false, false, false>(p, stream);
  }
  if (vs) {
    if (st) return launch_variant<4, false, false, true, true>(p, stream);
    if (ec) return launch_variant<4, false, true, true, false>(p, stream);
    return launch_variant<4, false, false, true, false>(p, stream);
  }
  if (st) return launch_variant<4, false, false, false, true>(p, stream);
  if (ec) return launch_variant<4, false, true, false, false>(p, stream);
  return launch_variant<4, false, false, false, false>(p, stream);
}

}  // namespace fp8attn
