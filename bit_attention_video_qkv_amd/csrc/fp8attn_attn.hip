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
//  * One wave owns 32 queries and software-pipelines them over the key blocks: the softmax of
//    block j (VALU) overlaps the PV MFMAs of block j-1 and the QK MFMAs of block j+1, whose
//    results take over the softmax's registers half by half. The kernel fits two waves per
//    SIMD, so two 4-wave workgroups share every CU and cover each other's stalls.
//  * K and V tiles (8 KB each per 64 keys) reach LDS by direct global->LDS copies, three key
//    blocks deep (two for two-wave workgroups); one barrier per key block. LDS chunks are XOR-swizzled so that every operand
//    read is free of bank conflicts.
//  * Work items are cut into one contiguous range per XCD, so each XCD works on few heads at a
//    time; persistent workgroups take them from per-XCD queues and, when theirs is empty, from
//    the others.
#include <type_traits>

#include "fp8attn_common.h"
#include "fp8attn_internal.h"

namespace fp8attn {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTileBytes = kBlock * kHeadDim;  // 8 KB: one 64-key K tile or V tile

// XOR swizzle of the 16-byte chunks of a K tile row (8 chunks per 128-byte row): logical chunk c
// of row `row` sits at c ^ swz_k(row). Chosen so that each operand read (ds_read_b128, lanes in
// the permuted row order of k_row_of) touches every bank once per group of 8 lanes over 32
// banks and per group of 16 lanes over 64 banks.
__device__ __forceinline__ int swz_k(int row) {
  return ((row >> 1) & 1) | (((row ^ (row >> 2)) & 1) << 1) | (((row >> 5) & 1) << 2);
}
// Same for the V tile (4 chunks per 64-byte channel row), for reads of 32 consecutive channels.
__device__ __forceinline__ int swz_v(int d) { return ((d >> 2) & 1) | ((((d >> 1) ^ (d >> 3)) & 1) << 1); }

// Key (row of the K tile) that feeds A-operand row i of key sub-tile t: chosen so that the
// S^T accumulator register r of lane half h holds key 32h + 16t + r.
__device__ __forceinline__ int k_row_of(int t, int i) {
  return 32 * ((i >> 2) & 1) + 16 * t + 4 * (i >> 3) + (i & 3);
}

__device__ __forceinline__ v16f mfma_f8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ExpCast row sums on the matrix cores: C += A B with B = the wave's E4M3 P bytes (the PV B
// operand: lane l holds query l % 32, keys [32 (l / 32), +32)) read as the B operand of a
// 16x16x128 MFMA, and A a 0/1 selector. Lane group g = l / 16 of either operand carries the
// same quarter of the 128-deep contraction, so output column n sums, over the groups g that row
// m selects, the bytes of lane 16 g + n: query n's keys in groups 0 and 2, query n + 16's in
// groups 1 and 3. Output lane L holds column L % 16 in rows 4 (L / 16) .. +3; selecting groups
// of L's parity, (L / 16) % 2 = (L / 4 of the row) % 2, gives every lane the sum over all 64 keys
// of the query it owns in the PV layout (L % 32), in all four registers.
__device__ __forceinline__ v8i rowsum_selector(int lane) {
  const int sel = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;  // E4M3 1.0 or 0
  v8i a;
#pragma unroll
  for (int w = 0; w < 8; w++) a[w] = sel;
  return a;
}
__device__ __forceinline__ v4f mfma_rowsum(const v8i& sel, const v8i& p8, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, p8, c, 0, 0, 0, 0, 0, 0);
}

// IEEE maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no NaN canonicalisation of
// its inputs; the logits carry no NaN.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float xmax(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xsum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Each byte of a packed word clamped to at most 126, two bytes at a time (v_pk_min_u16 on the
// even and on the odd bytes).
__device__ __forceinline__ uint32_t clamp_bytes_126(uint32_t w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 lim = {126, 126};
  const u16x2 lo = __builtin_elementwise_min(__builtin_bit_cast(u16x2, w & 0x00FF00FFu), lim);
  const u16x2 hi = __builtin_elementwise_min(__builtin_bit_cast(u16x2, (w >> 8) & 0x00FF00FFu), lim);
  return __builtin_bit_cast(uint32_t, lo) | (__builtin_bit_cast(uint32_t, hi) << 8);
}

__device__ __forceinline__ v8i load_op_lds(const uint8_t* base, int off0, int off1) {
  const uint4 a = *reinterpret_cast<const uint4*>(base + off0);
  const uint4 b = *reinterpret_cast<const uint4*>(base + off1);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ void copy4_to_lds(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(gbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

// Instruction interleaving inside one key block. The block is cut into three scheduling regions
// (sched_barrier): (1) PV of the previous block with the operand reads, the row max and the
// exp / convert of the first 32-key half, (2) QK of the next block's first key half with the
// exp / convert of the second half, (3) QK of the second key half. Inside a region every MFMA
// is followed by a run of VALU work long enough to cover its 64-cycle issue on the matrix
// core, so the wave never queues behind its own MFMAs while it has VALU work left.
__device__ __forceinline__ void interleave_region1() {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA (PV)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void interleave_region2() {
#pragma unroll
  for (int i = 0; i < 2; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA (QK, first key half)
    __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);  // VALU
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Dense/sparse key-block cursor of the copy engine.
struct KvCursor {
  int e;     // sparse: CSR entry; dense: block counter
  int bt;    // sparse: block within the KV tile
  int v;     // sparse: KV tile id col_idx[e]
  int len;   // sparse: valid tokens of tile v
  // sparse, loaded ahead so that a tile switch waits on no load: the next tile's id and valid
  // tokens, and the id of the tile after it (entries e + dir and e + 2 dir of the CSR row)
  int v1, len1, v2;
};

// One workgroup owns WAVES * 32 query rows of one (b, h); each wave owns 32 of them.
//
// Schedule of key block j inside a wave (the operands named are already in registers):
//   MFMA:  PV of block j-1 (V(j-1), P(j-1)) first, QK of block j+1 (K(j+1)) last
//   VALU:  online softmax of block j on S(j), producing P(j), in between
//   LDS:   the operands of the next block, V(j) and K(j+1), read from slot "pair j+1" after
//          the MFMAs that consumed the previous values
//   end:   rescale of O by alpha(j) (PV(j-1) long done), wait for pair j+2, barrier, copy
//          pair j+1+kSlots (j+4 with three slots) into the slot just read.
// Pair p (slot p % kSlots) holds the K tile of key block p with its s_k and valid-key count and the
// V tile of key block p-1 (for V-Smooth, with the mean factors of that block's 128-row V block).
// QK(j+1) writes its result into the registers the softmax of block j has just consumed, so a
// wave needs one S tile of registers; two workgroups share each CU, so every SIMD runs two such
// waves whose barriers and dependency stalls cover each other.
// attn_tile computes work item `work` (query tile fastest, then KV piece, then (b, h)); the
// kernel below hands out the items.
template <int WAVES, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS, bool SOL>
__device__ __forceinline__ void attn_tile(const AttnParams& p, const int work) {
  constexpr int kThreads = WAVES * 64;
  constexpr int kRowsPerWg = WAVES * 32;
  // Loops whose waves take turns by phase at the SIMD (see iteration): ExpCast, bound by the
  // matrix cores, and the sparse and V-Smooth paths, whose waves wait more; the plain dense
  // standard cast, bound by its VALU work, ran slower with any such arrangement and keeps one
  // priority throughout.
  constexpr bool kPhasePrio = EXPCAST || SPARSE || VSMOOTH;
  constexpr int kChunks = 512 / kThreads;       // 16-byte chunks per thread of one 8 KB tile
  constexpr int kMetaOff = 2 * kTileBytes;      // s_k (f32) and valid keys (i32) of the K block
  // V-Smooth: the mean operand records of a group of four 128-row V blocks, 128 channels x 32 B
  constexpr int kMeanOff = kMetaOff + 16;
  constexpr int kMeanBytes = VSMOOTH ? kHeadDim * 32 : 0;
  constexpr int kGmaxOff = kMeanOff;            // Sol: the K block's group summary maximum per row
  constexpr int kSlotBytes = kMeanOff + kMeanBytes + (SOL ? kRowsPerWg * 4 : 0);
  constexpr int kMeanLanes = kMeanBytes / 16 / WAVES;  // V-Smooth: lanes per wave copying them
  static_assert(kMeanLanes <= 64, "one 16-byte record chunk per lane");
  // copies every wave issues for every pair (wave 0 adds s_k; V-Smooth pairs may add the mean
  // records, which the waits do not count: they then wait one copy longer than they must)
  constexpr int kCopies = 2 * kChunks;
  // LDS slots of (K, V) pairs: three, two in flight while one is read; two-wave workgroups use
  // two (one in flight), so that four of them fit a CU's LDS instead of three
  constexpr int kSlots = WAVES == 2 ? 2 : 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSlots * kSlotBytes];
  auto slot = [&](int i) -> uint8_t* { return lds + i * kSlotBytes; };
  // the head's V channel scales and output shift, copied in the prologue for the epilogue
  __shared__ __attribute__((aligned(16))) float vsc_s[2 * kHeadDim];

  // ---- work item ----
  const int64_t bh = work / (p.n_qtiles * p.splits);
  const int split = (work / p.n_qtiles) % p.splits;
  const int64_t q0 = static_cast<int64_t>(work % p.n_qtiles) * kRowsPerWg;
  const int64_t b = bh / p.H, h = bh % p.H;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63;
  const int lh = lane >> 5;  // lane half
  const int l32 = lane & 31;

  // ---- sparse row of this query tile ----
  int e_begin = 0, e_end = 0, q_valid_len = 0;
  int q_tile_off = 0;  // first row of the workgroup within its query tile
  if constexpr (SPARSE && !SOL) {
    const int u = static_cast<int>(q0 / p.tile_tokens);
    q_tile_off = static_cast<int>(q0 - static_cast<int64_t>(u) * p.tile_tokens);
    e_begin = load_uniform(p.row_ptr, u);
    e_end = load_uniform(p.row_ptr, u + 1);
    q_valid_len = load_uniform(p.tile_len, u);
    if (q_tile_off >= q_valid_len) return;  // all padding rows
  }
  const int per_tile = p.tile_tokens / kBlock;
  auto nblk_of_len = [&](int len) -> int { return min((len + kBlock - 1) / kBlock, per_tile); };

  // ---- key-block sequence (dense: the piece [kb_lo, kb_hi) of the key blocks, visited in KV
  // order; e0 is its first position in the visiting order) ----
  int n_iter = 0;
  int64_t e0 = 0;
  bool has_last_block = true;  // the piece holds key block NB-1 (the only partial one)
  // Sol: the staged key blocks are the set bits of the workgroup's Q-block mask (four waves: the
  // union of its two Q blocks' masks, and each wave pair masks out the blocks that are not exact
  // for its own Q block), visited in KV order by uniform scans of the mask words
  constexpr bool kSolPair = SOL && WAVES == 4;  // two Q blocks per workgroup (else one)
  const int64_t sol_ua = q0 / kBlock;
  const bool sol_has_b = kSolPair && sol_ua + 1 < p.NB;
  const uint64_t* sol_row_a = SOL ? p.sol_mask + (bh * p.NB + sol_ua) * p.sol_words : nullptr;
  const uint64_t* sol_row_b = SOL && sol_has_b ? sol_row_a + p.sol_words : nullptr;
  const uint64_t* sol_row_mine = (SOL && wave >= 2) ? sol_row_b : sol_row_a;  // null: no Q block
  auto sol_word = [&](int64_t w) -> uint64_t { return sol_row_a[w] | (sol_has_b ? sol_row_b[w] : 0ull); };
  auto sol_next = [&](int64_t pos) -> int64_t {  // first staged block at or after pos, or -1
    if (pos >= p.NB) return -1;
    int64_t w = pos >> 6;
    uint64_t m = sol_word(w) & (~0ull << (pos & 63));
    while (m == 0ull && ++w < p.sol_words) m = sol_word(w);
    return m ? (w << 6) + __builtin_ctzll(m) : -1;
  };
  auto sol_prev = [&](int64_t pos) -> int64_t {  // last staged block at or before pos, or -1
    if (pos < 0) return -1;
    int64_t w = pos >> 6;
    uint64_t m = sol_word(w) & ((pos & 63) == 63 ? ~0ull : ((1ull << ((pos & 63) + 1)) - 1ull));
    while (m == 0ull && --w >= 0) m = sol_word(w);
    return m ? (w << 6) + 63 - __builtin_clzll(m) : -1;
  };
  if constexpr (SOL) {
    for (int64_t w = 0; w < p.sol_words; w++) n_iter += __builtin_popcountll(sol_word(w));
  } else if constexpr (SPARSE) {
    // the row's key blocks, the entries counted by the lanes in parallel (independent loads
    // instead of a chain of dependent scalar ones)
    int cnt = 0;
    for (int e = e_begin + lane; e < e_end; e += 64) cnt += nblk_of_len(p.tile_len[p.col_idx[e]]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    n_iter = __builtin_amdgcn_readfirstlane(cnt);
  } else {
    const int64_t kb_lo = static_cast<int64_t>(split) * p.split_blocks;
    const int64_t kb_hi = min(p.NB, kb_lo + p.split_blocks);
    n_iter = static_cast<int>(kb_hi - kb_lo);
    e0 = p.reverse ? p.NB - kb_hi : kb_lo;
    has_last_block = kb_hi == p.NB;
  }
  if (n_iter <= 0) {
    if constexpr (SOL) {
      // no exact block: the exact route has no weight, so O is the summary route's piece (with
      // the sequence-mean V shift), in BF16
      for (int r = threadIdx.x; r < kRowsPerWg * (kHeadDim / 4); r += kThreads) {
        const int64_t row = q0 + r / (kHeadDim / 4);
        if (row >= p.N) continue;
        const int c = 4 * (r % (kHeadDim / 4));
        const int64_t r1 = bh * p.N + row;
        const float4 o1 = *reinterpret_cast<const float4*>(p.o_part + r1 * kHeadDim + c);
        float4 sh = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (p.v_shift) sh = *reinterpret_cast<const float4*>(p.v_shift + bh * kHeadDim + c);
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16_rne(o1.x + sh.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(o1.y + sh.y)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16_rne(o1.z + sh.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(o1.w + sh.w)) << 16);
        *reinterpret_cast<uint2*>(p.out + ((b * p.n_out + row) * p.H + h) * kHeadDim + c) = o;
      }
    }
    return;  // (otherwise: a query tile without key blocks has no defined output)
  }

  const int edir = p.reverse ? -1 : 1;  // sparse: CSR entries in the KV order
  auto in_row = [&](int e) -> bool { return e >= e_begin && e < e_end; };
  KvCursor lc;  // the copy engine's cursor: the next K block to stage
  lc.e = static_cast<int>(e0);
  lc.bt = 0;
  lc.v = 0;
  lc.len = 0;
  lc.v1 = lc.len1 = lc.v2 = 0;
  if constexpr (SOL) {
    lc.v = static_cast<int>(p.reverse ? sol_prev(p.NB - 1) : sol_next(0));
  } else if constexpr (SPARSE) {
    lc.e = p.reverse ? e_end - 1 : e_begin;
    lc.v = load_uniform(p.col_idx, lc.e);
    lc.len = load_uniform(p.tile_len, lc.v);
    lc.bt = p.reverse ? nblk_of_len(lc.len) - 1 : 0;
    lc.v1 = in_row(lc.e + edir) ? load_uniform(p.col_idx, lc.e + edir) : 0;
    lc.len1 = in_row(lc.e + edir) ? load_uniform(p.tile_len, lc.v1) : 0;
    lc.v2 = in_row(lc.e + 2 * edir) ? load_uniform(p.col_idx, lc.e + 2 * edir) : 0;
  }
  auto block_of = [&](const KvCursor& c, int& limit) -> int64_t {
    if constexpr (SOL) {
      limit = static_cast<int>(min<int64_t>(kBlock, p.N - static_cast<int64_t>(c.v) * kBlock));
      return c.v;
    } else if constexpr (SPARSE) {
      limit = min(kBlock, c.len - c.bt * kBlock);
      return static_cast<int64_t>(c.v) * per_tile + c.bt;
    } else {
      const int64_t kb = p.reverse ? (p.NB - 1 - c.e) : c.e;
      limit = static_cast<int>(min<int64_t>(kBlock, p.N - kb * kBlock));
      return kb;
    }
  };
  auto advance = [&](KvCursor& c) {
    if constexpr (SOL) {
      c.v = static_cast<int>(p.reverse ? sol_prev(c.v - 1) : sol_next(c.v + 1));
    } else if constexpr (SPARSE) {
      const bool next_tile = p.reverse ? --c.bt < 0 : ++c.bt >= nblk_of_len(c.len);
      if (next_tile) {
        c.e += edir;
        if (in_row(c.e)) {
          c.v = c.v1;
          c.len = c.len1;
          c.bt = p.reverse ? nblk_of_len(c.len) - 1 : 0;
          c.v1 = c.v2;
          c.len1 = in_row(c.e + edir) ? load_uniform(p.tile_len, c.v1) : 0;
          c.v2 = in_row(c.e + 2 * edir) ? load_uniform(p.col_idx, c.e + 2 * edir) : 0;
        }
      }
    } else {
      c.e++;
    }
  };
  // Dense V-Smooth: key block j closes its 128-row V block when the next block lies elsewhere.
  auto closes_vblock = [&](int j) -> bool {
    if (j + 1 >= n_iter) return true;
    const int64_t e = e0 + j;
    const int64_t kb = p.reverse ? (p.NB - 1 - e) : e;
    const int64_t kn = p.reverse ? (p.NB - 2 - e) : e + 1;
    return (kb >> 1) != (kn >> 1);
  };
  // The same for blocks that are not the last of the piece: forward, key block kb closes its V
  // block when kb is odd; reverse, when kb is even, i.e. when e = e0 + j has the parity of NB - 1.
  const int close_parity = p.reverse ? static_cast<int>((p.NB - 1) & 1) : 1;
  auto closes_vblock_inner = [&](int j) -> bool { return ((static_cast<int>(e0) + j) & 1) == close_parity; };
  // The mean restore runs once per group of four V blocks (eight key blocks, kb / 8): block j
  // closes its group when the next block lies in another group or j is the piece's last block;
  // in the steady state, when kb % 8 is 7 (forward) or 0 (reverse), i.e. when e = e0 + j has the
  // phase of NB - 1 in reverse.
  auto closes_group = [&](int j) -> bool {
    if (j + 1 >= n_iter) return true;
    const int64_t e = e0 + j;
    const int64_t kb = p.reverse ? (p.NB - 1 - e) : e;
    const int64_t kn = p.reverse ? (p.NB - 2 - e) : e + 1;
    return (kb >> 3) != (kn >> 3);
  };
  const int group_phase = p.reverse ? static_cast<int>((p.NB - 1) & 7) : 7;
  auto closes_group_inner = [&](int j) -> bool { return ((static_cast<int>(e0) + j) & 7) == group_phase; };
  // position of block j's V block in its group (the records' and pending sums' index)
  auto vpos_of = [&](int j) -> int {
    const int64_t e = e0 + j;
    return static_cast<int>(((p.reverse ? (p.NB - 1 - e) : e) >> 1) & 3);
  };

  // ---- staging of pair `pidx` into slot `sl` (every thread copies its fixed 16-byte chunks;
  // per pair only the wave-uniform tile bases change) ----
  const uint8_t* kbase = p.k8 + bh * p.N64 * kHeadDim;
  const uint8_t* vbase = p.v8t + bh * kHeadDim * p.N64;
  // fixed extent 8 (>= kChunks): an extent that depends on the template parameters makes the
  // host pass of this toolchain drop the kernel launch stubs
  static_assert(kChunks <= 8, "at least 64 threads");
  uint32_t koff[8], voff[8];
#pragma unroll
  for (int r = 0; r < kChunks; r++) {
    const int L = r * kThreads + tid;
    const int row = L >> 3;
    koff[r] = static_cast<uint32_t>(row * kHeadDim + (((L & 7) ^ swz_k(row)) * 16));
    const int d = L >> 2;
    voff[r] = static_cast<uint32_t>(d * p.N64 + (((L & 3) ^ swz_v(d)) * 16));
  }
  int64_t kb_prev = 0;  // K block of the previous pair (= the V tile of this pair)
  auto stage = [&](int pidx, uint8_t* sl) {
    int64_t kb = kb_prev;  // pair n_iter carries no K block: its K copy repeats a valid tile
    int limit = kBlock;
    if (pidx < n_iter) {
      kb = block_of(lc, limit);
      advance(lc);
    }
    const int64_t vb = pidx >= 1 ? kb_prev : kb;  // pair 0 carries no V block (same: a valid tile)
    const uint8_t* kt = kbase + kb * kTileBytes;
    const uint8_t* vt = vbase + vb * kBlock;
    const uint32_t l0 = lds_addr_of(sl);
#pragma unroll
    for (int r = 0; r < kChunks; r++) copy16_to_lds(kt, koff[r], l0 + (r * kThreads + wave * 64) * 16);
#pragma unroll
    for (int r = 0; r < kChunks; r++) copy16_to_lds(vt, voff[r], l0 + kTileBytes + (r * kThreads + wave * 64) * 16);
    if constexpr (VSMOOTH) {
      if (lane < kMeanLanes)
        copy16_to_lds(p.mu_op + (bh * ((p.NB128 + 3) >> 2) + (vb >> 3)) * (kMeanBytes / 4),
                      16u * (wave * kMeanLanes + lane), l0 + kMeanOff + wave * kMeanLanes * 16);
    }
    if constexpr (SOL) {
      // the running summary maximum of the K block's route group, for the wave's 32 rows
      if (lane < 32)
        copy4_to_lds(p.sol_gmax + (bh * p.sol_groups + (kb >> 6)) * p.N64 + q0 + 32 * wave, 4u * lane,
                     l0 + kGmaxOff + wave * 128);
    }
    if (wave == 0 && lane == 0) {
      copy4_to_lds(p.k_scale + bh * p.NB + kb, 0u, l0 + kMetaOff);
      *reinterpret_cast<int*>(sl + kMetaOff + 4) = limit;
      if constexpr (kSolPair) *reinterpret_cast<int*>(sl + kMetaOff + 8) = static_cast<int>(kb);
    }
    kb_prev = kb;
  };
  // Dense steady state (a K block and a V block to stage, pair index >= 1): the same pair with
  // less bookkeeping. Wave 0 copies s_k first, so that after its K/V copies every wave has the
  // same number of copies of this pair in flight; the valid-key count is not staged (dense
  // blocks are full except NB-1, whose count is lim_tail).
  // The source pointers move by one tile per pair in the KV order: st_k / st_s at the next K
  // block kb and its s_k, st_v at the V tile of block kb_prev (set by stage_dense_init).
  const int64_t kv_dir = p.reverse ? -1 : 1;
  const uint8_t* st_k = kbase;
  const uint8_t* st_v = vbase;
  const float* st_s = p.k_scale;
  auto stage_dense_init = [&]() {
    const int64_t kb = p.reverse ? (p.NB - 1 - lc.e) : lc.e;
    st_k = kbase + kb * kTileBytes;
    st_v = vbase + kb_prev * kBlock;
    st_s = p.k_scale + bh * p.NB + kb;
  };
  auto stage_dense = [&](uint8_t* sl) {
    const uint32_t l0 = lds_addr_of(sl);
    if (wave == 0 && lane == 0) copy4_to_lds(st_s, 0u, l0 + kMetaOff);
#pragma unroll
    for (int r = 0; r < kChunks; r++) copy16_to_lds(st_k, koff[r], l0 + (r * kThreads + wave * 64) * 16);
#pragma unroll
    for (int r = 0; r < kChunks; r++) copy16_to_lds(st_v, voff[r], l0 + kTileBytes + (r * kThreads + wave * 64) * 16);
    if constexpr (VSMOOTH) {
      // only the restore of the block that closes a group of V blocks reads the records (from
      // the slot of the next pair, which carries that block's V tile); a steady pair's V block
      // never is the last of the piece
      if ((kb_prev & 7) == (kv_dir > 0 ? 7 : 0) && lane < kMeanLanes)
        copy16_to_lds(p.mu_op + (bh * ((p.NB128 + 3) >> 2) + (kb_prev >> 3)) * (kMeanBytes / 4),
                      16u * (wave * kMeanLanes + lane), l0 + kMeanOff + wave * kMeanLanes * 16);
    }
    st_k += kv_dir * kTileBytes;
    st_v += kv_dir * kBlock;
    st_s += kv_dir;
    kb_prev += kv_dir;
    lc.e++;
  };
  // Waits until only the copies of the newest kSlots - 2 staged pairs may still be in flight.
  auto wait_all_but_newest = [&]() {
    if constexpr (kSlots == 2) {
      wait_vmcnt<0>();
    } else {
      if (wave == 0) wait_vmcnt<kCopies + 1>();
      else wait_vmcnt<kCopies>();
    }
  };

  // ---- Q operand (B operand of S^T = K Q^T), straight from HBM ----
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
      for (int w = 0; w < 8; w++) qop[c][w] = 0;
    }
  }
  const int64_t qblk = (q0 + 32 * wave) / kBlock;  // the wave's 32 rows lie in one Q block
  const float s_q = qblk < p.NB ? p.q_scale[bh * p.NB + qblk] : 0.0f;
  const float sq_ls = s_q * p.logit_scale;
  // the output row of the scatter, loaded now so that the epilogue waits on no load
  int32_t out_row = 0;
  if (p.out_rows && qrow < p.N) out_row = p.out_rows[qrow];

  // ---- per-wave state ----
  v16f oacc[4], sacc[2];
#pragma unroll
  for (int dt = 0; dt < 4; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[dt][r] = 0.0f;
  v8i pop;  // E4M3 P bytes (B operand of O^T = V^T P^T)
#pragma unroll
  for (int w = 0; w < 8; w++) pop[w] = 0;
  float m_run = -INFINITY;  // running max, log2 units
  // Standard cast: this lane's 32-key share of the S-scaled row sum. ExpCast: the whole row's
  // S-scaled sum over the closed V blocks (V-Smooth), else unused.
  float l_part = 0.0f;
  float r_cur = 0.0f;       // V-Smooth, standard cast: S-scaled row sum of the open V block
  // V-Smooth: S-scaled row sums of the closed V blocks of the open group that this lane half
  // feeds to the restore (positions 2 lh and 2 lh + 1 in the group), rescaled with O until the
  // group's restore
  float r_pa = 0.0f, r_pb = 0.0f;
  // ExpCast: S-scaled row sums of the P codes accumulated on the matrix cores (lacc[0] in every
  // lane: the lane's whole query row), rescaled with O; with V-Smooth only since the last mean
  // restore.
  const v8i rs_sel = rowsum_selector(lane);
  v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
  unsigned long long n_under = 0;
  v8i kop[2][2], vop[4];
  float sk_cur = 0.0f, sk_next = 0.0f;
  int lim_cur = kBlock, lim_next = kBlock;
  const int lim_tail = static_cast<int>(p.N - (p.NB - 1) * kBlock);  // valid keys of block NB-1
  int kb_next = 0;                      // Sol: key block of the next K tile
  bool ex_cur = false, ex_next = false;  // Sol: that block is not exact for this wave's Q block
  float gm_cur = -INFINITY, gm_next = -INFINITY;  // Sol: summary maximum so far (log2 units)

  // Per-lane byte offsets of the 16-byte operand chunks inside a slot (K rows in the permuted
  // order, swizzled chunks).
  uint32_t kro[8], vro[8];
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const int row = k_row_of(t, l32);
    const int sw = swz_k(row);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      const int c0 = 4 * c + 2 * lh;
      kro[4 * t + 2 * c] = static_cast<uint32_t>(row * kHeadDim + (c0 ^ sw) * 16);
      kro[4 * t + 2 * c + 1] = static_cast<uint32_t>(row * kHeadDim + ((c0 + 1) ^ sw) * 16);
    }
  }
#pragma unroll
  for (int dt = 0; dt < 4; dt++) {
    const int d = 32 * dt + l32;
    const int sw = swz_v(d);
    vro[2 * dt] = static_cast<uint32_t>(kTileBytes + d * kBlock + ((2 * lh) ^ sw) * 16);
    vro[2 * dt + 1] = static_cast<uint32_t>(kTileBytes + d * kBlock + ((2 * lh + 1) ^ sw) * 16);
  }
  auto read_k = [&](const uint8_t* base) {
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int c = 0; c < 2; c++) kop[t][c] = load_op_lds(base, kro[4 * t + 2 * c], kro[4 * t + 2 * c + 1]);
  };
  auto read_v = [&](const uint8_t* base) {
#pragma unroll
    for (int dt = 0; dt < 4; dt++) vop[dt] = load_op_lds(base, vro[2 * dt], vro[2 * dt + 1]);
  };
  auto read_meta = [&](const uint8_t* base) {
    sk_next = *reinterpret_cast<const float*>(base + kMetaOff);
    lim_next = *reinterpret_cast<const int*>(base + kMetaOff + 4);
    if constexpr (SOL) gm_next = *reinterpret_cast<const float*>(base + kGmaxOff + (32 * wave + l32) * 4);
    if constexpr (kSolPair) {
      // looked up one block ahead, so the mask word's load has a whole block to land
      kb_next = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(base + kMetaOff + 8));
      ex_next = sol_row_mine == nullptr || ((sol_row_mine[kb_next >> 6] >> (kb_next & 63)) & 1ull) == 0ull;
    }
  };
  auto qk_half = [&](int t) {
    v16f z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.0f;
    sacc[t] = mfma_f8(kop[t][0], qop[0], z);
    sacc[t] = mfma_f8(kop[t][1], qop[1], sacc[t]);
  };
  auto qk = [&]() {
    qk_half(0);
    qk_half(1);
  };
  auto pv = [&]() {
#pragma unroll
    for (int dt = 0; dt < 4; dt++) oacc[dt] = mfma_f8(vop[dt], pop, oacc[dt]);
  };

  // Orders the QK MFMAs of key sub-tile t of the next block after the P bytes of sub-tile t of
  // this block (a register dependency through an empty asm): the compiler would otherwise issue
  // QK first and keep both S tiles alive, or sink the softmax past the end of the block.
  // The row-sum partial rides along so that its adds stay in this block as well.
  auto tie_k = [&](int t, float& lsum_part) {
    asm volatile("" : "+v"(kop[t][0]), "+v"(kop[t][1]), "+v"(lsum_part) : "v"(pop[4 * t]), "v"(pop[4 * t + 1]),
                 "v"(pop[4 * t + 2]), "v"(pop[4 * t + 3]));
  };

  // Online softmax of block j on the S^T accumulators: updates the running state, writes the
  // E4M3 P bytes into pop and returns alpha.
  auto softmax = [&](auto mask_tag, auto&& issue_qk_half) -> float {
    constexpr bool kMask = decltype(mask_tag)::value;
    // log2 units per MFMA unit; floored above zero where masked keys (-inf) could meet a zero
    // scale (0 * -inf would be NaN)
    const float cs = kMask ? fmaxf(sq_ls * sk_cur, 1e-30f) : sq_ls * sk_cur;
    float x[32];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) x[16 * t + r] = sacc[t][r];
    // two chains of three-input maxima, first over the first key half (whose QK finished first)
    float mlo = fmax_ieee(x[0], x[1]), mhi = fmax_ieee(x[2], x[3]);
#pragma unroll
    for (int q = 4; q < 32; q += 4) {
      mlo = fmax_ieee(fmax_ieee(mlo, x[q]), x[q + 1]);
      mhi = fmax_ieee(fmax_ieee(mhi, x[q + 2]), x[q + 3]);
    }
    const float mloc = fmax_ieee(mlo, mhi);
    // every dense block holds a valid key, so the max is finite from the first block on; the
    // sparse and Sol guard keeps a fully masked first block from producing NaN
    const float xrow = xmax(mloc);
    // Sol: the summary blocks of this block's route group and of the groups before it come first
    const float m_cand = fmax_ieee(SOL ? fmax_ieee(m_run, gm_cur) : m_run, xrow * cs);
    const float m_new = (SPARSE || SOL) && m_cand == -INFINITY ? 0.0f : m_cand;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_cand;
    float lsum = 0.0f;
    if constexpr (EXPCAST) {
      // code = clamp(rint(8 z + 56 - 0.35), 0, 126) with z = log2(S p~): one FMA per key, then
      // v_cvt_pk_u8_f32, which rounds to nearest even, saturates to [0, 255] (NaN and -inf to
      // 0) and inserts the byte into the P word. The FMA is monotone in x, so the largest byte
      // of a row's block is that of its maximum, 8 log2 S + 55.65 <= 126.11 for S <= 448, and
      // the upper clamp is inactive. Only the FP32 rounding of b8 at huge logits (|m| of order
      // 1e5 log2 units and beyond) can carry the maximum past 126.5, which would round to 0x7F
      // (E4M3 NaN): a block where that happens in some row clamps every byte at 126 instead.
      // The row sums come from the matrix cores (pv).
      const float c8 = 8.0f * cs;
      const float b8 = 8.0f * (p.log2S - m_new) + 55.65f;
      const bool clamp = __builtin_expect(__any(__builtin_fmaf(xrow, c8, b8) > 126.5f), 0);  // (uniform)
      // key half by key half, as in the standard cast: the QK MFMAs of the next block's key
      // half t take over half t's registers once its bytes exist and run beside the other
      // half's codes
#pragma unroll
      for (int t = 0; t < 2; t++) {
#pragma unroll
        for (int w = 4 * t; w < 4 * t + 4; w++) {
          uint32_t word = static_cast<uint32_t>(pop[w]);  // every byte is overwritten
#pragma unroll
          for (int q = 0; q < 4; q++) word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(x[4 * w + q], c8, b8), q, word);
          pop[w] = static_cast<int>(word);
        }
        tie_k(t, lsum);
        if (t == 0) interleave_region1();
        else interleave_region2();
        // the rest of the block (QK MFMAs, second half's codes, row sum) runs at raised wave
        // priority, the PV MFMAs and operand reads at the normal one (see iteration)
        if (kPhasePrio && t == 0) __builtin_amdgcn_s_setprio(1);
        issue_qk_half(t);
      }
      if (clamp) {
        // (rare) min(rint(t), 126) = rint(min(t, 126)): clamp the bytes themselves (after the
        // QK issue, so that the branch does not split the scheduling regions; only the row-sum
        // and PV MFMAs, later, read the bytes)
#pragma unroll
        for (int w = 0; w < 8; w++) pop[w] = static_cast<int>(clamp_bytes_126(static_cast<uint32_t>(pop[w])));
      }
    } else {
      const float bias = p.log2S - m_new;
      // key sub-tile by key sub-tile (t = 0: x[0..15], t = 1: x[16..31]), so that the QK MFMAs of
      // the next block can take over each sub-tile's accumulator registers as soon as its P bytes
      // exist (see tie_k)
      lsum = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; t++) {
        float pv[16];
#pragma unroll
        for (int q = 0; q < 16; q++) pv[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[16 * t + q], cs, bias));
        // tree sum (four independent chains) keeps the adds off one dependency chain
        float l4[4];
#pragma unroll
        for (int q = 0; q < 4; q++) l4[q] = (pv[q] + pv[q + 4]) + (pv[q + 8] + pv[q + 12]);
        float lt = (l4[0] + l4[1]) + (l4[2] + l4[3]);
#pragma unroll
        for (int w = 0; w < 4; w++) {
          // the previous block's P bytes are dead once PV(j-1) has issued: converting into them
          // saves clearing the destination (each convert writes one half of the word)
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * w], pv[4 * w + 1], pop[4 * t + w], false);
          pop[4 * t + w] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4 * w + 2], pv[4 * w + 3], lo, true);
        }
        if constexpr (STATS) {
          const unsigned long long valid = qrow < p.N ? 1ull : 0ull;
#pragma unroll
          for (int q = 0; q < 16; q++)
            n_under += (pv[q] > 0.0f && ((static_cast<uint32_t>(pop[4 * t + (q >> 2)]) >> (8 * (q & 3))) & 0xFFu) == 0u)
                           ? valid
                           : 0ull;
        }
        tie_k(t, lt);
        lsum += lt;
        // QK of the next block's key half t takes over this half's registers
        if (t == 0) interleave_region1();
        else interleave_region2();
        if (kPhasePrio && t == 0) __builtin_amdgcn_s_setprio(1);  // (as in the ExpCast branch)
        issue_qk_half(t);
      }
    }
    if constexpr (!EXPCAST) {
      l_part = alpha * l_part + lsum;
      if constexpr (VSMOOTH) r_cur = alpha * r_cur + xsum(lsum);
    }
    return alpha;
  };

  // V-Smooth rank-one mean restores O^T += sum_v mu_v r_v^T of the (up to four) V blocks v of a
  // group, mu_v = the block's mean factors (in the residual's units) and r_v the lanes' S-scaled
  // row sums over its keys, on the matrix cores as one BF16 32x32x16 MFMA per 32 channels with a
  // hi/lo split of both factors: per block, three k slots carry mu_hi r_hi + mu_hi r_lo +
  // mu_lo r_hi (the dropped mu_lo r_lo is below 2^-16 of the product, and the split loses below
  // 2^-17 of each factor), exact products with FP32 accumulation. Lane half h holds k slots
  // 8h..8h+7 for the group's blocks 2h (slots 0..2) and 2h+1 (slots 3..5): the A operand of
  // channel 32 dt + l32 is its 16-byte record {hiA|hiA, loA|hiB, hiB|loB, 0} at byte 16 h of the
  // channel's 32 bytes in the slot, the B operand {rhA|rlA, rhA|rhB, rlB|rhB, 0}. Blocks that do
  // not exist or were not visited have zero sums (and zero factors past the sequence).
  auto split_bf16 = [](float r, uint32_t& hi, uint32_t& lo) {
    const __bf16 rh = static_cast<__bf16>(r);  // round to nearest even
    const __bf16 rl = static_cast<__bf16>(r - static_cast<float>(rh));
    hi = __builtin_bit_cast(uint16_t, rh);
    lo = __builtin_bit_cast(uint16_t, rl);
  };
  auto restore_group = [&](const uint8_t* sl) {
    v4i a[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++) a[dt] = *reinterpret_cast<const v4i*>(sl + kMeanOff + (32 * dt + l32) * 32 + 16 * lh);
    uint32_t ha, la, hb, lb;
    split_bf16(r_pa, ha, la);
    split_bf16(r_pb, hb, lb);
    v4i b;
    b[0] = static_cast<int>(ha | (la << 16));
    b[1] = static_cast<int>(ha | (hb << 16));
    b[2] = static_cast<int>(lb | (hb << 16));
    b[3] = 0;
    const v8bf bb = __builtin_bit_cast(v8bf, b);
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[dt]), bb, oacc[dt], 0, 0, 0);
    if constexpr (EXPCAST) {
      // the four record reads in flight together (left to itself the compiler, short of
      // registers here, reads one record per MFMA and waits for each)
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 1);  // VALU (the row sums' split)
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // MFMA
    }
    r_pa = 0.0f;
    r_pb = 0.0f;
  };

  // Keys past a block's valid count get S = -inf, in blocks with padding keys only. This runs
  // at the start of the block, before its PV MFMAs, so that the branch leaves the common path's
  // interleave of PV MFMAs, operand reads and softmax intact; the empty asm keeps the compiler
  // from hoisting the per-key compares out of the (uniform) branch. Sol: a block outside this
  // wave's own Q-block mask counts as fully masked. (Dense: the one masked block is the partial
  // last key block.)
  auto mask_block = [&]() {
    bool excluded = false;
    if constexpr (kSolPair) excluded = ex_cur;
    const int lim = (SPARSE || SOL) ? lim_cur : lim_tail;
    if (__builtin_amdgcn_readfirstlane(lim) < kBlock || excluded) {
      int nv = excluded ? 0 : lim - 32 * lh;  // valid keys among this lane's 32
      asm volatile("" : "+v"(nv));
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) sacc[t][r] = 16 * t + r < nv ? sacc[t][r] : -INFINITY;
    }
  };

  // One key block j; `sl` is the slot of pair j+1 (read here, then refilled with pair
  // j+1+kSlots). The masked copy serves blocks with fewer than 64 valid keys.
  // Steady (dense and STA): pairs j+2 and j+1+kSlots hold key blocks, so the waits and the
  // staging need no checks; dense staging is stage_dense.
  auto iteration = [&](auto mask_tag, auto steady_tag, int j, uint8_t* sl) {
    constexpr bool kSteady = decltype(steady_tag)::value;
    if constexpr (decltype(mask_tag)::value) mask_block();
    // Phase priority: the two waves of a SIMD arbitrate by phase, a wave in the QK part of its
    // block (from the first QK MFMAs on) ahead of one in the PV part (PV MFMAs, operand reads,
    // row maximum, first half's P bytes).
    if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(0);
    pv();         // PV of block j-1 (zero P bytes before the first block)
    read_v(sl);   // V(j)
    read_k(sl);   // K(j+1)
    read_meta(sl);
    // QK of block j+1 is issued inside the softmax, half by half (a dummy K tile after the last
    // block: its result is unused)
    const float alpha = softmax(mask_tag, qk_half);
    // alpha == 1 in every lane leaves O bit-identical: skip the multiplies
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] *= alpha;
      if constexpr (EXPCAST) {
        lacc[0] *= alpha;  // the only register of the sum that is read
        if constexpr (VSMOOTH) l_part *= alpha;
      }
      if constexpr (VSMOOTH) {
        r_pa *= alpha;
        r_pb *= alpha;
      }
    }
    // ExpCast: block j's code sums, in the units of its running max like lacc by now
    if constexpr (EXPCAST) lacc = mfma_rowsum(rs_sel, pop, lacc);
    if constexpr (VSMOOTH) {
      if (kSteady ? closes_vblock_inner(j) : closes_vblock(j)) {
        // the V block that block j closes: its row sum joins the group's pending sums, in the
        // units of the running max of block j like O (which holds blocks up to j-1)
        float r;
        if constexpr (EXPCAST) {
          r = lacc[0];
          l_part += r;
          lacc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        } else {
          r = r_cur;
          r_cur = 0.0f;
        }
        const int pos = vpos_of(j);  // (uniform)
        if ((pos >> 1) == lh) {
          if (pos & 1) r_pb = r;
          else r_pa = r;
        }
        // the group's records travel in pair j+1 when block j closes the group
        if (kSteady ? closes_group_inner(j) : closes_group(j)) restore_group(sl);
      }
    }
    // hand-off: every read of this slot is complete, pair j+2 has landed everywhere
    wait_lgkm0();
    if constexpr (kSteady) {
      wait_vmcnt<(kSlots - 2) * kCopies>();
    } else if (j + kSlots <= n_iter) {
      wait_all_but_newest();
    } else {
      wait_vmcnt<0>();
    }
    barrier_nofence();
    sk_cur = sk_next;
    lim_cur = lim_next;
    ex_cur = ex_next;
    gm_cur = gm_next;
    if constexpr (kSteady) {
      if constexpr (SPARSE) stage(j + 1 + kSlots, sl);  // (its key block exists: < n_iter)
      else stage_dense(sl);
    } else if (j + 1 + kSlots <= n_iter) {
      stage(j + 1 + kSlots, sl);
    }
  };

  // ---- prologue: pairs 0..kSlots-1 staged; K(0) read; QK of block 0; pair kSlots staged ----
  // (first the V scales and shift for the epilogue: the oldest copies, so the prologue's waits
  // for the first pairs cover them; a workgroup only reaches here after every wave left the
  // previous item's epilogue)
  if (lane < 32) {
    if (wave == 0) copy16_to_lds(p.v_scale + bh * kHeadDim, 16u * lane, lds_addr_of(reinterpret_cast<const uint8_t*>(vsc_s)));
    if (wave == 1 && p.v_shift) copy16_to_lds(p.v_shift + bh * kHeadDim, 16u * lane, lds_addr_of(reinterpret_cast<const uint8_t*>(vsc_s + kHeadDim)));
  }
  stage(0, slot(0));
  stage(1, slot(1));
  if constexpr (kSlots == 3) {
    if (n_iter >= 2) {
      stage(2, slot(2));
      wait_all_but_newest();
    } else {
      wait_vmcnt<0>();
    }
  } else {
    wait_vmcnt<0>();
  }
  barrier_nofence();
  read_k(slot(0));
  read_v(slot(0));  // a valid tile; it only meets the zero P bytes of PV(-1)
  read_meta(slot(0));
  qk();
  wait_lgkm0();
  barrier_nofence();
  sk_cur = sk_next;
  lim_cur = lim_next;
  ex_cur = ex_next;
  gm_cur = gm_next;
  if (n_iter >= kSlots) stage(kSlots, slot(0));

  // ---- mainloop. Dense: the one block with fewer than 64 valid keys (the last key block, first
  // in reverse order) runs in a masked copy outside the loop. Sparse: partial blocks sit at the
  // end of tiles anywhere in the sequence, so every block checks its valid-key count. ----
  using kNoMask = std::integral_constant<bool, false>;
  using kMasked = std::integral_constant<bool, true>;
  using kLoopMask = std::integral_constant<bool, SPARSE || SOL>;
  using kGeneric = std::integral_constant<bool, false>;
  using kSteady = std::integral_constant<bool, true>;
  const bool partial_tail = !SPARSE && !SOL && (p.N % kBlock) != 0 && has_last_block;
  int j = 0, j_end = n_iter, sidx = 1;  // sidx: slot of pair j+1
  if (partial_tail && p.reverse) {
    iteration(kMasked{}, kGeneric{}, 0, slot(1));
    j = 1;
    sidx = 2 % kSlots;
  }
  if (partial_tail && !p.reverse) j_end = n_iter - 1;
  if constexpr (!SOL) {
    // dense and STA: generic blocks until pair j+1 sits in slot 0, then steady blocks three at a
    // time with constant slots while block j+2 stages a key block (j + 2 + 4 < n_iter). STA
    // blocks keep the per-block valid-key check (partial blocks end tiles anywhere).
    while (j < j_end && sidx != 0) {
      iteration(kLoopMask{}, kGeneric{}, j, slot(sidx));
      sidx = sidx == kSlots - 1 ? 0 : sidx + 1;
      j++;
    }
    // (the underflow-counting variant, a debugging aid, stays on the generic path)
    const int j_steady = STATS ? 0 : min(j_end, n_iter - 1 - kSlots);  // steady: j < j_steady
    using kSteadyMask = std::integral_constant<bool, SPARSE>;
    if constexpr (!SPARSE) {
      if (j + kSlots <= j_steady) stage_dense_init();
    }
    for (; j + kSlots <= j_steady; j += kSlots) {
      iteration(kSteadyMask{}, kSteady{}, j, slot(0));
      __builtin_amdgcn_sched_barrier(0);
      iteration(kSteadyMask{}, kSteady{}, j + 1, slot(1));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSlots == 3) {
        iteration(kSteadyMask{}, kSteady{}, j + 2, slot(2));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  for (; j < j_end; j++) {
    iteration(kLoopMask{}, kGeneric{}, j, slot(sidx));
    sidx = sidx == kSlots - 1 ? 0 : sidx + 1;
  }
  if (partial_tail && !p.reverse) iteration(kMasked{}, kGeneric{}, n_iter - 1, slot(sidx));
  pv();  // PV of the last block (vop = V(n_iter - 1))

  if constexpr (STATS) {
    unsigned long long tot = n_under;
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (lane == 0 && tot) atomicAdd(p.underflow + bh, tot);
  }

  // ---- epilogue: O = acc * g_d / l', BF16, scattered to the destination rows ----
  bool ok = qrow < p.N;
  if constexpr (SPARSE && !SOL) ok = ok && q_tile_off + 32 * wave + l32 < q_valid_len;
  // the S-scaled row sum: standard cast, the two lane halves' shares; ExpCast, the matrix-core
  // sum, whole in every lane (with V-Smooth, collected per V block in l_part)
  float l_tot;
  if constexpr (EXPCAST) l_tot = VSMOOTH ? l_part : lacc[0];
  else l_tot = xsum(l_part);
  // This lane's channels d0 .. d0 + 3 for output group i = 4 dt + g: d0 = 32 dt + 8 g + 4 lh.
  // The groups are written in two halves of eight, their V scales and shifts read from the
  // prologue's copy in LDS. The sched barrier keeps the second half's reads from being hoisted,
  // which would spill registers.
  auto chan = [&](int i) -> int { return 32 * (i >> 2) + 8 * (i & 3) + 4 * lh; };
  auto load8 = [&](float4 (&dst)[8], const float* src, int half) {
#pragma unroll
    for (int k = 0; k < 8; k++) dst[k] = *reinterpret_cast<const float4*>(src + chan(8 * half + k));
  };
  auto load_scales = [&](float4 (&sv)[8], float4 (&sh)[8], int half) {
    load8(sv, vsc_s, half);
    if (p.v_shift) {
      load8(sh, vsc_s + kHeadDim, half);
    } else {
#pragma unroll
      for (int k = 0; k < 8; k++) sh[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  if constexpr (SOL) {
    // Sol: the shared state's result. The summary contributions (written before this kernel as
    // their normalised sum o_part and log2 weight lse) and this route's accumulator are added,
    // each rescaled to the common maximum, and O = acc / l, in BF16
    if (ok) {
      const float lse0 = l_tot > 0.0f ? m_run + __log2f(l_tot) : -INFINITY;
      const int64_t r1 = bh * p.N + qrow;
      const float lse1 = p.lse[r1];
      const float mx = fmaxf(lse0, lse1);
      const float w0 = __builtin_amdgcn_exp2f(lse0 - mx), w1 = __builtin_amdgcn_exp2f(lse1 - mx);
      const float inv_w = 1.0f / (w0 + w1);
      const float a0 = l_tot > 0.0f ? w0 * inv_w / l_tot : 0.0f;  // on acc * v_scale
      const float a1 = w1 * inv_w;
      uint16_t* orow = p.out + ((b * p.n_out + qrow) * p.H + h) * kHeadDim;
#pragma unroll
      for (int half = 0; half < 2; half++) {
        float4 sv[8], sh[8], ov[8];
        load_scales(sv, sh, half);
        load8(ov, p.o_part + r1 * kHeadDim, half);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const int i = 8 * half + k;
          const float e0 = oacc[i >> 2][4 * (i & 3) + 0] * sv[k].x * a0 + ov[k].x * a1 + sh[k].x;
          const float e1 = oacc[i >> 2][4 * (i & 3) + 1] * sv[k].y * a0 + ov[k].y * a1 + sh[k].y;
          const float e2 = oacc[i >> 2][4 * (i & 3) + 2] * sv[k].z * a0 + ov[k].z * a1 + sh[k].z;
          const float e3 = oacc[i >> 2][4 * (i & 3) + 3] * sv[k].w * a0 + ov[k].w * a1 + sh[k].w;
          uint2 o;
          o.x = static_cast<uint32_t>(f32_to_bf16_rne(e0)) | (static_cast<uint32_t>(f32_to_bf16_rne(e1)) << 16);
          o.y = static_cast<uint32_t>(f32_to_bf16_rne(e2)) | (static_cast<uint32_t>(f32_to_bf16_rne(e3)) << 16);
          *reinterpret_cast<uint2*>(orow + chan(i)) = o;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return;
  }
  if constexpr (!SPARSE) {
    if (p.o_part) {
      // split-KV piece or Sol exact route: this piece's normalised O (FP32) and log2 of its
      // weight, m + log2(l)
      if (ok) {
        // (Sol: a wave none of whose staged blocks was exact for its Q block has no weight)
        const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t prow = (static_cast<int64_t>(split) * p.B * p.H + bh) * p.N + qrow;
        float* orow = p.o_part + prow * kHeadDim;
#pragma unroll
        for (int half = 0; half < 2; half++) {
          float4 sv[8], sh[8];
          load_scales(sv, sh, half);
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const int i = 8 * half + k;
            float gs[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
            if constexpr (VSMOOTH) {
#pragma unroll
              for (int e = 0; e < 4; e++) gs[e] = gs[e] > 0.0f ? gs[e] : 1.0f;
            }
            float4 o;
            o.x = oacc[i >> 2][4 * (i & 3) + 0] * gs[0] * inv_l;
            o.y = oacc[i >> 2][4 * (i & 3) + 1] * gs[1] * inv_l;
            o.z = oacc[i >> 2][4 * (i & 3) + 2] * gs[2] * inv_l;
            o.w = oacc[i >> 2][4 * (i & 3) + 3] * gs[3] * inv_l;
            *reinterpret_cast<float4*>(orow + chan(i)) = o;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (lh == 0) p.lse[prow] = l_tot > 0.0f ? m_run + __log2f(l_tot) : -INFINITY;
      }
      return;
    }
  }
  int64_t dst = qrow;
  if (ok && p.out_rows) dst = out_row;
  ok = ok && dst >= 0 && dst < p.n_out;
  if (ok) {
    const float inv_l = 1.0f / l_tot;
    uint16_t* orow = p.out + ((b * p.n_out + dst) * p.H + h) * kHeadDim;
#pragma unroll
    for (int half = 0; half < 2; half++) {
      float4 sv[8], sh[8];
      load_scales(sv, sh, half);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int i = 8 * half + k;
        float gs[4] = {sv[k].x, sv[k].y, sv[k].z, sv[k].w};
        if constexpr (VSMOOTH) {
#pragma unroll
          for (int e = 0; e < 4; e++) gs[e] = gs[e] > 0.0f ? gs[e] : 1.0f;
        }
        // sequence-mean smoothing: every softmax row sums to one, so the V shift comes back as
        // a constant vector
        const float c[4] = {sh[k].x, sh[k].y, sh[k].z, sh[k].w};
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; e++) ov[e] = oacc[i >> 2][4 * (i & 3) + e] * gs[e] * inv_l + c[e];
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16_rne(ov[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(ov[1])) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16_rne(ov[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(ov[3])) << 16);
        *reinterpret_cast<uint2*>(orow + chan(i)) = o;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Variants whose workgroups take their items from the per-XCD queues (the underflow-counting
// debugging variant would spill registers in the loop around attn_tile).
template <bool VSMOOTH, bool STATS, bool SOL>
constexpr bool kQueued = !STATS;

// The work items are cut into eight contiguous ranges, one per XCD, so that the workgroups of
// an XCD share the K/V tiles of few (b, h) in its L2. Queued variants: persistent workgroups
// (as many as fit the device) take the items of their XCD's range one at a time from a counter
// in the workspace, then those of the other ranges, so that an XCD that runs faster (or whose
// items are shorter: sparse rows and Sol masks differ in length) takes more; the counters are
// zeroed by attn_queue_reset before each launch. Otherwise one workgroup per item: the hardware
// dispatches workgroup i to XCD i % 8, so workgroup i takes item (i % 8) * per_xcd + i / 8.
template <int WAVES, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS, bool SOL>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(AttnParams p) {
  const int per_xcd = (p.total_work + 7) / 8;
  if constexpr (kQueued<VSMOOTH, STATS, SOL>) {
    __shared__ int work_s;
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    for (;;) {
      if (threadIdx.x == 0) {
        int w = -1;
        for (int k = 0; k < 8 && w < 0; k++) {
          const int q = static_cast<int>((xcc + k) & 7u);
          const int cnt = min(per_xcd, p.total_work - q * per_xcd);
          if (cnt <= 0) continue;
          const int i = static_cast<int>(atomicAdd(p.work_ctr + q, 1u));
          if (i < cnt) w = q * per_xcd + i;
        }
        work_s = w;
      }
      __syncthreads();
      const int work = work_s;
      __syncthreads();  // (work_s is rewritten for the next item)
      if (work < 0) return;
      attn_tile<WAVES, SPARSE, EXPCAST, VSMOOTH, STATS, SOL>(p, work);
    }
  } else {
    const int work = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
    if (work < p.total_work) attn_tile<WAVES, SPARSE, EXPCAST, VSMOOTH, STATS, SOL>(p, work);
  }
}

__global__ void attn_queue_reset(uint32_t* ctr) {
  if (threadIdx.x < 8) ctr[threadIdx.x] = 0u;
}

// V-Smooth: the factors mu_v = float(mean_hat[bh, v, d]) * (s_r[d] > 0 ? 1 / s_r[d] : 1) of the
// four V blocks v = 4 g .. 4 g + 3 of group g (0 past the sequence), split as mu_hi = BF16(mu),
// mu_lo = BF16(mu - mu_hi) (both rounded to nearest even), written as the restore's A-operand
// records of channel d: mu_op[bh, g, d] = {hiA|hiA, loA|hiB, hiB|loB, 0} for blocks (A, B) =
// (4g, 4g+1), then for (4g+2, 4g+3) (BF16 pairs, low half first; 32 bytes).
__global__ __launch_bounds__(128) void vsmooth_mean_factors(AttnParams p) {
  const int64_t g = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int d = threadIdx.x;
  const float sr = p.v_scale[bh * kHeadDim + d];
  const float f = sr > 0.0f ? __fdiv_rn(1.0f, sr) : 1.0f;
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int64_t v = 4 * g + k;
    const float mu = v < p.NB128 ? bf16_to_f32(p.v_mean[(bh * p.NB128 + v) * kHeadDim + d]) * f : 0.0f;
    hi[k] = f32_to_bf16_rne(mu);
    lo[k] = f32_to_bf16_rne(mu - __uint_as_float(hi[k] << 16));
  }
  uint4* rec = reinterpret_cast<uint4*>(p.mu_op) + ((bh * ((p.NB128 + 3) >> 2) + g) * kHeadDim + d) * 2;
#pragma unroll
  for (int h = 0; h < 2; h++)
    rec[h] = make_uint4(hi[2 * h] | (hi[2 * h] << 16), lo[2 * h] | (hi[2 * h + 1] << 16),
                        hi[2 * h + 1] | (lo[2 * h + 1] << 16), 0u);
}

// Split-KV merge ([TF] long-sequence split-KV, log-sum-exp reduction): per row,
// O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s, then the sequence-mean
// V shift, BF16 and the row scatter. 32 threads per row (4 channels each), 8 rows per workgroup.
__global__ __launch_bounds__(256) void split_merge(AttnParams p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int64_t bh = blockIdx.y;
  const int c = (threadIdx.x & 31) * 4;
  if (row >= p.N) return;
  int64_t dst = row;
  if (p.out_rows) dst = p.out_rows[row];
  if (dst < 0 || dst >= p.n_out) return;
  const int64_t BH = static_cast<int64_t>(p.B) * p.H;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; s++) M = fmaxf(M, p.lse[(s * BH + bh) * p.N + row]);
  float wsum = 0.0f;
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < p.splits; s++) {
    const int64_t prow = (s * BH + bh) * p.N + row;
    const float w = __builtin_amdgcn_exp2f(p.lse[prow] - M);
    const float4 o = *reinterpret_cast<const float4*>(p.o_part + prow * kHeadDim + c);
    wsum += w;
    a[0] = __builtin_fmaf(w, o.x, a[0]);
    a[1] = __builtin_fmaf(w, o.y, a[1]);
    a[2] = __builtin_fmaf(w, o.z, a[2]);
    a[3] = __builtin_fmaf(w, o.w, a[3]);
  }
  const float inv = 1.0f / wsum;
  float sh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (p.v_shift) {
    const float4 cv = *reinterpret_cast<const float4*>(p.v_shift + bh * kHeadDim + c);
    sh[0] = cv.x;
    sh[1] = cv.y;
    sh[2] = cv.z;
    sh[3] = cv.w;
  }
  const int64_t b = bh / p.H, h = bh % p.H;
  uint2 o;
  o.x = static_cast<uint32_t>(f32_to_bf16_rne(a[0] * inv + sh[0])) |
        (static_cast<uint32_t>(f32_to_bf16_rne(a[1] * inv + sh[1])) << 16);
  o.y = static_cast<uint32_t>(f32_to_bf16_rne(a[2] * inv + sh[2])) |
        (static_cast<uint32_t>(f32_to_bf16_rne(a[3] * inv + sh[3])) << 16);
  *reinterpret_cast<uint2*>(p.out + ((b * p.n_out + dst) * p.H + h) * kHeadDim + c) = o;
}

template <int WAVES, bool SPARSE, bool EXPCAST, bool VSMOOTH, bool STATS, bool SOL = false>
hipError_t launch_variant(AttnParams& p, hipStream_t stream) {
  const int rows = WAVES * 32;
  p.n_qtiles = static_cast<int>((p.N + rows - 1) / rows);
  p.total_work = p.B * p.H * p.n_qtiles * p.splits;
  unsigned grid = static_cast<unsigned>(((p.total_work + 7) / 8) * 8);
  if constexpr (kQueued<VSMOOTH, STATS, SOL>) {
    if (!p.work_ctr) return hipErrorInvalidValue;
    // resident workgroups: two waves per SIMD, four SIMDs per CU
    const int64_t slots = static_cast<int64_t>(p.cus > 0 ? p.cus : 256) * 8 / WAVES;
    grid = static_cast<unsigned>(p.total_work < slots ? p.total_work : slots);
    hipLaunchKernelGGL(attn_queue_reset, dim3(1), dim3(64), 0, stream, p.work_ctr);
  }
  hipLaunchKernelGGL((attn_fwd<WAVES, SPARSE, EXPCAST, VSMOOTH, STATS, SOL>), dim3(grid), dim3(WAVES * 64), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(split_merge, dim3(static_cast<unsigned>((p.N + 7) / 8), static_cast<unsigned>(p.B * p.H)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Sol: the exact blocks of the shared state (two waves per 64-row Q block over its mask's
// blocks, each block's running max raised first by the summary maximum of its route group; the
// kernel also has a four-wave form over the union of two Q blocks' masks, which only pays when
// neighbouring Q blocks share most exact blocks); its epilogue adds the summary contributions,
// which have been written before.
template <bool EXPCAST>
hipError_t launch_sol_exact(AttnParams p, hipStream_t stream) {
  p.splits = 1;
  return launch_variant<2, true, EXPCAST, false, false, true>(p, stream);
}

}  // namespace

hipError_t launch_attention(AttnParams p, int variant, hipStream_t stream) {
  const bool ec = variant & kVarExpCast, vs = variant & kVarVSmooth, sp = variant & kVarSparse,
             st = variant & kVarStats;
  if (variant & kVarSol) return ec ? launch_sol_exact<true>(p, stream) : launch_sol_exact<false>(p, stream);
  if (vs) {
    hipLaunchKernelGGL(vsmooth_mean_factors, dim3(static_cast<unsigned>((p.NB128 + 3) / 4), static_cast<unsigned>(p.B * p.H)),
                       dim3(kHeadDim), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Dense: 4 waves (128 queries) per workgroup. Sparse: a workgroup stays inside one query tile
  // (128 or 64 rows).
  if (sp && p.tile_tokens % 128 == 0) {
    if (st) return launch_variant<4, true, false, false, true>(p, stream);
    if (ec) return launch_variant<4, true, true, false, false>(p, stream);
    return launch_variant<4, true, false, false, false>(p, stream);
  }
  if (sp) {
    if (st) return launch_variant<2, true, false, false, true>(p, stream);
    if (ec) return launch_variant<2, true, true, false, false>(p, stream);
    return launch_variant<2, true, false, false, false>(p, stream);
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
