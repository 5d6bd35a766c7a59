// Paged attention on the matrix cores: bf16/fp16 queries over 16-bit or fp8
// (e4m3) K/V pools.
//
// One wave works on one (sequence, kv head) at a time; per 16-token block:
//   QK:  S^T[t][h] = sum_d K[t][d] Q[h][d]: 16x16x32 MFMAs over head_size,
//        tokens on M, the G query heads of the group on N (rows >= G zero).
//        Lane l receives S[h = l%16][t = 4*(l/16) + i], i < 4.
//   PV:  O[h][d] += sum_t P[h][t] V[t][d]: one 16x16x16 MFMA per 16-wide tile
//        of head_size.  The score layout above is exactly the A operand
//        (P[h = l%16][t = 4*(l/16) + j]).  V rows are loaded so that lane l
//        holds rows t = 4*(l/16) + j, j < 4, and the elements
//        d = VE*(l%16) .. VE*(l%16)+VE-1; output column n of tile T then maps
//        to d = VE*n + T, so each B operand is element T of the lane's four
//        rows (two byte permutes).  No LDS is used.
//   Softmax: base 2 (scale * log2(e) applied to the score), probabilities
//        rounded to the KV type for the PV product, sums in fp32.  Scores are
//        only rescaled when a block maximum exceeds the running reference by
//        more than 2^8; until then probabilities are taken against the stale
//        reference, which is the same sum re-associated.
//
// The K/V format only changes the loader (KvIo: where each lane's bytes are
// and how they become MFMA operands).  Launch shapes sharing this core:
//  * pa_decode_sk_kernel: balanced split.  The (sequence, block) pairs of the
//    whole batch are laid end to end and cut into equal ranges, one per
//    workgroup; a workgroup has one wave per kv head of a head group, so a
//    block's heads (one contiguous stretch of the pool) are read together,
//    with the waves kept in step.  A sequence that crosses a range boundary
//    leaves partial records that a merge kernel combines.  With MQ the 16
//    rows are (token, head) pairs of several query tokens (speculative
//    verification), masked causally on the final blocks.
//  * pa_decode_mfma_kernel: the split-context path with a fixed partition
//    size: work items (sequence, partition, head group), up to two per
//    workgroup.
//  * pa_prefill_kernel / pa_prefill_lds_kernel: multi-token queries, one
//    wave per 16-row tile; the LDS variant shares each K/V block among the
//    16 tiles of a workgroup, two per wave.
#pragma once

#include "common.h"

namespace pa {

// Rescale only when a score exceeds the reference by more than 2^8 (see above).
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct MfmaShape {
  static constexpr int kRow = D * 2;      // bytes of one token row of one head
  static constexpr int kKs = D / 32;      // QK steps, 16 bytes of K per lane each
  static constexpr int kVe = D / 16;      // V elements per lane per row = PV tiles
  static constexpr int kVw = kVe / 2;     // ... as dwords
  static_assert(D == 64 || D == 128, "head_size 64 or 128");
};

// Per-wave state of one (sequence, kv head) segment.
template <int D>
struct MfmaState {
  u32x4 qb[MfmaShape<D>::kKs];   // Q^T operand: lane l holds Q[h = l%16][d = 32*step + 8*(l/16) ..]
  float m_ref;                    // reference max of head l%16 (base-2 units)
  float l_part;                   // this lane's share of the softmax sum of head l%16
  f32x4 acc[MfmaShape<D>::kVe];   // O[h = 4*(l/16) + i][d = VE*(l%16) + T]
};

// Where each lane's K/V bytes are and how they become MFMA operands.  For a
// QK step the lane (c = l%16, g = l/16) supplies 8 consecutive elements of K
// row c; which 8 (the map d(g, step)) only has to agree with the query
// operand, since QK sums over d.
template <class KV, class E, int D>
struct KvIo;

template <class E, int D>
struct KvIo<Kv16, E, D> {
  using SH = MfmaShape<D>;
  static constexpr int kRowBytes = D * 2;
  struct Blk {
    u32x4 k[SH::kKs];                 // K row c, d = 32*step + 8*g ..
    uint32_t v[4][SH::kVw];           // V rows 4*g + j, d = VE*c ..
  };
  __device__ static int q_elem(int g, int step) { return 32 * step + 8 * g; }
  __device__ static int k_off(int c, int g, int hkv, int kvh) { return (c * hkv + kvh) * kRowBytes + 16 * g; }
  __device__ static int v_off(int c, int g, int hkv, int kvh) { return (4 * g * hkv + kvh) * kRowBytes + SH::kVe * 2 * c; }
  template <bool NT>
  __device__ static void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int k_off, int v_off,
                              int row_stride, Blk& b) {
#pragma unroll
    for (int k = 0; k < SH::kKs; ++k) b.k[k] = load16<NT>(rk, k_off, 64 * k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (SH::kVw == 4) {
        const u32x4 t = load16<NT>(rv, v_off, j * row_stride);
        b.v[j][0] = t[0]; b.v[j][1] = t[1]; b.v[j][2] = t[2]; b.v[j][3] = t[3];
      } else {
        const u32x2 t = load8<NT>(rv, v_off, j * row_stride);
        b.v[j][0] = t[0]; b.v[j][1] = t[1];
      }
    }
  }
  __device__ static u32x4 k_operand(const Blk& b, int step) { return b.k[step]; }
  __device__ static uint32_t v_word(const Blk& b, int j, int q) { return b.v[j][q]; }
};

template <class E, int D>
struct KvIo<KvFp8, E, D> {
  using SH = MfmaShape<D>;
  static constexpr int kRowBytes = D;
  static constexpr int kKq = D / 64;  // 16-byte K loads per lane (its D/4 contiguous codes)
  static constexpr int kVq = SH::kVe / 4;   // dwords of V codes per row per lane
  struct Blk {
    u32x4 k[kKq];                     // K row c, d = (D/4)*g .. (D/4)*g + D/4 - 1
    uint32_t v[4][kVq];               // V rows 4*g + j, d = VE*c ..
  };
  __device__ static int q_elem(int g, int step) { return (D / 4) * g + 8 * step; }
  __device__ static int k_off(int c, int g, int hkv, int kvh) { return (c * hkv + kvh) * kRowBytes + (D / 4) * g; }
  __device__ static int v_off(int c, int g, int hkv, int kvh) { return (4 * g * hkv + kvh) * kRowBytes + SH::kVe * c; }
  template <bool NT>
  __device__ static void load(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int k_off, int v_off,
                              int row_stride, Blk& b) {
#pragma unroll
    for (int k = 0; k < kKq; ++k) b.k[k] = load16<NT>(rk, k_off, 16 * k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kVq == 2) {
        const u32x2 t = load8<NT>(rv, v_off, j * row_stride);
        b.v[j][0] = t[0]; b.v[j][1] = t[1];
      } else {
        b.v[j][0] = load4<NT>(rv, v_off, j * row_stride);
      }
    }
  }
  __device__ static u32x4 k_operand(const Blk& b, int step) {
    const uint32_t w0 = b.k[step >> 1][(2 * step) & 3], w1 = b.k[step >> 1][(2 * step + 1) & 3];
    return u32x4{fp8x2_to<E, false>(w0), fp8x2_to<E, true>(w0), fp8x2_to<E, false>(w1), fp8x2_to<E, true>(w1)};
  }
  __device__ static uint32_t v_word(const Blk& b, int j, int q) {   // q is unrolled: the branch folds
    return (q & 1) ? fp8x2_to<E, true>(b.v[j][q >> 1]) : fp8x2_to<E, false>(b.v[j][q >> 1]);
  }
};

template <class KV, int D, int G>
__device__ __forceinline__ void mfma_begin(MfmaState<D>& st, const void* query, int64_t q_row0, int g, int c) {
  using SH = MfmaShape<D>;
  using IO = KvIo<KV, ElemBF16, D>;              // the query map does not depend on E
  const char* qrow = static_cast<const char*>(query) + (q_row0 + c) * SH::kRow;
#pragma unroll
  for (int k = 0; k < SH::kKs; ++k)
    st.qb[k] = c < G ? *reinterpret_cast<const u32x4*>(qrow + 2 * IO::q_elem(g, k)) : u32x4{0u, 0u, 0u, 0u};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;
#pragma unroll
  for (int T = 0; T < SH::kVe; ++T) st.acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Start a segment whose 16 rows are arbitrary query rows: lane l loads row
// q_row (its row l%16; zeros when !live) with the d map of KV.
template <class KV, int D>
__device__ __forceinline__ void mfma_begin_row(MfmaState<D>& st, const void* query, int64_t q_row, bool live, int g) {
  using SH = MfmaShape<D>;
  using IO = KvIo<KV, ElemBF16, D>;
  const char* qrow = static_cast<const char*>(query) + q_row * SH::kRow;
#pragma unroll
  for (int k = 0; k < SH::kKs; ++k)
    st.qb[k] = live ? *reinterpret_cast<const u32x4*>(qrow + 2 * IO::q_elem(g, k)) : u32x4{0u, 0u, 0u, 0u};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;
#pragma unroll
  for (int T = 0; T < SH::kVe; ++T) st.acc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Blocks [b_begin, b_end) of one sequence for kv head `kvh`; tokens at or past
// t_end are masked.  Returns true if a block id of the range is out of the
// pool (the segment's result is then undefined and must be reported as NaN).
// LOCK: every wave of the workgroup runs the same segment for its own kv head
// and the waves meet at a barrier before each block's loads, so the slices of
// one block's token rows are requested together (DRAM rows stay open for the
// whole block instead of being reopened by waves that have drifted apart).
template <class E, class KV, int D, bool NT, bool LOCK>
__device__ __forceinline__ bool mfma_segment(MfmaState<D>& st, const char* __restrict__ k_cache,
                                             const char* __restrict__ v_cache, const int* __restrict__ bt_row,
                                             int b_begin, int b_end, int t_end, int num_blocks,
                                             int num_kv_heads, int kvh, float qk_scale, int lane) {
  using SH = MfmaShape<D>;
  using M = Mfma<E>;
  using IO = KvIo<KV, E, D>;
  using Blk = typename IO::Blk;
  constexpr int BS = kBlockSize, KS = SH::kKs, VE = SH::kVe, VW = SH::kVw;
  const int g = lane >> 4, c = lane & 15;
  const int blk_bytes = BS * num_kv_heads * IO::kRowBytes;
  const int row_stride = num_kv_heads * IO::kRowBytes;
  const int k_off = IO::k_off(c, g, num_kv_heads, kvh);     // K row t = l%16
  const int v_off = IO::v_off(c, g, num_kv_heads, kvh);     // V rows t = 4*(l/16) + j

  auto load_block = [&](int phys, Blk& b) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(k_cache + (int64_t)phys * blk_bytes, blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(v_cache + (int64_t)phys * blk_bytes, blk_bytes);
    IO::template load<NT>(rk, rv, k_off, v_off, row_stride, b);
  };

  auto consume = [&](const Blk& b, int valid, bool masked) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) sc = M::qk(IO::k_operand(b, k), st.qb[k], sc);
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = sc[i] * qk_scale;
      if (masked && 4 * g + i >= valid) z[i] = -INFINITY;
    }
    const float bm = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    if (__ballot(bm > st.m_ref + kRescaleThreshold)) {
      const float m_new = fmaxf(st.m_ref, bm);
      const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);   // 0 on the first block
      st.l_part *= alpha;
      float ar[4];                                                     // factors of rows h = 4*(l/16) + i
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int T = 0; T < VE; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[T][i] *= ar[i];
      st.m_ref = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - st.m_ref);
    st.l_part += (p[0] + p[1]) + (p[2] + p[3]);
    const u32x2 pa = {pack2<E>(p[0], p[1]), pack2<E>(p[2], p[3])};

    uint32_t v[4][VW];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < VW; ++q) v[j][q] = (masked && 4 * g + j >= valid) ? 0u : IO::v_word(b, j, q);
#pragma unroll
    for (int T = 0; T < VE; ++T) {
      const uint32_t sel = (T & 1) ? 0x07060302u : 0x05040100u;   // high or low half of each dword
      const u32x2 vb = {__builtin_amdgcn_perm(v[1][T >> 1], v[0][T >> 1], sel),
                        __builtin_amdgcn_perm(v[3][T >> 1], v[2][T >> 1], sel)};
      st.acc[T] = M::pv(pa, vb, st.acc[T]);
    }
  };

  // Block ids: up to 64 per batch, one per lane, then broadcast with readlane.
  // Two register sets alternate so the next block's loads are in flight while
  // the current block is consumed; inside the steady-state loop every load is
  // unconditional, which lets each consume wait only for its own block.  Only
  // the segment's last block can be partial.
  const int last_valid = t_end - (b_end - 1) * BS;
  for (int cb = b_begin; cb < b_end; cb += 64) {
    const int n = min(64, b_end - cb);
    const int id = lane < n ? bt_row[cb + lane] : 0;
    if (__ballot(lane < n && (unsigned)id >= (unsigned)num_blocks)) return true;
    const bool last_batch = cb + 64 >= b_end;
    Blk A, B;
    if constexpr (LOCK) __builtin_amdgcn_s_barrier();
    load_block(__builtin_amdgcn_readlane(id, 0), A);
    int j = 0;
    for (; j + 2 < n; j += 2) {
      if constexpr (LOCK) __builtin_amdgcn_s_barrier();
      load_block(__builtin_amdgcn_readlane(id, j + 1), B);
      consume(A, BS, false);
      if constexpr (LOCK) __builtin_amdgcn_s_barrier();
      load_block(__builtin_amdgcn_readlane(id, j + 2), A);
      consume(B, BS, false);
    }
    const int vj = (last_batch && j == n - 1) ? last_valid : BS;
    if (j + 1 < n) {
      if constexpr (LOCK) __builtin_amdgcn_s_barrier();
      load_block(__builtin_amdgcn_readlane(id, j + 1), B);
      consume(A, BS, false);
      const int vj1 = last_batch ? last_valid : BS;
      if (vj1 >= BS) consume(B, BS, false);
      else consume(B, vj1, true);
    } else if (vj >= BS) {
      consume(A, BS, false);
    } else {
      consume(A, vj, true);
    }
  }
  return false;
}

// Causal variant for multi-token queries: the 16 rows of each of the NTILE
// tiles are (token, head) pairs with their own last visible position
// `row_last[t]` (one per lane and tile: this lane's row l%16).  Blocks
// [b_begin, b_end) of the sequence are streamed once for all tiles (each
// loaded block feeds every tile's QK and PV); blocks from `mask_from` on are
// masked per row.  V rows past the sequence's last token `seq_last` are
// zeroed (they may hold anything); inside the sequence a masked key only
// needs its zero probability.  A row may see no key of the whole range (a
// range holding only the sequence's last keys): its max stays -inf and its
// probabilities and sum stay 0, so a partial result of such a row weighs
// nothing in the merge.  LOCK as in mfma_segment.
template <class E, class KV, int D, bool NT, bool LOCK, int NTILE>
__device__ __forceinline__ bool mfma_segment_rows(MfmaState<D> (&st)[NTILE], const char* __restrict__ k_cache,
                                                  const char* __restrict__ v_cache, const int* __restrict__ bt_row,
                                                  int b_begin, int b_end, int mask_from,
                                                  const int (&row_last)[NTILE], int seq_last, int num_blocks,
                                                  int num_kv_heads, int kvh, float qk_scale, int lane) {
  using SH = MfmaShape<D>;
  using M = Mfma<E>;
  using IO = KvIo<KV, E, D>;
  using Blk = typename IO::Blk;
  constexpr int BS = kBlockSize, KS = SH::kKs, VE = SH::kVe, VW = SH::kVw;
  const int g = lane >> 4;
  const int blk_bytes = BS * num_kv_heads * IO::kRowBytes;
  const int row_stride = num_kv_heads * IO::kRowBytes;
  const int k_off = IO::k_off(lane & 15, g, num_kv_heads, kvh);
  const int v_off = IO::v_off(lane & 15, g, num_kv_heads, kvh);

  auto load_block = [&](int phys, Blk& b) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(k_cache + (int64_t)phys * blk_bytes, blk_bytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(v_cache + (int64_t)phys * blk_bytes, blk_bytes);
    IO::template load<NT>(rk, rv, k_off, v_off, row_stride, b);
  };

  // key0: position of the block's first key
  auto consume = [&](const Blk& b, int key0, bool masked) {
    u32x2 pa[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) sc = M::qk(IO::k_operand(b, k), st[t].qb[k], sc);
      // lane l holds S[row = l%16][key = key0 + 4*(l/16) + i]; row_last is that row's limit
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = sc[i] * qk_scale;
        if (masked && key0 + 4 * g + i > row_last[t]) z[i] = -INFINITY;
      }
      const float bm = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      if (__ballot(bm > st[t].m_ref + kRescaleThreshold)) {
        const float m_new = fmaxf(st[t].m_ref, bm);
        // 0 on a row's first visible block; a row with nothing visible yet keeps 0 state
        const float alpha = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[t].m_ref - m_new);
        st[t].l_part *= alpha;
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int T = 0; T < VE; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[t].acc[T][i] *= ar[i];
        st[t].m_ref = m_new;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = (masked && z[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[i] - st[t].m_ref);
      st[t].l_part += (p[0] + p[1]) + (p[2] + p[3]);
      pa[t] = u32x2{pack2<E>(p[0], p[1]), pack2<E>(p[2], p[3])};
    }
    uint32_t v[4][VW];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < VW; ++q) v[j][q] = (masked && key0 + 4 * g + j > seq_last) ? 0u : IO::v_word(b, j, q);
#pragma unroll
    for (int T = 0; T < VE; ++T) {
      const uint32_t sel = (T & 1) ? 0x07060302u : 0x05040100u;
      const u32x2 vb = {__builtin_amdgcn_perm(v[1][T >> 1], v[0][T >> 1], sel),
                        __builtin_amdgcn_perm(v[3][T >> 1], v[2][T >> 1], sel)};
#pragma unroll
      for (int t = 0; t < NTILE; ++t) st[t].acc[T] = M::pv(pa[t], vb, st[t].acc[T]);
    }
  };

  // Blocks before mask_from and from mask_from on run as two separate
  // pipelines, each with the mask fixed at compile time: a branch between a
  // load and its use would make every consume wait for all loads in flight.
  auto run = [&](auto masked_tag, int lo, int hi) -> bool {
    constexpr bool MASKED = decltype(masked_tag)::value;
    for (int cb = lo; cb < hi; cb += 64) {
      const int n = min(64, hi - cb);
      const int id = lane < n ? bt_row[cb + lane] : 0;
      if (__ballot(lane < n && (unsigned)id >= (unsigned)num_blocks)) return true;
      Blk A, B;
      if constexpr (LOCK) __builtin_amdgcn_s_barrier();
      load_block(__builtin_amdgcn_readlane(id, 0), A);
      int j = 0;
      for (; j + 2 < n; j += 2) {
        if constexpr (LOCK) __builtin_amdgcn_s_barrier();
        load_block(__builtin_amdgcn_readlane(id, j + 1), B);
        consume(A, (cb + j) * BS, MASKED);
        if constexpr (LOCK) __builtin_amdgcn_s_barrier();
        load_block(__builtin_amdgcn_readlane(id, j + 2), A);
        consume(B, (cb + j + 1) * BS, MASKED);
      }
      if (j + 1 < n) {
        if constexpr (LOCK) __builtin_amdgcn_s_barrier();
        load_block(__builtin_amdgcn_readlane(id, j + 1), B);
        consume(A, (cb + j) * BS, MASKED);
        consume(B, (cb + j + 1) * BS, MASKED);
      } else {
        consume(A, (cb + j) * BS, MASKED);
      }
    }
    return false;
  };
  const int split = min(max(mask_from, b_begin), b_end);
  if (run(std::false_type{}, b_begin, split)) return true;
  return run(std::true_type{}, split, b_end);
}

// Normalise and write the G heads of the segment: to `out` rows
// out_row0 + h (rec == nullptr), or as partial records rec + h * rec_stride.
template <class E, int D, int G>
__device__ __forceinline__ void mfma_finish(const MfmaState<D>& st, bool bad, void* __restrict__ out,
                                            int64_t out_row0, float* __restrict__ rec, int64_t rec_stride,
                                            float out_scale, int lane) {
  constexpr int VE = MfmaShape<D>::kVe;
  const int g = lane >> 4, c = lane & 15;
  const float l_head = rows_sum(st.l_part);                 // softmax sum of head l%16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;                                  // this lane's output row
    const float lh = __shfl(l_head, h);
    const float mh = __shfl(st.m_ref, h);
    if (h >= G) continue;
    const float inv = lh > 0.f ? out_scale / lh : 0.f;
    float o[VE];
#pragma unroll
    for (int T = 0; T < VE; ++T) o[T] = bad ? qnan() : st.acc[T][i] * inv;
    if (rec == nullptr) {
      store_run<E, VE>(out, (out_row0 + h) * D + VE * c, o);
    } else {
      float* r = rec + h * rec_stride;
      store_f32_run<VE>(r + kRecHead + VE * c, o);
      if (c == 0) {
        r[0] = bad ? qnan() : mh;
        r[1] = bad ? qnan() : lh;
      }
    }
  }
}

// ---- split-context path: work items (sequence, partition, head group),
// one wave per kv head of the group (hpw kv heads, as in the balanced split,
// so a block's heads are read together and the waves run in step).
// Workgroup b takes items b, b + grid, ... (the launch makes that two at
// most, and only when all items fit in one round; with head groups innermost
// and the grid a multiple of their number, the workgroups of one partition's
// head groups run side by side).  An item's partial record is written after
// the workgroup's next item has streamed: records written as items end were
// flushed to HBM in the middle of the K/V stream (8 x 32k tokens, 64/8
// heads: 185 -> 172 us).
// ws: partial records [num_seqs * num_heads * num_parts].
// queue (or nullptr): as in the vector-ALU launch, the grid is at most what
// the GPU holds at once and a workgroup takes its next item from the counter
// (thread 0 fetches it when the item starts; it reaches the other waves
// through LDS at the item's end, before its stores).
template <class E, class KV, int D, int G, bool NT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 8)))
pa_decode_mfma_kernel(void* __restrict__ out, const void* __restrict__ query,
                      const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                      const int* __restrict__ block_tables, const int* __restrict__ seq_lens,
                      int num_heads, int num_kv_heads, int max_blocks, int num_blocks,
                      float qk_scale, float v_scale, int part_tokens, int num_parts, int hpw,
                      int num_items, float* __restrict__ ws, int* __restrict__ queue) {
  constexpr int BS = kBlockSize;
  constexpr int REC = rec_floats<D>();
  __shared__ int s_tk[2];
  const int lane = threadIdx.x & 63;
  const int groups = num_kv_heads / hpw;
  const int64_t cap = min((int64_t)max_blocks * BS, (int64_t)num_parts * part_tokens);
  const bool queued = queue != nullptr;
  // 0, but not known to the compiler to be uniform (see the vector-ALU launch)
  int* const counter = queued ? queue + (int)__builtin_amdgcn_mbcnt_lo(0u, 0u) : nullptr;

  MfmaState<D> held;                          // the previous item's record, not yet written
  bool held_bad = false, have_held = false;
  float* held_rec = nullptr;
  int64_t held_row0 = 0;
  int parity = 0;
  for (int64_t item = blockIdx.x; item < num_items;) {   // 64-bit: item + grid may pass 2^31
    int tk = 0;
    if (queued && threadIdx.x == 0) tk = atomicAdd(counter, 1);
    auto next_item = [&]() {
      if (queued) {
        asm volatile("" : "+v"(tk) :: "memory");
        if (threadIdx.x == 0) s_tk[parity] = __builtin_amdgcn_readfirstlane(tk);
        __syncthreads();
        item = (int64_t)gridDim.x + s_tk[parity];
        parity ^= 1;
      } else {
        item += gridDim.x;
      }
    };
    int w = (int)item;
    const int kvh = (w % groups) * hpw + (int)(threadIdx.x >> 6);
    w /= groups;
    const int part = w % num_parts;
    const int s = w / num_parts;
    const int64_t row0 = (int64_t)s * num_heads + kvh * G;

    const int L = seq_lens[s];
    const bool bad_len = L < 0 || (int64_t)L > cap;
    const int nparts_seq = bad_len ? 1 : ceil_div(L, part_tokens);
    if (part >= (nparts_seq > 0 ? nparts_seq : 1)) {          // empty partition
      next_item();
      continue;
    }
    const bool final_write = nparts_seq <= 1;

    MfmaState<D> st;
    mfma_begin<KV, D, G>(st, query, row0, lane >> 4, lane & 15);
    const int t_begin = part * part_tokens;
    const int t_end = bad_len ? 0 : min(L, t_begin + part_tokens);
    bool bad = bad_len;
    if (!bad_len && t_end > t_begin)
      bad = mfma_segment<E, KV, D, NT, true>(st, k_cache, v_cache, block_tables + (int64_t)s * max_blocks,
                                             t_begin / BS, ceil_div(t_end, BS), t_end, num_blocks, num_kv_heads,
                                             kvh, qk_scale, lane);
    next_item();
    if (have_held) {
      mfma_finish<E, D, G>(held, held_bad, out, held_row0, held_rec, (int64_t)num_parts * REC, v_scale, lane);
      have_held = false;
    }
    if (final_write) {
      mfma_finish<E, D, G>(st, bad, out, row0, nullptr, (int64_t)num_parts * REC, v_scale, lane);
    } else {
      held = st;
      held_bad = bad;
      held_rec = ws + (row0 * num_parts + part) * REC;
      held_row0 = row0;
      have_held = true;
    }
  }
  if (have_held)
    mfma_finish<E, D, G>(held, held_bad, out, held_row0, held_rec, (int64_t)num_parts * REC, v_scale, lane);
}

// Multi-token rows: accumulator row r = 4*(l/16) + i is (token r/G, head
// r%G) of kv head kvh; rows of tokens >= nq are padding.  Whole rows go to
// out[(q_tok0 + token) * num_heads + kvh*G + head]; partial rows to records
// rec + r * rec_stride (16 per wave).
template <class E, int D, int G>
__device__ __forceinline__ void mfma_finish_rows(const MfmaState<D>& st, bool bad, void* __restrict__ out,
                                                 int q_tok0, int nq, int num_heads, int kvh,
                                                 float* __restrict__ rec, int64_t rec_stride, float out_scale,
                                                 int lane) {
  constexpr int VE = MfmaShape<D>::kVe;
  const int g = lane >> 4, c = lane & 15;
  const float l_head = rows_sum(st.l_part);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const float lh = __shfl(l_head, r);
    const float mh = __shfl(st.m_ref, r);
    if (r / G >= nq) continue;
    const float inv = lh > 0.f ? out_scale / lh : 0.f;
    float o[VE];
#pragma unroll
    for (int T = 0; T < VE; ++T) o[T] = bad ? qnan() : st.acc[T][i] * inv;
    if (rec == nullptr) {
      store_run<E, VE>(out, ((int64_t)(q_tok0 + r / G) * num_heads + kvh * G + r % G) * D + VE * c, o);
    } else {
      float* rr = rec + r * rec_stride;
      store_f32_run<VE>(rr + kRecHead + VE * c, o);
      if (c == 0) {
        rr[0] = bad ? qnan() : mh;
        rr[1] = bad ? qnan() : lh;
      }
    }
  }
}

// ---- balanced split (stream-K over the batch's blocks)

// Range of flattened blocks of workgroup `rank` (of nwg) when U blocks are
// split evenly: [rank*U/nwg, (rank+1)*U/nwg).
__host__ __device__ inline int sk_range_begin(int rank, int U, int nwg) {
  return (int)(((int64_t)rank * U) / nwg);
}

// Workgroup whose range holds flattened block u (u < U).
__host__ __device__ inline int sk_owner(int u, int U, int nwg) {
  return (int)((((int64_t)u + 1) * nwg - 1) / U);
}

// Exclusive prefix sums of the blocks per sequence into s_cum[0..num_seqs];
// sequences with an out-of-contract length count zero blocks.
__device__ inline void blocks_prefix_sum(const int* __restrict__ seq_lens, int num_seqs, int max_blocks,
                                         int* s_cum, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  int carry = 0;
  for (int base = 0; base < num_seqs; base += blockDim.x) {
    const int s = base + tid;
    int x = 0;
    if (s < num_seqs) {
      const int L = seq_lens[s];
      x = (L > 0 && (int64_t)L <= (int64_t)max_blocks * kBlockSize) ? ceil_div(L, kBlockSize) : 0;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
    for (int w2 = 0; w2 < nwaves; ++w2) {
      const int t = s_wsum[w2];
      before += w2 < wave ? t : 0;
      total += t;
    }
    if (s < num_seqs) s_cum[s + 1] = carry + before + x;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) s_cum[0] = 0;
  __syncthreads();
}

// Grid: head_groups * nwg workgroups of hpw waves (kv heads hg*hpw + wave).
// Dynamic LDS: (num_seqs + 1) ints, twice that with MQ.  ws_seq[s] (written by head group 0):
// {w1, first block, end block, total blocks} where w1 is the range holding
// the sequence's first block if the sequence runs past that range's end, -1
// otherwise (written whole here, or no blocks).  ws_rec: partial records, 2
// slots per workgroup (first and last segment of its range) * hpw * G heads.
// Workgroup `rank` also writes the rows of the sequences s = rank (mod nwg)
// that have no blocks: zeros for length 0, NaN for an out-of-contract length.
// A workgroup is up to 8 waves; 12 wave slots per CU would still hold only
// one, so the register budget is that of 2 waves per SIMD.
// MQ: several query tokens per sequence (query_start[s] .. query_start[s+1]),
// at most 16 * TILES / G: the wave of a kv head holds TILES 16-row tiles of
// its (token, head) pairs (tile t: rows 16t .. 16t + 15) and feeds each
// loaded block to all of them, so every K/V line is read once.  The
// sequence's final blocks are masked per row (causal), partial records hold
// 16 * TILES rows per kv head, and pa_sk_merge_mq_kernel merges them.
// Two 16-row tiles of 128-wide heads need more than the 256 registers of two
// waves per SIMD: that launch gives each wave a SIMD of its own (at most 4
// kv heads per workgroup).
template <int D, int TILES> constexpr bool sk_wide() { return TILES == 2 && D == 128; }
constexpr int kSkWideHeads = 4;

template <class E, class KV, int D, int G, bool NT, bool MQ = false, int TILES = 1>
__global__ void __launch_bounds__((sk_wide<D, TILES>() ? 64 * kSkWideHeads : 512))
__attribute__((amdgpu_waves_per_eu(sk_wide<D, TILES>() ? 1 : 2, sk_wide<D, TILES>() ? 1 : 8)))
pa_decode_sk_kernel(void* __restrict__ out, const void* __restrict__ query,
                    const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                    const int* __restrict__ block_tables, const int* __restrict__ seq_lens,
                    int num_seqs, int num_heads, int num_kv_heads, int max_blocks, int num_blocks,
                    float qk_scale, float v_scale, int hpw, int nwg, int4* __restrict__ ws_seq,
                    float* __restrict__ ws_rec, const int* __restrict__ query_start = nullptr) {
  constexpr int BS = kBlockSize;
  constexpr int REC = rec_floats<D>();
  constexpr int RPK = MQ ? 16 * TILES : G;     // record rows per kv head and slot
  extern __shared__ int s_cum[];
  __shared__ int s_wsum[16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hg = blockIdx.x / nwg, rank = blockIdx.x - hg * nwg;
  const int kvh = hg * hpw + wv;

  blocks_prefix_sum(seq_lens, num_seqs, max_blocks, s_cum, s_wsum);
  int* s_qs = s_cum + num_seqs + 1;            // MQ: query_start staged in LDS
  if constexpr (MQ) {
    for (int i = tid; i <= num_seqs; i += blockDim.x) s_qs[i] = query_start[i];
    __syncthreads();
  }
  const int U = s_cum[num_seqs];
  const int u0 = sk_range_begin(rank, U, nwg), u1 = sk_range_begin(rank + 1, U, nwg);
  if (hg == 0 && u0 < u1) {
    int lo = -1, hi = num_seqs;                // first sequence with s_cum[s] >= u0: hi
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] >= u0) hi = mid; else lo = mid;
    }
    for (int s = hi + tid; s < num_seqs && s_cum[s] < u1; s += blockDim.x) {
      const int c0 = s_cum[s], c1 = s_cum[s + 1];
      if (c1 > c0) ws_seq[s] = int4{c1 > u1 ? rank : -1, c0, c1, U};
    }
  }
  for (int s = rank; s < num_seqs; s += nwg) {
    if (s_cum[s + 1] != s_cum[s]) continue;
    if (hg == 0 && tid == 0) ws_seq[s] = int4{-1, 0, 0, U};
    if constexpr (MQ) {                        // query rows of a sequence without blocks break the contract
      const int a = s_qs[s], nq = s_qs[s + 1] - a;
      for (int t = 0; t < nq; ++t) {
        const int64_t e0 = ((int64_t)(a + t) * num_heads + kvh * G) * D;
        for (int i = lane; i < G * D; i += 64) store_elem<E>(out, e0 + i, qnan());
      }
    } else {
      const float v = seq_lens[s] == 0 ? 0.f : qnan();
      const int64_t e0 = ((int64_t)s * num_heads + kvh * G) * D;
      for (int i = lane; i < G * D; i += 64) store_elem<E>(out, e0 + i, v);
    }
  }
  if (u0 >= u1) return;

  // first sequence: the last s with s_cum[s] <= u0 (then s_cum[s + 1] > u0)
  int lo = 0, hi = num_seqs;                 // invariant: s_cum[lo] <= u0 < s_cum[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_cum[mid] <= u0) lo = mid; else hi = mid;
  }
  int s = lo;
  float* rec_wg = ws_rec + ((int64_t)blockIdx.x * 2 * hpw + wv) * RPK * REC;
  // The record of a first segment that ends inside the range is held in
  // registers and written after the range's last segment: records written
  // early are flushed to HBM in the middle of the K/V stream (4 rows per
  // wave: 8B batch 248.8 -> 245.0 us; 16 rows per wave, where the records
  // outgrow an XCD's L2: 288 -> 260 us).
  MfmaState<D> held[MQ ? TILES : 1];
  bool held_bad = false, have_held = false;
  int held_a = 0, held_nq = 0;
  int64_t held_row0 = 0;
  for (int u = u0; u < u1;) {
    const int c0 = s_cum[s], c1 = s_cum[s + 1];
    if (c1 == c0) { ++s; continue; }
    const int b0 = u - c0, b1 = min(c1, u1) - c0;
    const int L = seq_lens[s];
    const bool whole = b0 == 0 && b1 == c1 - c0;
    float* rec = whole ? nullptr : rec_wg + (u == u0 ? 0 : (int64_t)hpw * RPK * REC);
    if constexpr (MQ) {
      const int a = s_qs[s], nq = s_qs[s + 1] - a;
      if (nq > 0) {                            // same for every wave of the workgroup
        const int g = lane >> 4, c = lane & 15;
        MfmaState<D> st[TILES];
        int row_last[TILES];
#pragma unroll
        for (int t = 0; t < TILES; ++t) {      // tile t: tokens 16t/G + r/G (rows past nq are padding)
          const int tok = 16 * t / G + c / G;
          const bool live = tok < nq;
          mfma_begin_row<KV, D>(st[t], query, (int64_t)(a + (live ? tok : 0)) * num_heads + kvh * G + c % G, live,
                                g);
          row_last[t] = L - nq + min(tok, nq - 1);
        }
        bool bad = nq > L;
        if (!bad)
          bad = mfma_segment_rows<E, KV, D, NT, true, TILES>(st, k_cache, v_cache,
                                                             block_tables + (int64_t)s * max_blocks, b0, b1,
                                                             (L - nq + 1) / BS, row_last, L - 1, num_blocks,
                                                             num_kv_heads, kvh, qk_scale, lane);
        const bool hold = u == u0 && rec != nullptr && c1 < u1;      // first segment, not the range's last
        if (hold) {
#pragma unroll
          for (int t = 0; t < TILES; ++t) held[t] = st[t];
          held_bad = bad;
          held_a = a;
          held_nq = nq;
          have_held = true;
        } else {
#pragma unroll
          for (int t = 0; t < TILES; ++t) {
            const int t0 = 16 * t / G;
            mfma_finish_rows<E, D, G>(st[t], bad, out, a + t0, nq - t0, num_heads, kvh,
                                      rec != nullptr ? rec + 16 * t * REC : nullptr, REC, v_scale, lane);
          }
        }
      }
    } else {
      const int64_t row0 = (int64_t)s * num_heads + kvh * G;
      MfmaState<D> st;
      mfma_begin<KV, D, G>(st, query, row0, lane >> 4, lane & 15);
      const bool bad = mfma_segment<E, KV, D, NT, true>(st, k_cache, v_cache, block_tables + (int64_t)s * max_blocks,
                                                        b0, b1, min(L, b1 * BS), num_blocks, num_kv_heads, kvh,
                                                        qk_scale, lane);
      if (u == u0 && rec != nullptr && c1 < u1) {
        held[0] = st;
        held_bad = bad;
        held_row0 = row0;
        have_held = true;
      } else {
        mfma_finish<E, D, G>(st, bad, out, row0, rec, REC, v_scale, lane);
      }
    }
    u += b1 - b0;
    ++s;
  }
  if (have_held) {
    if constexpr (MQ) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int t0 = 16 * t / G;
        mfma_finish_rows<E, D, G>(held[t], held_bad, out, held_a + t0, held_nq - t0, num_heads, kvh,
                                  rec_wg + 16 * t * REC, REC, v_scale, lane);
      }
    } else {
      mfma_finish<E, D, G>(held[0], held_bad, out, held_row0, rec_wg, REC, v_scale, lane);
    }
  }
}

// ---- multi-token queries (chunked prefill, speculative verification)

// Grid (ceil(max_tiles / 4), num_seqs, num_kv_heads); 4 waves, wave w owns
// query tile 4*blockIdx.x + w of the sequence: rows r = 0..15 are (token
// tile*16/G + r/G, query head kvh*G + r%G).  Tiles past the sequence's query
// rows exit.  Token i of the n query rows sits at position L - n + i and sees
// positions 0 .. L - n + i.  Out-of-contract lengths (n > L, L past the table
// row) or block ids give NaN rows.
template <class E, class KV, int D, int G, bool NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
pa_prefill_kernel(void* __restrict__ out, const void* __restrict__ query, const char* __restrict__ k_cache,
                  const char* __restrict__ v_cache, const int* __restrict__ block_tables,
                  const int* __restrict__ seq_lens, const int* __restrict__ query_start, int num_heads,
                  int num_kv_heads, int max_blocks, int num_blocks, float qk_scale, float v_scale) {
  using SH = MfmaShape<D>;
  using IO = KvIo<KV, ElemBF16, D>;
  constexpr int BS = kBlockSize, TPT = 16 / G, VE = SH::kVe;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x * 4 + wave, s = blockIdx.y, kvh = blockIdx.z;
  const int q0 = query_start[s], n = query_start[s + 1] - q0, L = seq_lens[s];
  const int tok0 = tile * TPT;
  if (n <= 0 || tok0 >= n) return;
  const bool bad_len = n > L || (int64_t)L > (int64_t)max_blocks * BS;
  const int g = lane >> 4, c = lane & 15;

  // this lane's row c: token tok0 + c/G (padding rows past n reuse the last token's limit)
  const int my_tok = tok0 + c / G;
  const bool row_live = my_tok < n;
  MfmaState<D> sts[1];
  MfmaState<D>& st = sts[0];
  mfma_begin_row<KV, D>(st, query, (int64_t)(q0 + (row_live ? my_tok : 0)) * num_heads + kvh * G + c % G, row_live, g);
  bool bad = bad_len;
  if (!bad_len) {
    const int first_pos = L - n + tok0;                          // the tile's smallest limit
    const int last_pos = L - n + min(tok0 + TPT, n) - 1;          // and largest
    const int row_last[1] = {L - n + min(my_tok, n - 1)};
    bad = mfma_segment_rows<E, KV, D, NT, false, 1>(sts, k_cache, v_cache, block_tables + (int64_t)s * max_blocks,
                                                     0, last_pos / BS + 1, (first_pos + 1) / BS, row_last, L - 1,
                                                     num_blocks, num_kv_heads, kvh, qk_scale, lane);
  }
  // rows r = 4*(l/16) + i of the accumulator: token tok0 + r/G, head r%G
  const float l_row = rows_sum(st.l_part);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const float lr = __shfl(l_row, r);
    const int tok = tok0 + r / G;
    if (tok >= n) continue;
    const float inv = lr > 0.f ? v_scale / lr : 0.f;
    float o[VE];
#pragma unroll
    for (int T = 0; T < VE; ++T) o[T] = bad ? qnan() : st.acc[T][i] * inv;
    store_run<E, VE>(out, ((int64_t)(q0 + tok) * num_heads + kvh * G + r % G) * D + VE * c, o);
  }
}

// ---- multi-token queries, K/V shared through LDS

// LDS stage of kPfStageBlocks blocks, K rows then V rows, 16-bit elements
// whatever the pool type, each region row-major at a padded pitch:
//  * K (pitch 2D + 32): each lane reads 16 bytes of one of 16 rows for a QK
//    operand; the counters show no bank conflicts at this pitch (at 2D + 16:
//    0.40 conflict cycles per LDS access, the LDS busy 34 % instead of 24 %);
//  * V (pitch 2D + 32): the PV operands come from transposing reads, where 8
//    rows x 32 bytes are read together; a 32-byte shift per row keeps those
//    in different banks.
constexpr int kPfStageBlocks = 4;
template <int D> constexpr int pf_k_pitch() { return D * 2 + 32; }
template <int D> constexpr int pf_v_pitch() { return D * 2 + 32; }
template <int D> constexpr int pf_k_bytes() { return kPfStageBlocks * kBlockSize * pf_k_pitch<D>(); }
template <int D> constexpr int pf_stage_bytes() { return kPfStageBlocks * kBlockSize * (pf_k_pitch<D>() + pf_v_pitch<D>()); }

// Transposing LDS read (gfx950): in each 16-lane group, lane 4j + q gives the
// address of 4 consecutive 16-bit elements (row j, columns 4q..4q+3 of a
// 4 x 16 tile); lane i gets back column i, rows 0..3.  That is the B operand
// of a matrix-core step over 4 consecutive k from a row-major [k][n] tile.
__device__ inline u32x2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Query tiles of one pa_prefill_lds_kernel workgroup (TPG) and per wave (TW).
// TW = 2 is built (two waves per SIMD); TW = 4 (one wave per SIMD, the
// accumulators in AGPRs) measured slower.  TPG = 16 (8 waves) for many
// tiles per (sequence, kv head), TPG = 8 (4 waves, two workgroups per CU)
// when a (sequence, kv head) has at most 8 tiles, so fewer waves idle; with
// very few tiles TW = 1, TPG = 4 (4 waves of one tile).
constexpr int kPfTilesPerWave = 2;
constexpr int kPfSmallGroupTiles = 8;

// Grid: one workgroup of TPG / TW waves per (sequence, kv head, TPG
// consecutive query tiles); wave w owns tiles TPG*grp + TW*w .. TW*w + TW - 1
// (16 (token, head) rows each, as in pa_prefill_kernel).  The workgroup
// streams the sequence's blocks in stages of kPfStageBlocks, double-buffered
// in LDS with one barrier per stage: the waves copy the next stage's K and V
// blocks (8 waves: one block of K (w < 4) or V each; 4 waves: block w of K
// and of V), while every wave consumes the current stage's blocks it can see,
// two blocks per step, all of its tiles on each operand read from LDS:
//   QK: TW 16-key score tiles per block (16x16x32 MFMAs over head_size);
//   PV: one 16x16x32 MFMA per 16 output columns over the pair's 32 keys, and
//       one more against a column of ones, which sums each row's weights as
//       rounded for the PV step (the softmax denominator).
// Each K/V byte is read from memory once per TPG tiles instead of once per
// tile, and from LDS once per TW tiles.  Rows past the sequence end, blocks
// past the workgroup's last block and out-of-pool block ids load as zeros
// (the buffer range of the block is cut to its valid rows).  The linear
// workgroup id is split so that all workgroups of one (sequence, kv head)
// land on the same XCD (workgroups are dealt to the 8 XCDs round robin),
// where its K/V stay in that XCD's L2.  order: nullptr, or the sequence each
// sequence index stands for (a permutation: longest first).
template <class E, class KV, int D, int G, bool NT, int TW, int TPG>
__global__ void __launch_bounds__(64 * TPG / TW)
__attribute__((amdgpu_waves_per_eu(TW == 4 ? 1 : 2, TW == 4 ? 1 : 8)))
pa_prefill_lds_kernel(void* __restrict__ out, const void* __restrict__ query, const char* __restrict__ k_cache,
                      const char* __restrict__ v_cache, const int* __restrict__ block_tables,
                      const int* __restrict__ seq_lens, const int* __restrict__ query_start, int num_seqs,
                      int num_heads, int num_kv_heads, int max_blocks, int num_blocks, int groups_per_pair,
                      float qk_scale, float v_scale, const int* __restrict__ order) {
  using SH = MfmaShape<D>;
  using M = Mfma<E>;
  constexpr int BS = kBlockSize, TPT = 16 / G, KS = SH::kKs, VE = SH::kVe;
  constexpr int WAVES = TPG / TW;
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves per workgroup");
  static_assert(TW == 1 || TW == 2 || TW == 4, "one, two or four tiles per wave");
  constexpr int RP = pf_k_pitch<D>(), VP = pf_v_pitch<D>(), KB = pf_k_bytes<D>(), SB = pf_stage_bytes<D>();
  constexpr int KVB = KV::kBytes;                     // bytes per element in the pools
  constexpr int CPR = D * KVB / 16;                   // 16-byte chunks per pool row
  constexpr int DPC = 16 / KVB;                       // elements per chunk
  constexpr int KC = CPR / 4;                         // chunks per lane and block: 16 rows per block
  constexpr int JOBS = 2 * kPfStageBlocks / WAVES;    // blocks (of K or V) each wave copies per stage
  static_assert(kPfStageBlocks == 4 && KC >= 1, "stage layout");
  __shared__ __align__(16) char smem[2 * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets block loads use SGPR descriptors
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int pair = (slot / groups_per_pair) * 8 + xcd, grp = slot % groups_per_pair;
  if (pair >= num_seqs * num_kv_heads) return;
  const int si = pair / num_kv_heads, kvh = pair - si * num_kv_heads;
  const int s = order != nullptr ? order[si] : si;
  const int q0 = query_start[s], n = query_start[s + 1] - q0, L = seq_lens[s];
  const int wg_tok0 = grp * TPG * TPT;
  if (n <= 0 || wg_tok0 >= n) return;                // the whole workgroup: uniform
  const bool bad_len = n > L || (int64_t)L > (int64_t)max_blocks * BS;

  const int g = lane >> 4, c = lane & 15;
  const int tok0 = wg_tok0 + wave * TW * TPT;          // first token of the wave's tiles
  const bool active = tok0 < n && !bad_len;
  // scores are scaled after the max (one multiply per row instead of one per
  // score), which needs a non-negative scale: a negative one moves its sign
  // into the query (exact)
  const uint32_t q_sign = qk_scale < 0.f ? 0x80008000u : 0u;
  qk_scale = fabsf(qk_scale);
  MfmaState<D> st[TW];
  f32x4 acc_l[TW];                                    // row sums of the rounded weights, rows as acc
  int row_last[TW];                                   // last visible key of this lane's row l%16, per tile
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int my_tok = tok0 + t * TPT + c / G;
    const bool row_live = my_tok < n;
    mfma_begin_row<Kv16, D>(st[t], query, (int64_t)(q0 + (row_live ? my_tok : 0)) * num_heads + kvh * G + c % G,
                            row_live, g);
#pragma unroll
    for (int k = 0; k < KS; ++k) st[t].qb[k] ^= q_sign;
    acc_l[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    row_last[t] = L - n + min(my_tok, n - 1);
  }
  const u32x4 ones = {M::kOnes, M::kOnes, M::kOnes, M::kOnes};
  const float inf = opaque_inf();
  // a tile rescales when a lane maximum (raw) exceeds thr = (m_ref + 8) / scale
  // (the threshold is a heuristic: rounding here changes nothing but when
  // the exact re-association happens); updated with m_ref
  const float inv_scale = 1.f / qk_scale;
  float thr[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) thr[t] = -INFINITY;
  const int my_first = L - n + tok0, my_last = L - n + min(tok0 + TW * TPT, n) - 1;
  const int my_b_end = active ? my_last / BS + 1 : 0;
  const int my_p_end = (my_b_end + 1) / 2;            // block pairs this wave consumes
  const int my_p_open = ((my_first + 1) / BS) / 2;    // pairs before this one are visible to every row
  const int wg_last = L - n + min(wg_tok0 + TPG * TPT, n) - 1;
  const int wg_b_end = bad_len ? 0 : wg_last / BS + 1;
  const int* bt_row = block_tables + (int64_t)s * max_blocks;

  // staging jobs of this wave: block sblk of every stage, of K and/or V
  const int sblk = wave & 3;
  auto v_job = [&](int j) { return WAVES == 4 ? j == 1 : wave >= 4; };   // j is unrolled: folds for 4 waves
  const int row_stride = num_kv_heads * D * KVB;
  const int blk_bytes = BS * row_stride;
  const int head_off = kvh * D * KVB;
  int voff[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int q = lane + 64 * i;                      // chunk: row q / CPR, column q % CPR
    voff[i] = (q / CPR) * row_stride + head_off + (q % CPR) * 16;
  }

  u32x4 regs[JOBS][KC];
  int ids = 0;                                        // block ids of the current window of 64 blocks
  bool bad_id = false;
  auto issue = [&](int stage) {
    if ((stage & (64 / kPfStageBlocks - 1)) == 0) {   // the stage starts a new window
      const int idx = stage * kPfStageBlocks + lane;
      ids = idx < wg_b_end ? bt_row[idx] : 0;
      bad_id |= __ballot(idx < wg_b_end && (unsigned)ids >= (unsigned)num_blocks) != 0;
    }
    const int bi = stage * kPfStageBlocks + sblk;
    const int id = __builtin_amdgcn_readlane(ids, bi & 63);
    const bool ok = bi < wg_b_end && (unsigned)id < (unsigned)num_blocks;
    const int rows = ok ? min(BS, L - bi * BS) : 0;
#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
      const char* pool = v_job(j) ? v_cache : k_cache;
      const __amdgpu_buffer_rsrc_t r = block_rsrc(pool + (int64_t)(ok ? id : 0) * blk_bytes, rows * row_stride);
#pragma unroll
      for (int i = 0; i < KC; ++i) regs[j][i] = load16<NT>(r, voff[i], 0);
    }
  };
  // word w (elements 2w, 2w+1) of a staged chunk as 16-bit elements
  auto word = [&](const u32x4& x, int w) -> uint32_t {
    if constexpr (KVB == 2) return x[w];
    else return (w & 1) ? fp8x2_to<E, true>(x[w >> 1]) : fp8x2_to<E, false>(x[w >> 1]);
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < JOBS; ++j) {
      const bool vr = v_job(j);
      char* sb = smem + buf * SB + (vr ? KB : 0);
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int q = lane + 64 * i;
        char* dst = sb + (sblk * BS + q / CPR) * (vr ? VP : RP) + (q % CPR) * DPC * 2;
        const u32x4& x = regs[j][i];
#pragma unroll
        for (int h = 0; h < DPC / 8; ++h)
          *reinterpret_cast<u32x4*>(dst + 16 * h) =
              u32x4{word(x, 4 * h), word(x, 4 * h + 1), word(x, 4 * h + 2), word(x, 4 * h + 3)};
      }
    }
  };

  // A step covers blocks 2p, 2p+1 of a stage for all tiles (key0: position
  // of block 2p's first key), in three parts: scores (QK and the lane maxima),
  // rescale (rare: one branch for all tiles) and weights_pv (exponentials
  // and PV).  Every row sees key 0, and the first pair is consumed before any
  // other, so m_ref is finite whenever weights are taken.
  // raw scores: lane l holds row l%16, keys key0 + 16*(i/4) + 4*(l/16) + i%4
  struct Scores {
    float z[TW][8];
    float zl[TW];                                     // this lane's maximum (raw); its row's is over 4 lanes
    bool vis[TW][8];                                  // visible keys (masked steps)
  };
  struct KOps { u32x4 a[KS], b[KS]; };                // K operands of blocks 2p and 2p+1
  auto k_read = [&](const char* sbuf, int p, KOps& x) {
    const char* ka = sbuf + 2 * p * BS * RP + c * RP + 16 * g;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      x.a[k] = *reinterpret_cast<const u32x4*>(ka + 64 * k);
      x.b[k] = *reinterpret_cast<const u32x4*>(ka + BS * RP + 64 * k);
    }
  };
  // B operand of output columns d = 16T + c: V rows 4g..4g+3 of both blocks
  auto v_read = [&](const char* sbuf, int p, u32x4* vb) {
    const char* va = sbuf + KB + (2 * p * BS + 4 * g + (c >> 2)) * VP + 8 * (c & 3);
#pragma unroll
    for (int T = 0; T < VE; ++T) {
      const u32x2 x = lds_read_tr16(va + 32 * T), y = lds_read_tr16(va + BS * VP + 32 * T);
      vb[T] = u32x4{x[0], x[1], y[0], y[1]};
    }
  };
  auto qk = [&](int t, const KOps& x, Scores& r) {
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      sa = M::qk(x.a[k], st[t].qb[k], sa);
      sb = M::qk(x.b[k], st[t].qb[k], sb);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.z[t][i] = sa[i];
      r.z[t][4 + i] = sb[i];
    }
  };
  auto maxima = [&](auto masked_tag, int t, int key0, Scores& r) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r.vis[t][i] = !MASKED || key0 + 16 * (i >> 2) + 4 * g + (i & 3) <= row_last[t];
      if (MASKED && !r.vis[t][i]) r.z[t][i] = -INFINITY;
    }
    r.zl[t] =
        max_nonan(max_nonan(max_nonan(r.z[t][0], r.z[t][1], inf), max_nonan(r.z[t][2], r.z[t][3], inf), inf),
                  max_nonan(max_nonan(r.z[t][4], r.z[t][5], inf), max_nonan(r.z[t][6], r.z[t][7], inf), inf), inf);
  };
  // A row's maximum beats its reference by the threshold iff one of its four
  // lanes' maxima does, so the (rare) rescale decides on the lane maxima and
  // only then reduces them across the row's lanes.
  auto rescale = [&](const Scores& r) {
    bool up[TW], any = false;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      up[t] = r.zl[t] > thr[t];
      any = any || up[t];
    }
    if (__ballot(any)) {
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        if (!__ballot(up[t])) continue;
        const float bm = rows_max_nonan(r.zl[t], inf) * qk_scale;       // row maxima, scaled
        const float m_new = fmaxf(st[t].m_ref, bm);
        const float alpha = __builtin_amdgcn_exp2f(st[t].m_ref - m_new);   // 0 on the first pair
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int T = 0; T < VE; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[t].acc[T][i] *= ar[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_l[t][i] *= ar[i];
        st[t].m_ref = m_new;
        thr[t] = (m_new + kRescaleThreshold) * inv_scale;
      }
    }
  };
  auto weights = [&](auto masked_tag, int t, const Scores& r) -> u32x4 {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float p8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = fmaf(r.z[t][i], qk_scale, -st[t].m_ref);
      p8[i] = __builtin_amdgcn_exp2f(MASKED && !r.vis[t][i] ? -INFINITY : e);
    }
    return u32x4{pack2<E>(p8[0], p8[1]), pack2<E>(p8[2], p8[3]), pack2<E>(p8[4], p8[5]), pack2<E>(p8[6], p8[7])};
  };
  auto pv = [&](int t, const u32x4& pa, const u32x4* vb) {
#pragma unroll
    for (int T = 0; T < VE; ++T) st[t].acc[T] = M::qk(pa, vb[T], st[t].acc[T]);
    acc_l[t] = M::qk(pa, ones, acc_l[t]);
  };
  // one step over a pair, not pipelined
  auto step = [&](auto masked_tag, const char* sbuf, int p, int key0) {
    Scores r;
    KOps x;
    k_read(sbuf, p, x);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      qk(t, x, r);
      maxima(masked_tag, t, key0, r);
    }
    rescale(r);
    u32x4 vb[VE];
    v_read(sbuf, p, vb);
#pragma unroll
    for (int t = 0; t < TW; ++t) pv(t, weights(masked_tag, t, r), vb);
  };

  const int stages = (wg_b_end + kPfStageBlocks - 1) / kPfStageBlocks;
  issue(0);                                           // with no blocks at all it loads zeros
  commit(0);
  // nothing of this wave's memory reads may stay in flight into the stage
  // loop (the query rows included): the loop's only loads are the next stage's
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int stg = 0; stg < stages; ++stg) {
    if (stg + 1 < stages) issue(stg + 1);
    const char* sbuf = smem + (stg & 1) * SB;
    const int p_lo = stg * (kPfStageBlocks / 2), p_hi = min(p_lo + kPfStageBlocks / 2, my_p_end);
    const int p_mid = min(max(my_p_open, p_lo), p_hi);
    // pairs every row sees, software-pipelined: the exponentials and PV of
    // one pair and the QK and maxima of the next form one scheduling region,
    // ordered so that each group of vector instructions has matrix-core work
    // of another tile or pair beside it
    if (p_lo < p_mid) {
      Scores cur;
      {
        KOps x;
        k_read(sbuf, 0, x);
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          qk(t, x, cur);
          maxima(std::false_type{}, t, 0, cur);
        }
      }
#pragma unroll 1
      for (int p = p_lo; p + 1 < p_mid; ++p) {
        rescale(cur);
        Scores nxt;
        KOps x;
        u32x4 vb[VE];
        v_read(sbuf, p - p_lo, vb);
        k_read(sbuf, p + 1 - p_lo, x);
        // the matrix-core groups run at raised wave priority, so while one
        // wave of the SIMD issues them the other's vector work fills the
        // gaps (chunked-prefill batch: 265.9 -> 259.8 us on one box)
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          const u32x4 pa = weights(std::false_type{}, t, cur);
          __builtin_amdgcn_s_setprio(1);
          qk(t, x, nxt);
          __builtin_amdgcn_s_setprio(0);
          if (t > 0) maxima(std::false_type{}, t - 1, 0, nxt);
          __builtin_amdgcn_s_setprio(1);
          pv(t, pa, vb);
          __builtin_amdgcn_s_setprio(0);
        }
        maxima(std::false_type{}, TW - 1, 0, nxt);
        cur = nxt;
      }
      rescale(cur);
      u32x4 vb[VE];
      v_read(sbuf, p_mid - 1 - p_lo, vb);
#pragma unroll
      for (int t = 0; t < TW; ++t) pv(t, weights(std::false_type{}, t, cur), vb);
    }
    // pairs on the causal diagonal
#pragma unroll 1
    for (int p = p_mid; p < p_hi; ++p) step(std::true_type{}, sbuf, p - p_lo, p * 2 * BS);
    if (stg + 1 < stages) commit((stg + 1) & 1);
    __syncthreads();
  }
  const bool bad = bad_len || __syncthreads_or(bad_id);

#pragma unroll
  for (int t = 0; t < TW; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i;                        // rows r of the accumulators: token r/G of the tile, head r%G
      const int tok = tok0 + t * TPT + r / G;
      if (tok >= n) continue;
      const float inv = acc_l[t][i] > 0.f ? v_scale / acc_l[t][i] : 0.f;
      const int64_t o0 = ((int64_t)(q0 + tok) * num_heads + kvh * G + r % G) * D + c;
#pragma unroll
      for (int T = 0; T < VE; ++T) store_elem<E>(out, o0 + 16 * T, bad ? qnan() : st[t].acc[T][i] * inv);
    }
  }
}

}  // namespace pa
