// Paged decode on the vector ALUs (fp32 KV, and 16-bit or fp8 KV with one
// query head per kv head, where a matrix-core tile would be 1/16 dense).
//
// One 64-lane wave (one workgroup) per work item (sequence, kv head, chunk of
// tokens; with part_tokens == 0 the chunk is the whole sequence):
//  * Gather loader: the item's block ids are read one per lane and broadcast
//    with readlane.  One row of one head (head_size * elem bytes) is read by
//    LPR lanes with 16-byte buffer loads, so one load instruction covers
//    64/LPR token rows and a block is NI = 16 / (64/LPR) instructions per
//    cache.  Two register sets alternate so the next block is in flight while
//    the current one is consumed.
//  * Scores: q stays in registers; each lane forms partial dots of its
//    16-byte slice for all G query heads of the group, so each K byte is read
//    once per kv head.  A halving butterfly over the LPR lanes (DPP row/half
//    mirror and quad permutes) leaves every score on one lane.
//  * Online softmax (base 2, scale * log2(e) applied to the score) per
//    "sub-wave" (the LPR lanes that share token rows); probabilities and
//    rescale factors go through a small LDS buffer of the wave so every lane
//    can weight its V slice; PV accumulates in fp32 registers.
//  * At the end the sub-waves are merged with log-sum-exp weights.
//  * Masking uses selects only (the pool may hold NaN in dead slots).
//  * fp8 (e4m3) pools: a 16-byte load holds 16 codes of a row; K codes are
//    widened in pairs to the query type for the dot products, V codes to
//    fp32; the pool scales enter the score scale (K) and the final
//    normalisation (V).
#pragma once

#include "common.h"

namespace pa {

template <class E, class KV, int D, int G>
struct ValuCfg {
  static constexpr bool kFp8 = std::is_same<KV, KvFp8>::value;
  static constexpr int kKvBytes = kFp8 ? 1 : E::kBytes;   // bytes per pool element
  static constexpr int kRow = D * kKvBytes;         // bytes of one token row of one head in the pools
  static constexpr int kQRow = D * E::kBytes;       // ... of the query
  static constexpr int kLpr = kRow / 16;            // lanes per row
  static constexpr int kRpi = 64 / kLpr;            // rows per load instruction
  static constexpr int kNi = kBlockSize / kRpi;     // load instructions per block
  static constexpr int kEpl = 16 / kKvBytes;        // elements per lane per instruction
  static constexpr int kQw = kEpl * E::kBytes / 16; // 16-byte query chunks per lane and head
  static constexpr int kNv = kNi * G;               // partial scores per lane per block
  static constexpr int kNvl = kNv > kLpr ? kNv / kLpr : 1;
  static constexpr int kNh = ilog2(kNv < kLpr ? kNv : kLpr);
  static constexpr int kPStride = round_up4(kNv + G);
  static_assert(kLpr >= 4 && kLpr <= 32, "row must span 4..32 lanes");
  static_assert(kBlockSize % kRpi == 0 && kNi == kLpr / 4, "block must be whole load instructions");
  static_assert(D % 64 == 0, "head_size must be a multiple of 64");
};

// Most kv heads (waves) per workgroup of the queued vector-ALU launch (fp8
// 13B-shaped batch: 8 heads 140.2 us, 4 heads 141.7, 2 heads 175.2).
constexpr int kValuMaxHeadsPerWg = 8;

template <class E, class KV, int D, int G>
struct ValuOccupancy {
  // 3 waves per SIMD need <= 168 VGPRs, which 16-bit pools with head_size 64
  // meet up to G = 4; 128-wide 16-bit rows (three blocks of K and V in
  // registers), fp8 rows and 64-wide fp32 rows take 2
  static constexpr bool k16 = E::kBytes == 2 && !std::is_same<KV, KvFp8>::value;
  static constexpr int kWaves = G > 4 ? 1 : (k16 && D == 64) ? 3 : (E::kBytes == 2 || D == 64) ? 2 : 1;
};

// Dot product of a lane's query chunks with one 16-byte chunk of a K row.
template <class E, class KV>
__device__ inline float dot_chunk(const u32x4* q, const u32x4& k) {
  if constexpr (std::is_same<KV, KvFp8>::value) {
    // 16 codes; code pair (2j, 2j+1) against query dword j
    const uint32_t qw[8] = {q[0][0], q[0][1], q[0][2], q[0][3], q[1][0], q[1][1], q[1][2], q[1][3]};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = dot2<E>(qw[2 * j], fp8x2_to<E, false>(k[j]), acc);
      acc = dot2<E>(qw[2 * j + 1], fp8x2_to<E, true>(k[j]), acc);
    }
    return acc;
  } else {
    return dot16<E>(q[0], k, 0.f);
  }
}

// One 16-byte chunk of a V row as fp32.
template <class E, class KV>
__device__ inline void widen_chunk(const u32x4& v, float* f) {
  if constexpr (std::is_same<KV, KvFp8>::value) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)v[j], 1.0f, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)v[j], 1.0f, true);
      f[4 * j] = lo.x;
      f[4 * j + 1] = lo.y;
      f[4 * j + 2] = hi.x;
      f[4 * j + 3] = hi.y;
    }
  } else {
    widen16<E>(v, f);
  }
}

// ws: partial records [num_seqs * num_heads * num_parts] (split mode only).
// NT: K/V loads with the non-temporal policy (blocks read once per call).
// v_scale multiplies the output (the V pool's scale; 1 for 16-bit pools).
// A workgroup is hpw = blockDim.x / 64 waves, one per kv head of a head group
// (kv heads hg * hpw + wave); work items w < num_items = num_seqs * num_parts
// * (num_kv_heads / hpw) are (sequence, partition, head group), the head
// group varying fastest.  queue == nullptr: workgroup b runs item b (grid =
// num_items).  Otherwise the grid is at most what the GPU holds at once (grid
// <= num_items): workgroup b starts with item b, then takes item gridDim.x +
// atomicAdd(queue, 1), fetched while the current one streams, until they run
// out; *queue must be 0 at launch.  order: nullptr, or the sequence each
// item's sequence index stands for (a permutation), so that the grid can run
// the longest sequences first.  The hardware dispatcher hands workgroups
// to the XCDs in turn, in grid order, so with items of unequal length the
// slots of an XCD whose turn has not come stay empty; workgroups that fetch
// their next item keep every slot busy, and one counter keeps the items in
// order, so the head groups of a block are read at about the same time.
// (A counter serves an atomic about every 40 ns: one per wave and item would
// be too many, and one counter per XCD let the XCDs drift apart.)
template <class E, class KV, int D, int G, bool NT>
__global__ void __launch_bounds__(64 * kValuMaxHeadsPerWg)
__attribute__((amdgpu_waves_per_eu(ValuOccupancy<E, KV, D, G>::kWaves, 8)))
pa_decode_valu_kernel(void* __restrict__ out, const void* __restrict__ query,
                      const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                      const int* __restrict__ block_tables, const int* __restrict__ seq_lens,
                      int num_heads, int num_kv_heads, int max_blocks, int num_blocks,
                      float qk_scale, float v_scale, int part_tokens, int num_parts, float* __restrict__ ws,
                      int num_items, int* __restrict__ queue, const int* __restrict__ order) {
  using C = ValuCfg<E, KV, D, G>;
  constexpr int BS = kBlockSize;
  constexpr int LPR = C::kLpr, RPI = C::kRpi, NI = C::kNi, EPL = C::kEpl;
  constexpr int NV = C::kNv, NVL = C::kNvl, NH = C::kNh;
  constexpr int REC = rec_floats<D>();

  __shared__ __align__(16) float s_p_all[kValuMaxHeadsPerWg][RPI][C::kPStride];
  __shared__ float s_m_all[kValuMaxHeadsPerWg][RPI][G];
  __shared__ float s_l_all[kValuMaxHeadsPerWg][RPI][G];
  __shared__ int s_tk[2];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hpw = blockDim.x >> 6, groups = num_kv_heads / hpw;
  const int r = lane / LPR, c = lane % LPR;
  auto& s_p = s_p_all[wv];
  auto& s_m = s_m_all[wv];
  auto& s_l = s_l_all[wv];

  // tk: lane 0's ticket of the next item (queue mode), read into a uniform
  // value before the item's stores: a wait for it after them would also wait
  // for the stores (the vector memory counter counts both).
  const bool queued = queue != nullptr;
  auto run_item = [&](int w, int& tk) {
    auto take_ticket = [&]() {
      if (queued) {
        asm volatile("" : "+v"(tk) :: "memory");
        tk = __builtin_amdgcn_readfirstlane(tk);
      }
    };
    // Work item; the head group varies fastest.
    const int kvh = (w % groups) * hpw + wv;
    w /= groups;
    const int part = w % num_parts;
    const int s = order != nullptr ? order[w / num_parts] : w / num_parts;
    const int hq0 = kvh * G;                                      // first query head of the group

    u32x4 qv[G][C::kQw];                                          // query elements c*EPL .. c*EPL+EPL-1
    {
      const char* qb = static_cast<const char*>(query) + ((int64_t)s * num_heads + hq0) * C::kQRow +
                       c * EPL * E::kBytes;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int w = 0; w < C::kQw; ++w) qv[h][w] = *reinterpret_cast<const u32x4*>(qb + h * C::kQRow + 16 * w);
    }

    const int L = seq_lens[s];
    const bool split = part_tokens > 0;
    // tokens this launch can cover: the table row, and in split mode the grid's partitions
    const int64_t cap = split ? min((int64_t)max_blocks * BS, (int64_t)num_parts * part_tokens)
                              : (int64_t)max_blocks * BS;
    const bool bad_len = L < 0 || (int64_t)L > cap;
    const int nparts_seq = bad_len ? 1 : (split ? ceil_div(L, part_tokens) : 1);
    if (part >= (nparts_seq > 0 ? nparts_seq : 1)) {           // empty partition (next item)
      take_ticket();
      return;
    }
    const bool final_write = !split || nparts_seq <= 1;          // this item writes `out`

    const int t_begin = split ? part * part_tokens : 0;
    const int t_end = bad_len ? 0 : (split ? min(L, t_begin + part_tokens) : L);
    const int b_begin = t_begin / BS;
    const int b_end = ceil_div(t_end, BS);

    const int blk_bytes = BS * num_kv_heads * C::kRow;
    const int row_stride = num_kv_heads * C::kRow;                // bytes between token rows
    const int lane_off = (r * num_kv_heads + kvh) * C::kRow + c * 16;

    float m_run[NVL], l_run[NVL];
    float acc[G][EPL];
#pragma unroll
    for (int k = 0; k < NVL; ++k) { m_run[k] = -INFINITY; l_run[k] = 0.f; }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    const int idx0 = (c >> (ilog2(LPR) - NH)) * NVL;             // first score index this lane owns
    float* pbuf = &s_p[r][0];

    auto load_block = [&](int phys, u32x4* kb, u32x4* vb) {
      const __amdgpu_buffer_rsrc_t rk = block_rsrc(k_cache + (int64_t)phys * blk_bytes, blk_bytes);
      const __amdgpu_buffer_rsrc_t rv = block_rsrc(v_cache + (int64_t)phys * blk_bytes, blk_bytes);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kb[i] = load16<NT>(rk, lane_off, i * RPI * row_stride);
        vb[i] = load16<NT>(rv, lane_off, i * RPI * row_stride);
      }
    };

    auto consume = [&](const u32x4* kb, const u32x4* vb, int valid, bool masked) {
      float sc[NV];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[i * G + h] = dot_chunk<E, KV>(qv[h], kb[i]);
      transpose_reduce<LPR, NV, ilog2(LPR) - 1>(sc, c);

      float p[NVL], alpha[NVL];
#pragma unroll
      for (int k = 0; k < NVL; ++k) {
        const int i = (idx0 + k) / G;
        float z = sc[k] * qk_scale;
        if (masked && i * RPI + r >= valid) z = -INFINITY;
        const float bm = igroup_max<LPR>(z);
        const float m_new = fmaxf(m_run[k], bm);
        // a sub-wave may not have seen a valid token yet: keep exp2 away from -inf - -inf
        const float m_use = (masked && m_new == -INFINITY) ? 0.f : m_new;
        alpha[k] = __builtin_amdgcn_exp2f(m_run[k] - m_use);
        p[k] = __builtin_amdgcn_exp2f(z - m_use);
        l_run[k] = fmaf(l_run[k], alpha[k], p[k]);
        m_run[k] = m_new;
      }
#pragma unroll
      for (int k = 0; k < NVL; ++k) {
        pbuf[idx0 + k] = p[k];
        if (idx0 + k < G) pbuf[NV + idx0 + k] = alpha[k];
      }
      wave_lds_sync();
      float pall[C::kPStride];
#pragma unroll
      for (int j = 0; j < C::kPStride; j += 4) {
        const float4 t = *reinterpret_cast<const float4*>(pbuf + j);
        pall[j] = t.x; pall[j + 1] = t.y; pall[j + 2] = t.z; pall[j + 3] = t.w;
      }
      wave_lds_sync();

#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= pall[NV + h];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        u32x4 v = vb[i];
        if (masked && i * RPI + r >= valid) v = u32x4{0u, 0u, 0u, 0u};
        float vf[EPL];
        widen_chunk<E, KV>(v, vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = pall[i * G + h];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
        }
      }
    };

    const int* bt = block_tables + (int64_t)s * max_blocks;
    bool bad = bad_len;
    for (int cb = b_begin; cb < b_end; cb += 64) {
      // a wave with another batch of blocks after this one gets the SIMD's
      // issue slots first (13B-shaped batch, longest first: 234.1 -> 231.0
      // us; the waves that start second on a SIMD otherwise lag behind)
      if (b_end - cb > 64) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      const int n = min(64, b_end - cb);
      const int id = lane < n ? bt[cb + lane] : 0;
      if (__ballot(lane < n && (unsigned)id >= (unsigned)num_blocks)) { bad = true; break; }
      // valid rows of the batch's last block (only the sequence's last block is partial)
      const int v_last = cb + 64 >= b_end ? t_end - (b_end - 1) * BS : BS;
      auto blk = [&](int j) { return __builtin_amdgcn_readlane(id, j); };
      auto consume_last = [&](const u32x4* kb, const u32x4* vb) {
        if (v_last >= BS) consume(kb, vb, BS, false);
        else consume(kb, vb, v_last, true);
      };
      // three register sets: two blocks in flight while one is consumed
      u32x4 ka[NI], va[NI], kb2[NI], vb2[NI], kc[NI], vc[NI];
      load_block(blk(0), ka, va);
      if (n > 1) load_block(blk(1), kb2, vb2);
      int j = 0;
      for (; j + 4 < n; j += 3) {                                 // blocks j..j+2 full; j+3, j+4 exist
        load_block(blk(j + 2), kc, vc);
        consume(ka, va, BS, false);
        load_block(blk(j + 3), ka, va);
        consume(kb2, vb2, BS, false);
        load_block(blk(j + 4), kb2, vb2);
        consume(kc, vc, BS, false);
      }
      // 1..4 blocks left: j in ka/va, j + 1 (if any) in kb2/vb2
      const int rem = n - j;
      if (rem == 1) {
        consume_last(ka, va);
      } else if (rem == 2) {
        consume(ka, va, BS, false);
        consume_last(kb2, vb2);
      } else {
        load_block(blk(j + 2), kc, vc);
        consume(ka, va, BS, false);
        if (rem == 4) load_block(blk(j + 3), ka, va);
        consume(kb2, vb2, BS, false);
        if (rem == 3) {
          consume_last(kc, vc);
        } else {
          consume(kc, vc, BS, false);
          consume_last(ka, va);
        }
      }
    }

    // ---- merge the sub-waves (token rows r) with log-sum-exp weights
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
      l_run[k] = igroup_sum<LPR>(l_run[k]);
      if (idx0 + k < G) {
        s_m[r][idx0 + k] = m_run[k];
        s_l[r][idx0 + k] = l_run[k];
      }
    }
    wave_lds_sync();
    float Mh[G], Lh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float M = -INFINITY;
#pragma unroll
      for (int r2 = 0; r2 < RPI; ++r2) M = fmaxf(M, s_m[r2][h]);
      const float Ms = M == -INFINITY ? 0.f : M;
      float Ls = 0.f;
#pragma unroll
      for (int r2 = 0; r2 < RPI; ++r2) Ls += s_l[r2][h] * __builtin_amdgcn_exp2f(s_m[r2][h] - Ms);
      const float f = __builtin_amdgcn_exp2f(s_m[r][h] - Ms);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[h][e] * f;
#pragma unroll
        for (int m = LPR; m < 64; m <<= 1) a += __shfl_xor(a, m);
        acc[h][e] = a;
      }
      Mh[h] = M;
      Lh[h] = Ls;
    }
    take_ticket();
    if (r != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = Lh[h] > 0.f ? v_scale / Lh[h] : 0.f;
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = bad ? qnan() : acc[h][e] * inv;
      const int64_t sh = (int64_t)s * num_heads + hq0 + h;
      if (final_write) {
        store_run<E, EPL>(out, sh * D + c * EPL, o);
      } else {
        float* rec = ws + (sh * num_parts + part) * REC;
        store_f32_run<EPL>(rec + kRecHead + c * EPL, o);
        if (c == 0) {
          rec[0] = bad ? qnan() : Mh[h];
          rec[1] = bad ? qnan() : Lh[h];
        }
      }
    }
  };

  if (!queued) {
    int unused = 0;
    run_item(blockIdx.x, unused);
    return;
  }
  // The offset is 0 but not known to the compiler to be uniform: on a
  // uniform address its atomic optimizer would read the result back at once,
  // and the wave would wait for the atomic there.
  int* const counter = queue + (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);
  for (int w = blockIdx.x, it = 0;; ++it) {
    int t = 0;
    if (threadIdx.x == 0) t = atomicAdd(counter, 1);        // the next item, fetched while this one streams
    run_item(w, t);
    if (threadIdx.x == 0) s_tk[it & 1] = t;
    __syncthreads();
    w = (int)gridDim.x + s_tk[it & 1];
    if (w >= num_items) break;
  }
}

}  // namespace pa
