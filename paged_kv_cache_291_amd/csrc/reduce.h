// Log-sum-exp merge of partial records into the output.
#pragma once

#include "common.h"
#include "decode_mfma.h"

namespace pa {

// Merge the n records of one (sequence, head) into one output row (one wave;
// lane l owns elements PER*l ..):
//   M = max_j m_j,  w_j = l_j * 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j.
// rec_of(j) is record j; live(j) says whether record j exists (absent records
// weigh nothing).  A NaN in a record's max or sum makes the row NaN.  Lane j
// reads the max and sum of record base + j (64 per step); outputs are read NB
// records at a time, the first NB together with the maxima.
template <int D, class RecOf, class Live>
__device__ inline void lse_merge(RecOf rec_of, Live live, int n, float* res) {
  constexpr int PER = D / 64;
  constexpr int NB = 16;
  const int lane = threadIdx.x & 63;
  auto load_o = [&](uint64_t mask, int j, int k, float* o) {
    if ((mask >> k) & 1) {
      const float* r = rec_of(j + k) + kRecHead + lane * PER;
      if constexpr (PER == 2) {
        const float2 v = *reinterpret_cast<const float2*>(r);
        o[0] = v.x; o[1] = v.y;
      } else {
        o[0] = r[0];
      }
    } else {
#pragma unroll
      for (int x = 0; x < PER; ++x) o[x] = 0.f;
    }
  };
  // pass 1: maxima (the first step also loads the first NB records' outputs)
  const bool lv0 = lane < n && live(lane);
  const uint64_t mask0 = __ballot(lv0);
  float o[NB][PER];
#pragma unroll
  for (int k = 0; k < NB; ++k) load_o(mask0, 0, k, o[k]);
  const float* r0 = rec_of(lv0 ? lane : 0);
  const float m0 = lv0 ? r0[0] : -INFINITY, l0 = lv0 ? r0[1] : 0.f;
  bool nan = __ballot(m0 != m0 || l0 != l0) != 0;
  float M = m0;
  for (int base = 64; base < n; base += 64) {
    const bool lv = base + lane < n && live(base + lane);
    const float* r = rec_of(lv ? base + lane : 0);
    const float m = lv ? r[0] : -INFINITY, l = lv ? r[1] : 0.f;
    nan = nan || __ballot(m != m || l != l);
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  // pass 2: weighted sum
  float acc[PER], wsum = 0.f;
#pragma unroll
  for (int x = 0; x < PER; ++x) acc[x] = 0.f;
  for (int base = 0; base < n; base += 64) {
    bool lv = lv0;
    uint64_t mask = mask0;
    float m = m0, l = l0;
    if (base > 0) {
      lv = base + lane < n && live(base + lane);
      mask = __ballot(lv);
      const float* r = rec_of(lv ? base + lane : 0);
      m = lv ? r[0] : -INFINITY;
      l = lv ? r[1] : 0.f;
    }
    const float wl = lv ? l * __builtin_amdgcn_exp2f(m - M) : 0.f;   // weight of record base + lane
    wsum += wl;
    const int cnt = min(64, n - base);
    for (int j = 0; j < cnt; j += NB) {
      if (base > 0 || j > 0) {
#pragma unroll
        for (int k = 0; k < NB; ++k) load_o(mask >> j, base + j, k, o[k]);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wk = __shfl(wl, (j + k) & 63);
#pragma unroll
        for (int x = 0; x < PER; ++x) acc[x] = fmaf(j + k < cnt ? wk : 0.f, o[k][x], acc[x]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
  for (int x = 0; x < PER; ++x) res[x] = nan ? qnan() : acc[x] / wsum;
}

// The same merge for one row per 16-lane group (four rows per wave; lane
// c = l%16 owns elements PER*c .., PER = D/16).  Records are walked 16 at a
// time for the maxima; outputs are read NB records at a time, and records
// that are absent or weigh nothing are never read.
template <int D, class RecOf, class Live>
__device__ inline void lse_merge16(RecOf rec_of, Live live, int n, float* res) {
  constexpr int PER = D / 16;
  constexpr int NB = 4;
  const int lane = threadIdx.x & 63, c = lane & 15;
  float M = -INFINITY;
  int nan = 0;
  for (int base = 0; base < n; base += 16) {
    const bool lv = base + c < n && live(base + c);
    const float* rr = rec_of(lv ? base + c : 0);
    const float m = lv ? rr[0] : -INFINITY, l = lv ? rr[1] : 0.f;
    nan |= (m != m || l != l) ? 1 : 0;
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    M = fmaxf(M, __shfl_xor(M, off));
    nan |= __shfl_xor(nan, off);
  }
  float acc[PER], wsum = 0.f;
#pragma unroll
  for (int x = 0; x < PER; ++x) acc[x] = 0.f;
  for (int base = 0; base < n; base += 16) {
    const bool lv = base + c < n && live(base + c);
    const float* rr = rec_of(lv ? base + c : 0);
    const float wl = lv ? rr[1] * __builtin_amdgcn_exp2f(rr[0] - M) : 0.f;   // weight of record base + c
    wsum += wl;
    const int cnt = min(16, n - base);
    for (int j = 0; j < cnt; j += NB) {
      float o[NB][PER];
      float wk[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        wk[k] = __shfl(wl, (lane & 48) + ((j + k) & 15));
        const bool use = j + k < cnt && wk[k] != 0.f;
#pragma unroll
        for (int x = 0; x < PER; x += 4) {
          const float4 v = use ? *reinterpret_cast<const float4*>(rec_of(base + j + k) + kRecHead + PER * c + x)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
          o[k][x] = v.x; o[k][x + 1] = v.y; o[k][x + 2] = v.z; o[k][x + 3] = v.w;
        }
        if (!use) wk[k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < NB; ++k)
#pragma unroll
        for (int x = 0; x < PER; ++x) acc[x] = fmaf(wk[k], o[k][x], acc[x]);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
  for (int x = 0; x < PER; ++x) res[x] = nan ? qnan() : acc[x] / wsum;
}

template <class E, int D>
__device__ inline void write_row(void* out, int64_t sh, const float* res) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_elem<E>(out, sh * D + lane * PER + e, res[e]);
}

// Fixed partitions: one wave per (sequence, query head).  Rows of sequences
// with one partition (or none, or an out-of-contract length) were written by
// the decode kernel.
template <class E, int D>
__global__ void __launch_bounds__(64)
pa_reduce_kernel(void* __restrict__ out, const float* __restrict__ ws, const int* __restrict__ seq_lens,
                 int num_heads, int max_blocks, int part_tokens, int num_parts) {
  constexpr int REC = rec_floats<D>();
  const int sh = blockIdx.x;
  const int s = sh / num_heads;
  const int L = seq_lens[s];
  const int64_t cap = min((int64_t)max_blocks * kBlockSize, (int64_t)num_parts * part_tokens);
  if (L < 0 || (int64_t)L > cap) return;
  const int np = ceil_div(L, part_tokens);
  if (np <= 1) return;
  const float* base = ws + (int64_t)sh * num_parts * REC;
  float res[D / 64];
  lse_merge<D>([&](int p) { return base + (int64_t)p * REC; }, [](int) { return true; }, np, res);
  write_row<E, D>(out, sh, res);
}

// Merge of one balanced-split row: a whole wave per row (RPW = 1; lane l
// owns elements D/64*l ..) or a 16-lane group per row (RPW = 4; lane l owns
// D/16*(l%16) ..).  Four rows per wave need a quarter of the waves and read
// a row's records with 16 lanes; with few long sequences (many records per
// row) the whole-wave form, which reads 16 records at once, is faster.
template <int D, int RPW>
struct MergeRow {
  static constexpr int kPer = RPW == 4 ? D / 16 : D / 64;
  template <class RecOf, class Live>
  __device__ static void merge(RecOf rec_of, Live live, int n, float* res) {
    if constexpr (RPW == 4) lse_merge16<D>(rec_of, live, n, res);
    else lse_merge<D>(rec_of, live, n, res);
  }
  template <class E>
  __device__ static void store(void* out, int64_t row, const float* res) {
    if constexpr (RPW == 4) store_run<E, kPer>(out, row * D + kPer * (threadIdx.x & 15), res);
    else write_row<E, D>(out, row, res);
  }
};

// Balanced split: one wave per (sequence, RPW consecutive query heads) of the
// sequences that ran past the range holding their first block (ws_seq[s] =
// {w1, first block, end block, total blocks}; w1 = -1: the decode kernel
// wrote the rows).  Each range the sequence touched left one record per
// head: the first range's is its second slot when that range began in an
// earlier sequence; ranges left empty (more workgroups than blocks) hold none.
template <class E, int D, int G, int RPW>
__global__ void __launch_bounds__(64)
pa_sk_merge_kernel(void* __restrict__ out, const int4* __restrict__ ws_seq, const float* __restrict__ ws_rec,
                   int num_heads, int hpw, int nwg) {
  constexpr int REC = rec_floats<D>();
  using MR = MergeRow<D, RPW>;
  const int per_seq = (num_heads + RPW - 1) / RPW;
  const int64_t id = blockIdx.x;
  const int s = (int)(id / per_seq);
  const int hq = (int)(id - (int64_t)s * per_seq) * RPW + (RPW == 4 ? (int)(threadIdx.x & 63) >> 4 : 0);
  const int4 e = ws_seq[s];
  if (e.x < 0) return;
  const bool head_ok = hq < num_heads;
  const int w1 = e.x, c0 = e.y, c1 = e.z, U = e.w;
  const int n = sk_owner(c1 - 1, U, nwg) - w1 + 1;
  const int h = head_ok ? hq : 0;                      // heads past the last one merge head 0 and drop it
  const int kvh = h / G, hl = h - kvh * G;
  const int hg = kvh / hpw, wv = kvh - hg * hpw;
  const int first_slot = sk_range_begin(w1, U, nwg) < c0 ? 1 : 0;
  auto rec_of = [&](int j) {                           // record of the sequence's j-th range
    const int w = w1 + j, slot = j == 0 ? first_slot : 0;
    return ws_rec + (int64_t)((((hg * nwg + w) * 2 + slot) * hpw + wv) * G + hl) * REC;
  };
  float res[MR::kPer];
  MR::merge(rec_of, [&](int j) { return sk_range_begin(w1 + j, U, nwg) != sk_range_begin(w1 + j + 1, U, nwg); },
            n, res);
  if (head_ok) MR::template store<E>(out, (int64_t)s * num_heads + hq, res);
}

// Balanced split with several query tokens per sequence (rows = (token,
// head) pairs, rows_kv record rows per kv head of the decode kernel): one wave per
// (sequence, kv head, RPW consecutive record rows).  Rows past the
// sequence's query rows and sequences written whole by the decode kernel
// return at once.
template <class E, int D, int G, int RPW>
__global__ void __launch_bounds__(64)
pa_sk_merge_mq_kernel(void* __restrict__ out, const int4* __restrict__ ws_seq, const float* __restrict__ ws_rec,
                      const int* __restrict__ query_start, int num_heads, int hpw, int nwg, int max_q,
                      int rows_kv) {
  constexpr int REC = rec_floats<D>();
  using MR = MergeRow<D, RPW>;
  const int per_kv = (max_q * G + RPW - 1) / RPW, num_kv = num_heads / G;
  const int64_t id = blockIdx.x;
  const int rq = (int)(id % per_kv);
  const int64_t t = id / per_kv;
  const int kvh = (int)(t % num_kv), s = (int)(t / num_kv);
  const int r = RPW * rq + (RPW == 4 ? (int)(threadIdx.x & 63) >> 4 : 0);   // token r / G, head kvh*G + r%G
  const int i = r / G;
  const int a = query_start[s], nq = query_start[s + 1] - a;
  const int4 e = ws_seq[s];
  if (e.x < 0 || RPW * rq / G >= nq) return;          // uniform: the wave's first row is its lowest token
  const bool row_ok = i < nq;
  const int w1 = e.x, c0 = e.y, c1 = e.z, U = e.w;
  const int n = sk_owner(c1 - 1, U, nwg) - w1 + 1;
  const int hg = kvh / hpw, wv = kvh - hg * hpw;
  const int first_slot = sk_range_begin(w1, U, nwg) < c0 ? 1 : 0;
  auto rec_of = [&](int j) {
    const int w = w1 + j, slot = j == 0 ? first_slot : 0;
    return ws_rec + (int64_t)((((hg * nwg + w) * 2 + slot) * hpw + wv) * rows_kv + r) * REC;
  };
  float res[MR::kPer];
  MR::merge(rec_of, [&](int j) { return sk_range_begin(w1 + j, U, nwg) != sk_range_begin(w1 + j + 1, U, nwg); },
            n, res);
  if (row_ok) MR::template store<E>(out, (int64_t)(a + i) * num_heads + kvh * G + r % G, res);
}

}  // namespace pa
