// Log-sum-exp merge of partial records into the output.
#pragma once

#include "common.h"
#include "decode_mfma.h"

namespace pa {

// Merge n records (stride in floats) of one (sequence, head) into one output
// row: M = max_p m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p.
// A NaN record makes the row NaN.  One wave; lane l owns elements PER*l ..
template <int D, class RecAt>
__device__ inline void lse_merge(RecAt rec_at, int n, float* res) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  float M = -INFINITY;
  bool nan = false;
  for (int p = 0; p < n; ++p) {
    const float m = rec_at(p)[0];
    nan = nan || (m != m);
    M = fmaxf(M, m);
  }
  float wsum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = 0.f;
  for (int p = 0; p < n; ++p) {
    const float* r = rec_at(p);
    const float wp = r[1] * __builtin_amdgcn_exp2f(r[0] - M);
    wsum += wp;
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = fmaf(wp, r[kRecHead + lane * PER + e], res[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = nan ? qnan() : res[e] / wsum;
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
  lse_merge<D>([&](int p) { return base + (int64_t)p * REC; }, np, res);
  write_row<E, D>(out, sh, res);
}

// Balanced split: one wave per (sequence, query head).  Writes the rows the
// decode kernel could not: sequences that crossed a range boundary (merged
// from the records of every workgroup they touched), empty sequences (zero)
// and out-of-contract lengths (NaN).
template <class E, int D>
__global__ void __launch_bounds__(64)
pa_sk_merge_kernel(void* __restrict__ out, const int* __restrict__ seq_lens, const int* __restrict__ ws_cum,
                   const float* __restrict__ ws_rec, int num_seqs, int num_heads, int group, int hpw, int nwg,
                   int max_blocks) {
  constexpr int REC = rec_floats<D>();
  constexpr int PER = D / 64;
  const int sh = blockIdx.x;
  const int s = sh / num_heads, hq = sh - s * num_heads;
  const int L = seq_lens[s];
  float res[PER];
  if (L < 0 || (int64_t)L > (int64_t)max_blocks * kBlockSize) {
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = qnan();
    write_row<E, D>(out, sh, res);
    return;
  }
  const int c0 = ws_cum[s], c1 = ws_cum[s + 1], U = ws_cum[num_seqs];
  if (c0 == c1) {
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = 0.f;
    write_row<E, D>(out, sh, res);
    return;
  }
  const int w1 = sk_owner(c0, U, nwg), w2 = sk_owner(c1 - 1, U, nwg);
  if (w1 == w2) return;                                  // written whole by the decode kernel
  const int kvh = hq / group, hl = hq - kvh * group;
  const int hg = kvh / hpw, wv = kvh - hg * hpw;
  // One record per workgroup the sequence touched (in range order); the first
  // workgroup's record is its second slot when its range began in an earlier
  // sequence.  Workgroups with an empty range (more workgroups than blocks)
  // hold none: their weight is zero.
  const int first_begin = sk_range_begin(w1, U, nwg);
  auto rec_of = [&](int w) {
    const int slot = (w == w1 && first_begin < c0) ? 1 : 0;
    return ws_rec + (int64_t)((((hg * nwg + w) * 2 + slot) * hpw + wv) * group + hl) * REC;
  };
  const int lane = threadIdx.x & 63;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  bool nan = false;
  // up to 64 records per pass: lane j reads record w1 + base + j's max and sum
  float M = -INFINITY;
  for (int base = w1; base <= w2; base += 64) {
    const int w = base + lane;
    const bool live = w <= w2 && sk_range_begin(w, U, nwg) != sk_range_begin(w + 1, U, nwg);
    const float m = live ? rec_of(w)[0] : -INFINITY;
    nan = nan || __ballot(m != m);
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  for (int base = w1; base <= w2; base += 64) {
    const int w = base + lane;
    const bool live = w <= w2 && sk_range_begin(w, U, nwg) != sk_range_begin(w + 1, U, nwg);
    const float* r = rec_of(live ? w : w1);
    const float wl = live ? r[1] * __builtin_amdgcn_exp2f(r[0] - M) : 0.f;   // weight of record `w`
    wsum += wl;
    const int n = min(64, w2 - base + 1);
    int j = 0;
    for (; j + 4 <= n; j += 4) {                        // four records' loads in flight
      float o[4][PER], wj[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wj[k] = __shfl(wl, j + k);
        const float* rk = rec_of(base + j + k);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[k][e] = wj[k] != 0.f ? rk[kRecHead + lane * PER + e] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj[k], o[k][e], acc[e]);
    }
    for (; j < n; ++j) {
      const float wj = __shfl(wl, j);
      const float* rk = rec_of(base + j);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, wj != 0.f ? rk[kRecHead + lane * PER + e] : 0.f, acc[e]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = nan ? qnan() : acc[e] / wsum;
  write_row<E, D>(out, sh, res);
}

}  // namespace pa
