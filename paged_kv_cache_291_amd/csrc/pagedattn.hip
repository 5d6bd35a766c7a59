// Paged decode attention and KV-cache scatter for MI355X (gfx950, CDNA4).
//
// What is computed follows the devpress.csdn.net article on the vLLM
// architecture, section 3 ("PagedAttention kernel: from concept to CUDA"):
// part 1 fixes the inputs (query, block tables, one K and one V pool of
// [blocks, block_size, kv_heads, head_size]); part 2 fixes the flow (take the
// sequence's table and length, gather K/V from the physical blocks it names,
// run standard attention, write the output).  The kernel design below is our
// own and is written for 64-lane wavefronts and HBM3E, not taken from the
// CUDA kernel the article describes.
//
// Decode kernel, one workgroup per (sequence, kv head, partition), 4 waves:
//  * Gather loader: each wave owns every 4th block of the range.  One row of
//    one head (head_size * elem bytes) is read by LPR lanes with 16-byte
//    loads, so one load instruction covers 64/LPR token rows; a block is
//    NI = 16 / (64/LPR) instructions per cache.  The next block's K and V
//    are in flight while the current one is consumed.
//  * Scores: q stays in registers; each lane forms partial dots of its
//    16-byte slice with v_dot2 (bf16/f16) or FMA (f32) for all G query heads
//    of the group, so each K byte is read once per KV head.  A halving
//    butterfly over the LPR lanes (DPP row/half mirror and quad permutes)
//    leaves every score on one lane.
//  * Online softmax (base 2, scale * log2(e) applied to the score) per
//    "sub-wave" (the LPR lanes that share token rows): block max over the
//    sub-wave's tokens with DPP rotates, running max/sum, rescale factor.
//    Probabilities and rescale factors go through a small per-wave LDS
//    buffer so every lane can weight its V slice.
//  * PV in fp32 registers; at the end the sub-waves and waves are merged with
//    log-sum-exp weights through LDS.
//  * Masking uses selects only (the pool may hold NaN in dead slots).
// With a partition size the workgroup writes fp32 partials (max in log2 units,
// sum, normalised output) and a reduce kernel merges them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kIdChunk = 512;   // block ids staged in LDS per round

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
constexpr int round_up4(int x) { return (x + 3) & ~3; }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct ElemF32 { static constexpr int kBytes = 4; };
struct ElemF16 { static constexpr int kBytes = 2; };
struct ElemBF16 { static constexpr int kBytes = 2; };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ element helpers

// acc + <q slice, k slice> over one 16-byte chunk.
template <class E>
__device__ inline float dot16(const uint4& q, const uint4& k, float acc);

template <>
__device__ inline float dot16<ElemBF16>(const uint4& q, const uint4& k, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x), __builtin_bit_cast(bf16x2_t, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y), __builtin_bit_cast(bf16x2_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z), __builtin_bit_cast(bf16x2_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w), __builtin_bit_cast(bf16x2_t, k.w), acc, false);
  return acc;
}

template <>
__device__ inline float dot16<ElemF16>(const uint4& q, const uint4& k, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.x), __builtin_bit_cast(f16x2_t, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.y), __builtin_bit_cast(f16x2_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.z), __builtin_bit_cast(f16x2_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q.w), __builtin_bit_cast(f16x2_t, k.w), acc, false);
  return acc;
}

template <>
__device__ inline float dot16<ElemF32>(const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Widen one 16-byte chunk to fp32 (exact for all three types).
template <class E>
__device__ inline void widen16(const uint4& v, float* f);

template <>
__device__ inline void widen16<ElemBF16>(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

template <>
__device__ inline void widen16<ElemF16>(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, w[j]);
    f[2 * j] = (float)h.x;
    f[2 * j + 1] = (float)h.y;
  }
}

template <>
__device__ inline void widen16<ElemF32>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

// Round fp32 to the storage type (round to nearest even) and store.
template <class E>
__device__ inline void store_elem(void* base, int64_t i, float x);

template <>
__device__ inline void store_elem<ElemF32>(void* base, int64_t i, float x) {
  static_cast<float*>(base)[i] = x;
}

template <>
__device__ inline void store_elem<ElemF16>(void* base, int64_t i, float x) {
  static_cast<_Float16*>(base)[i] = (_Float16)x;
}

template <>
__device__ inline void store_elem<ElemBF16>(void* base, int64_t i, float x) {
  uint32_t u = __float_as_uint(x);
  uint16_t b;
  if ((u & 0x7fffffffu) > 0x7f800000u) {
    b = (uint16_t)((u >> 16) | 0x0040u);            // quiet NaN, sign kept
  } else {
    u += 0x7fffu + ((u >> 16) & 1u);                 // round to nearest, ties to even
    b = (uint16_t)(u >> 16);
  }
  static_cast<uint16_t*>(base)[i] = b;
}

// ------------------------------------------------------------ lane exchange

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Value of the butterfly partner for lane bit MASK.  Within a 16-lane row the
// partners are row mirror (bit 3), half-row mirror (bit 2) and quad permutes
// (bits 1, 0); each flips the bit being reduced and keeps the higher bits,
// which is all the halving butterfly needs.  Bits 4 and 5 cross rows.
template <int MASK>
__device__ inline float xchg(float v) {
  if constexpr (MASK == 8) return dpp<0x140>(v);
  else if constexpr (MASK == 4) return dpp<0x141>(v);
  else if constexpr (MASK == 2) return dpp<0x4e>(v);
  else if constexpr (MASK == 1) return dpp<0xb1>(v);
  else return __shfl_xor(v, MASK);
}

// Max / sum over the lanes of a sub-wave that hold the same head and
// different token rows: lane bits 2 .. log2(LPR)-1.
template <int LPR>
__device__ inline float igroup_max(float v) {
  if constexpr (LPR == 16) {
    v = fmaxf(v, dpp<0x124>(v));    // row rotate by 4
    v = fmaxf(v, dpp<0x128>(v));    // row rotate by 8
  } else {
#pragma unroll
    for (int m = 4; m < LPR; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  }
  return v;
}

template <int LPR>
__device__ inline float igroup_sum(float v) {
  if constexpr (LPR == 16) {
    v += dpp<0x124>(v);
    v += dpp<0x128>(v);
  } else {
#pragma unroll
    for (int m = 4; m < LPR; m <<= 1) v += __shfl_xor(v, m);
  }
  return v;
}

// Halving butterfly: on entry every lane of an LPR-lane group holds NV
// partial sums; on exit lane c holds the full sums of NVL consecutive
// indices starting at idx0(c).
template <int LPR, int NV, int BIT>
__device__ inline void transpose_reduce(float* v, int c) {
  if constexpr (BIT >= 0) {
    constexpr int MASK = 1 << BIT;
    constexpr int N = NV >> (ilog2(LPR) - 1 - BIT);   // values still held
    const bool hi = (c & MASK) != 0;
    if constexpr (N > 1) {
      constexpr int H = N / 2;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const float send = hi ? v[j] : v[j + H];
        const float keep = hi ? v[j + H] : v[j];
        v[j] = keep + xchg<MASK>(send);
      }
    } else {
      v[0] += xchg<MASK>(v[0]);
    }
    transpose_reduce<LPR, NV, BIT - 1>(v, c);
  }
}

template <class E, int D, int BS, int G>
struct Cfg {
  static constexpr int kRow = D * E::kBytes;        // bytes of one token row of one head
  static constexpr int kLpr = kRow / 16;            // lanes per row
  static constexpr int kRpi = 64 / kLpr;            // rows per load instruction
  static constexpr int kNi = BS / kRpi;             // load instructions per block
  static constexpr int kEpl = 16 / E::kBytes;       // elements per lane per instruction
  static constexpr int kNv = kNi * G;               // partial scores per lane per block
  static constexpr int kNvl = kNv > kLpr ? kNv / kLpr : 1;
  static constexpr int kNh = ilog2(kNv < kLpr ? kNv : kLpr);
  static constexpr int kPStride = round_up4(kNv + G);
  static_assert(kLpr >= 4 && kLpr <= 32, "row must span 4..32 lanes");
  static_assert(BS % kRpi == 0 && kNi == kLpr / 4, "block must be whole load instructions");
  static_assert(D % 64 == 0, "head_size must be a multiple of 64");
};

// ------------------------------------------------------------ decode kernel

template <class E, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads)
pa_decode_kernel(void* __restrict__ out, const void* __restrict__ query,
                 const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                 const int* __restrict__ block_tables, const int* __restrict__ seq_lens,
                 int num_heads, int num_kv_heads, int max_blocks, int num_blocks,
                 float qk_scale, int part_tokens, int num_parts,
                 float* __restrict__ ws_ml, float* __restrict__ ws_o) {
  using C = Cfg<E, D, BS, G>;
  constexpr int LPR = C::kLpr, RPI = C::kRpi, NI = C::kNi, EPL = C::kEpl;
  constexpr int NV = C::kNv, NVL = C::kNvl, NH = C::kNh;

  __shared__ int s_ids[kIdChunk];
  __shared__ int s_bad;
  __shared__ __align__(16) float s_p[kWaves][RPI][C::kPStride];
  __shared__ float s_m[kWaves][RPI][G];
  __shared__ float s_l[kWaves][RPI][G];
  __shared__ __align__(16) float s_o[kWaves][G][D];
  __shared__ float s_fin[2][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;

  // Work item.  The kv head varies fastest, so the 8 XCDs (dispatched round
  // robin) each see a fixed subset of kv heads and shared blocks stay in one L2.
  int w = blockIdx.x;
  const int kvh = w % num_kv_heads;
  w /= num_kv_heads;
  const int part = w % num_parts;
  const int s = w / num_parts;

  const int L = seq_lens[s];
  const bool split = part_tokens > 0;
  // tokens this launch can cover: the table row, and in split mode the grid's partitions
  const int64_t cap = split ? min((int64_t)max_blocks * BS, (int64_t)num_parts * part_tokens)
                            : (int64_t)max_blocks * BS;
  const bool bad_len = L < 0 || (int64_t)L > cap;
  const int nparts_seq = bad_len ? 1 : (split ? ceil_div(L, part_tokens) : 1);
  if (part >= (nparts_seq > 0 ? nparts_seq : 1)) return;      // empty partition
  const bool final_write = !split || nparts_seq <= 1;          // this WG writes `out`

  const int t_begin = split ? part * part_tokens : 0;
  const int t_end = bad_len ? 0 : (split ? min(L, t_begin + part_tokens) : L);
  const int b_begin = t_begin / BS;
  const int b_end = ceil_div(t_end, BS);

  const int hq0 = kvh * G;                                      // first query head of the group
  const int64_t blk_bytes = (int64_t)BS * num_kv_heads * C::kRow;
  const int row_stride = num_kv_heads * C::kRow;                // bytes between token rows
  const int lane_off = (r * num_kv_heads + kvh) * C::kRow + c * 16;

  // Query slices of the G heads (same 16-byte chunk for every token row).
  uint4 qv[G];
  {
    const char* qb = static_cast<const char*>(query) + ((int64_t)s * num_heads + hq0) * C::kRow + c * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const uint4*>(qb + h * C::kRow);
  }

  float m_run[NVL], l_run[NVL];
  float acc[G][EPL];
#pragma unroll
  for (int k = 0; k < NVL; ++k) { m_run[k] = -INFINITY; l_run[k] = 0.f; }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

  const int idx0 = (c >> (ilog2(LPR) - NH)) * NVL;             // first score index this lane owns
  float* pbuf = &s_p[wave][r][0];

  if (tid == 0) s_bad = 0;

  auto load_block = [&](int phys, uint4* kb, uint4* vb) {
    const char* kp = k_cache + (int64_t)phys * blk_bytes + lane_off;
    const char* vp = v_cache + (int64_t)phys * blk_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      kb[i] = *reinterpret_cast<const uint4*>(kp + i * RPI * row_stride);
      vb[i] = *reinterpret_cast<const uint4*>(vp + i * RPI * row_stride);
    }
  };

  auto consume = [&](const uint4* kb, const uint4* vb, int valid, bool masked) {
    // partial dots of this lane's slice for every (token row i, head h)
    float sc[NV];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[i * G + h] = dot16<E>(qv[h], kb[i], 0.f);
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
    // publish probabilities and per-head rescale factors to the sub-wave
#pragma unroll
    for (int k = 0; k < NVL; ++k) {
      pbuf[idx0 + k] = p[k];
      if (idx0 + k < G) pbuf[NV + idx0 + k] = alpha[k];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float pall[C::kPStride];
#pragma unroll
    for (int j = 0; j < C::kPStride; j += 4) {
      const float4 t = *reinterpret_cast<const float4*>(pbuf + j);
      pall[j] = t.x; pall[j + 1] = t.y; pall[j + 2] = t.z; pall[j + 3] = t.w;
    }
    __builtin_amdgcn_wave_barrier();

#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= pall[NV + h];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint4 v = vb[i];
      if (masked && i * RPI + r >= valid) v = make_uint4(0u, 0u, 0u, 0u);
      float vf[EPL];
      widen16<E>(v, vf);
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
  for (int cb = b_begin; cb < b_end; cb += kIdChunk) {
    const int ce = min(b_end, cb + kIdChunk);
    __syncthreads();                                 // previous chunk consumed
    for (int j = cb + tid; j < ce; j += kThreads) {
      int id = bt[j];
      if ((unsigned)id >= (unsigned)num_blocks) { s_bad = 1; id = 0; }
      s_ids[j - cb] = id;
    }
    __syncthreads();
    if (s_bad) { bad = true; break; }

    int j = cb + wave;
    if (j < ce) {
      uint4 kb[NI], vb[NI];
      load_block(s_ids[j - cb], kb, vb);
      while (true) {
        const int jn = j + kWaves;
        const bool more = jn < ce;
        uint4 kn[NI], vn[NI];
        if (more) load_block(s_ids[jn - cb], kn, vn);
        const int valid = t_end - j * BS;
        if (valid >= BS) consume(kb, vb, BS, false);
        else consume(kb, vb, valid, true);
        if (!more) break;
#pragma unroll
        for (int i = 0; i < NI; ++i) { kb[i] = kn[i]; vb[i] = vn[i]; }
        j = jn;
      }
    }
  }

  // ---- merge sub-waves and waves with log-sum-exp weights
  __syncthreads();
  bad = bad || (s_bad != 0);
#pragma unroll
  for (int k = 0; k < NVL; ++k) {
    l_run[k] = igroup_sum<LPR>(l_run[k]);
    if (idx0 + k < G) {
      s_m[wave][r][idx0 + k] = m_run[k];
      s_l[wave][r][idx0 + k] = l_run[k];
    }
  }
  __syncthreads();
  float f_own[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2)
#pragma unroll
      for (int r2 = 0; r2 < RPI; ++r2) M = fmaxf(M, s_m[w2][r2][h]);
    const float Ms = M == -INFINITY ? 0.f : M;
    f_own[h] = __builtin_amdgcn_exp2f(s_m[wave][r][h] - Ms);
    if (tid == h) {
      float Ls = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2)
#pragma unroll
        for (int r2 = 0; r2 < RPI; ++r2) Ls += s_l[w2][r2][h] * __builtin_amdgcn_exp2f(s_m[w2][r2][h] - Ms);
      s_fin[0][h] = M;
      s_fin[1][h] = Ls;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float a = acc[h][e] * f_own[h];
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) a += __shfl_xor(a, m);
      acc[h][e] = a;
    }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(&s_o[wave][h][c * EPL + e]) =
            make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
  }
  __syncthreads();

  for (int o = tid; o < G * D; o += kThreads) {
    const int h = o / D, d = o % D;
    float sum = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) sum += s_o[w2][h][d];
    const float Ls = s_fin[1][h];
    float val = Ls > 0.f ? sum / Ls : 0.f;
    if (bad) val = __int_as_float(0x7fc00000);
    const int64_t sh = (int64_t)s * num_heads + hq0 + h;
    if (final_write) {
      store_elem<E>(out, sh * D + d, val);
    } else {
      ws_o[(sh * num_parts + part) * D + d] = val;
      if (d == 0) {
        ws_ml[(sh * num_parts + part) * 2] = bad ? __int_as_float(0x7fc00000) : s_fin[0][h];
        ws_ml[(sh * num_parts + part) * 2 + 1] = bad ? __int_as_float(0x7fc00000) : Ls;
      }
    }
  }
}

// ------------------------------------------------------------ LSE reduce kernel

// One wave per (sequence, query head): merge the partitions of a split
// sequence.  M = max_p m_p, w_p = l_p * 2^(m_p - M), out = sum w_p o_p / sum w_p.
template <class E, int D>
__global__ void __launch_bounds__(64)
pa_reduce_kernel(void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
                 const int* __restrict__ seq_lens, int num_heads, int max_blocks, int block_size,
                 int part_tokens, int num_parts) {
  constexpr int PER = D / 64;
  const int sh = blockIdx.x;
  const int s = sh / num_heads;
  const int L = seq_lens[s];
  const int64_t cap = min((int64_t)max_blocks * block_size, (int64_t)num_parts * part_tokens);
  if (L < 0 || (int64_t)L > cap) return;             // NaN row written by the partition kernel
  const int np = ceil_div(L, part_tokens);
  if (np <= 1) return;                               // written by the partition kernel
  const float* ml = ws_ml + (int64_t)sh * num_parts * 2;
  const float* o = ws_o + (int64_t)sh * num_parts * D + threadIdx.x * PER;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  float wsum = 0.f, a[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) a[e] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float wp = ml[2 * p + 1] * __builtin_amdgcn_exp2f(ml[2 * p] - M);
    wsum += wp;
#pragma unroll
    for (int e = 0; e < PER; ++e) a[e] = fmaf(wp, o[(int64_t)p * D + e], a[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    store_elem<E>(out, (int64_t)sh * D + threadIdx.x * PER + e, a[e] / wsum);
}

// ------------------------------------------------------------ scatter kernel

__global__ void __launch_bounds__(256)
pa_cache_scatter_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                        uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                        const int* __restrict__ slot_mapping, int row_chunks, int64_t num_slots) {
  const int t = blockIdx.x;
  const int chunk = blockIdx.y * blockDim.x + threadIdx.x;
  if (chunk >= row_chunks) return;
  const int slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t src = (int64_t)t * row_chunks + chunk;
  const int64_t dst = (int64_t)slot * row_chunks + chunk;
  k_cache[dst] = key[src];
  v_cache[dst] = value[src];
}

// ------------------------------------------------------------ host side

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : 2; }

size_t workspace_bytes_for(int num_seqs, int num_heads, int head_size, int num_parts) {
  const size_t rows = (size_t)num_seqs * num_heads * num_parts;
  const size_t ml = (rows * 2 * sizeof(float) + 255) & ~(size_t)255;
  return ml + rows * head_size * sizeof(float);
}

struct DecodeArgs {
  void* out; const void* query; const char* kc; const char* vc;
  const int* bt; const int* sl;
  int num_heads, num_kv_heads, max_blocks, num_blocks;
  float qk_scale; int part_tokens, num_parts;
  float* ws_ml; float* ws_o;
};

template <class E, int D, int G>
int launch_decode(const DecodeArgs& a, int num_seqs, hipStream_t stream) {
  const long long grid = (long long)num_seqs * a.num_parts * a.num_kv_heads;
  if (grid > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((pa_decode_kernel<E, D, 16, G>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     a.out, a.query, a.kc, a.vc, a.bt, a.sl, a.num_heads, a.num_kv_heads, a.max_blocks,
                     a.num_blocks, a.qk_scale, a.part_tokens, a.num_parts, a.ws_ml, a.ws_o);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (a.part_tokens > 0) {
    hipLaunchKernelGGL((pa_reduce_kernel<E, D>), dim3((unsigned)(num_seqs * a.num_heads)), dim3(64), 0, stream,
                       a.out, a.ws_ml, a.ws_o, a.sl, a.num_heads, a.max_blocks, 16, a.part_tokens, a.num_parts);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

template <class E, int D>
int dispatch_group(const DecodeArgs& a, int num_seqs, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch_decode<E, D, 1>(a, num_seqs, st);
    case 2: return launch_decode<E, D, 2>(a, num_seqs, st);
    case 4: return launch_decode<E, D, 4>(a, num_seqs, st);
    case 8: return launch_decode<E, D, 8>(a, num_seqs, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <class E>
int dispatch_head(const DecodeArgs& a, int num_seqs, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return dispatch_group<E, 64>(a, num_seqs, group, st);
    case 128: return dispatch_group<E, 128>(a, num_seqs, group, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_size,
                                           int max_seq_len, int partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_seq_len < 0) return 0;
  const int np = max_seq_len > 0 ? ceil_div(max_seq_len, partition_size) : 1;
  return workspace_bytes_for(num_seqs, num_heads, head_size, np);
}

extern "C" int paged_attention_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int dtype, int partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 ||
      max_blocks_per_seq < 0 || num_blocks < 0 || max_seq_len < 0 || partition_size < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  const int group = num_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % block_size != 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(query) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  if (max_blocks_per_seq == 0 && max_seq_len > 0) return PA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.out = out; a.query = query;
  a.kc = static_cast<const char*>(k_cache); a.vc = static_cast<const char*>(v_cache);
  a.bt = block_tables; a.sl = seq_lens;
  a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks;
  a.qk_scale = (float)((double)scale * 1.4426950408889634);
  a.part_tokens = 0; a.num_parts = 1;
  if (partition_size > 0) {
    const long long cap = (long long)max_blocks_per_seq * block_size;
    const int msl = max_seq_len > 0 ? max_seq_len : (int)(cap < 0x7fffffffLL ? cap : 0x7fffffffLL);
    const int np = msl > 0 ? ceil_div(msl, partition_size) : 1;
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_size, np);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_WORKSPACE;
    const size_t rows = (size_t)num_seqs * num_heads * np;
    a.part_tokens = partition_size; a.num_parts = np;
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((rows * 2 * sizeof(float) + 255) & ~(size_t)255));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PA_F32: return dispatch_head<ElemF32>(a, num_seqs, head_size, group, st);
    case PA_F16: return dispatch_head<ElemF16>(a, num_seqs, head_size, group, st);
    default: return dispatch_head<ElemBF16>(a, num_seqs, head_size, group, st);
  }
}

extern "C" int reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_size, int block_size, int num_blocks, int dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  const long long row_bytes = (long long)num_kv_heads * head_size * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_INVALID_ARG;
  const long long chunks = row_bytes / 16;
  if (chunks > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  const int threads = chunks >= 256 ? 256 : (int)((chunks + 63) / 64 * 64);
  const dim3 grid((unsigned)num_tokens, (unsigned)((chunks + threads - 1) / threads));
  hipLaunchKernelGGL(pa_cache_scatter_kernel, grid, dim3(threads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping,
                     (int)chunks, (int64_t)num_blocks * block_size);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}
