// Device helpers shared by the paged decode kernels (gfx950, 64-lane waves).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per cache block (the only size built)

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
constexpr int round_up4(int x) { return (x + 3) & ~3; }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Partial result of one (sequence, query head, token range): fp32 record of
// head_size + 4 floats: [0] max of the base-2 scores, [1] sum of 2^(z - max),
// [2..3] unused, [4 ..] output normalised by that sum.
constexpr int kRecHead = 4;
template <int D> constexpr int rec_floats() { return D + kRecHead; }

struct ElemF32 { static constexpr int kBytes = 4; };
struct ElemF16 { static constexpr int kBytes = 2; };
struct ElemBF16 { static constexpr int kBytes = 2; };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

__device__ inline float qnan() { return __int_as_float(0x7fc00000); }

// Order LDS writes before later LDS reads of other lanes of the same wave.
// A wave's LDS operations execute in program order, so only the compiler has
// to be kept from moving them across this point.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint16_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------ element helpers

// acc + <q slice, k slice> over one 16-byte chunk.
// Elements are copied out of the vectors before __builtin_bit_cast: applied
// directly to a vector-subscript lvalue, the cast reads element 0.
// acc + q.lo*k.lo + q.hi*k.hi over two 16-bit elements per dword (fp32 sum).
template <class E>
__device__ inline float dot2(uint32_t q, uint32_t k, float acc) {
  if constexpr (std::is_same<E, ElemBF16>::value)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q), __builtin_bit_cast(bf16x2_t, k), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q), __builtin_bit_cast(f16x2_t, k), acc, false);
}

template <class E>
__device__ inline float dot16(const u32x4& q, const u32x4& k, float acc);

template <>
__device__ inline float dot16<ElemBF16>(const u32x4& q, const u32x4& k, float acc) {
  const uint32_t qw[4] = {q[0], q[1], q[2], q[3]};
  const uint32_t kw[4] = {k[0], k[1], k[2], k[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[j]), __builtin_bit_cast(bf16x2_t, kw[j]), acc, false);
  return acc;
}

template <>
__device__ inline float dot16<ElemF16>(const u32x4& q, const u32x4& k, float acc) {
  const uint32_t qw[4] = {q[0], q[1], q[2], q[3]};
  const uint32_t kw[4] = {k[0], k[1], k[2], k[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, qw[j]), __builtin_bit_cast(f16x2_t, kw[j]), acc, false);
  return acc;
}

template <>
__device__ inline float dot16<ElemF32>(const u32x4& q, const u32x4& k, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(q[j]), __uint_as_float(k[j]), acc);
  return acc;
}

// Widen one 16-byte chunk to fp32 (exact for all three types).
template <class E>
__device__ inline void widen16(const u32x4& v, float* f);

template <>
__device__ inline void widen16<ElemBF16>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

template <>
__device__ inline void widen16<ElemF16>(const u32x4& v, float* f) {
  const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, w[j]);
    f[2 * j] = (float)h.x;
    f[2 * j + 1] = (float)h.y;
  }
}

template <>
__device__ inline void widen16<ElemF32>(const u32x4& v, float* f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(v[j]);
}

// Round fp32 to the storage type (round to nearest even) and store one element.
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
  static_cast<uint16_t*>(base)[i] = bf16_bits(x);
}

// Two fp32 values rounded to the 16-bit type and packed (low = x).
template <class E>
__device__ inline uint32_t pack2(float x, float y);

template <>
__device__ inline uint32_t pack2<ElemBF16>(float x, float y) {
  const bf16x2_t v = {(__bf16)x, (__bf16)y};          // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint32_t, v);
}

template <>
__device__ inline uint32_t pack2<ElemF16>(float x, float y) {
  const f16x2_t v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(uint32_t, v);
}

// Store N consecutive outputs (N * elem bytes = 8 or 16 bytes) rounded to the type.
template <class E, int N>
__device__ inline void store_run(void* base, int64_t elem, const float* f) {
  if constexpr (E::kBytes == 4) {
    static_assert(N % 4 == 0, "fp32 runs are whole float4s");
#pragma unroll
    for (int e = 0; e < N; e += 4)
      *reinterpret_cast<float4*>(static_cast<float*>(base) + elem + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
  } else if constexpr (N % 8 == 0) {
#pragma unroll
    for (int e = 0; e < N; e += 8) {
      const u32x4 w = {pack2<E>(f[e], f[e + 1]), pack2<E>(f[e + 2], f[e + 3]), pack2<E>(f[e + 4], f[e + 5]),
                       pack2<E>(f[e + 6], f[e + 7])};
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + elem + e) = w;
    }
  } else {
    static_assert(N == 4, "16-bit runs are 4 or a multiple of 8 elements");
    const u32x2 w = {pack2<E>(f[0], f[1]), pack2<E>(f[2], f[3])};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + elem) = w;
  }
}

// Store N fp32 values (N a multiple of 4) to a partial record.
template <int N>
__device__ inline void store_f32_run(float* dst, const float* f) {
#pragma unroll
  for (int e = 0; e < N; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
}

// ------------------------------------------------------------ cache block loads

// Buffer descriptor over one physical block (base in SGPRs, range-checked by
// the hardware: offsets past `bytes` read zero).  Raw (untyped) dword access.
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, 0x00020000);
}

// 16- and 8-byte buffer loads.  NT sets the non-temporal cache policy (bit 1):
// blocks read once per step stream past the caches; blocks that several
// sequences share are loaded with the default policy so they stay cached.
template <bool NT>
__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0);
}

template <bool NT>
__device__ inline u32x2 load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, NT ? 2 : 0);
}

template <bool NT>
__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, NT ? 2 : 0);
}

// Formats of the K/V pools.  Kv16: elements of the query type (bf16 or
// fp16).  KvFp8: OCP fp8 e4m3 codes, dequantised in registers to the query
// type (exactly: every e4m3 value is a bf16 and an fp16 value); the pools'
// scales enter the score scale (K) and the final normalisation (V).
struct Kv16 { static constexpr int kBytes = 2; };   // (fp32 queries: fp32 pools)
struct KvFp8 { static constexpr int kBytes = 1; };

// Two OCP fp8 e4m3 values (bytes 0-1, or 2-3 when `hi`) of a dword as two
// 16-bit values of type E in one dword.  Every e4m3 value is exact in bf16
// and fp16, so this conversion is exact.
template <class E, bool HI>
__device__ inline uint32_t fp8x2_to(uint32_t w) {
  if constexpr (E::kBytes == 2 && std::is_same<E, ElemBF16>::value)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
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

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// gfx950 row swaps: each swap pairs every lane with its partner row, and
// combining both results leaves the two-row total in every lane.
__device__ inline float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max(a, b) for values that are never NaN (scores, -inf for masked keys) in
// one instruction: the median of (a, b, +inf).  Written with fmaxf, every
// input that the compiler cannot prove canonical (matrix-core results, lane
// swaps) is first quieted by an extra instruction.  The +inf is hidden from
// the compiler (an SGPR it cannot see through), which would otherwise turn the
// median back into fmaxf.
__device__ inline float opaque_inf() {
  float v = INFINITY;
  asm volatile("" : "+s"(v));
  return v;
}

__device__ inline float max_nonan(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }

// rows_max for values that are never NaN.
__device__ inline float rows_max_nonan(float v, float inf) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_nonan(__uint_as_float(a[0]), __uint_as_float(a[1]), inf);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nonan(__uint_as_float(b[0]), __uint_as_float(b[1]), inf);
}

__device__ inline float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------------------------ matrix cores

// Matrix-core steps for one 16-bit element type.  Operand layouts (lane l):
//   16x16x32: A[m = l%16][k = 8*(l/16) + j], B[k = 8*(l/16) + j][n = l%16], j < 8
//   16x16x16: A[m = l%16][k = 4*(l/16) + j], B[k = 4*(l/16) + j][n = l%16], j < 4
//   C (both): C[m = 4*(l/16) + i][n = l%16], i < 4
template <class E>
struct Mfma;

template <>
struct Mfma<ElemBF16> {
  static constexpr uint32_t kOnes = 0x3F803F80u;   // two 1.0 elements
  __device__ static f32x4 qk(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(const u32x2& a, const u32x2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<ElemF16> {
  static constexpr uint32_t kOnes = 0x3C003C00u;
  __device__ static f32x4 qk(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(const u32x2& a, const u32x2& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};

}  // namespace pa
