// Paged decode attention and KV-cache scatter for MI355X (gfx950, CDNA4):
// the C ABI of include/pagedattn.h, its argument checks and launches.
//
// What is computed follows the devpress.csdn.net article on the vLLM
// architecture, section 3 ("PagedAttention kernel: from concept to CUDA"):
// part 1 fixes the inputs (query, block tables, one K and one V pool of
// [blocks, block_size, kv_heads, head_size]); part 2 fixes the flow (take the
// sequence's table and length, gather K/V from the physical blocks it names,
// run standard attention, write the output).  The kernels are our own design
// for 64-lane waves, matrix cores and HBM3E:
//   decode_mfma.h  bf16/fp16/fp8 KV on the matrix cores (fixed partitions,
//                  a balanced split of the whole batch over the GPU, and
//                  several query tokens per sequence)
//   decode_valu.h  fp32 KV, and 16-bit or fp8 KV without query-head
//                  grouping, on the vector ALUs (one workgroup per item, or
//                  workgroups fed from a work queue)
//   reduce.h       log-sum-exp merge of partial results
// The scatter kernel below writes new tokens' K/V rows into their slots.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "pagedattn.h"
#include "common.h"
#include "decode_mfma.h"
#include "decode_valu.h"
#include "reduce.h"

namespace pa {
namespace {

// Workgroups of the balanced split per launch: one per CU of an MI355X, so
// all ranges run in one round.
constexpr int kSkWorkgroups = 256;
// Largest batch the balanced split handles (its prefix sums live in LDS).
constexpr int kSkMaxSeqs = 16383;
// Most kv heads per workgroup of the queue-fed fixed split on the matrix cores.
constexpr int kMfmaQueueHeads = 8;
// Multi-token queries off the balanced split: from this many 16-row query
// tiles per (sequence, kv head) on, the tiles share each K/V block through
// LDS (16 per workgroup); one tile runs one wave per tile (8B batch, 5..8
// tokens: 391-402 us through LDS, 608-618 us one wave per tile).
constexpr int kPrefillLdsTiles = 2;
// Up to this many tiles the many-tile kernel runs one tile per wave.
constexpr int kPfOneTileWaveTiles = 4;

// ------------------------------------------------------------ scatter kernel

__global__ void __launch_bounds__(256)
pa_cache_scatter_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                        u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
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

// Scatter with quantisation to OCP fp8 e4m3: one thread per 16 elements of a
// token's row.  code = RNE_e4m3(saturate(x * inv_scale)), where x * inv_scale
// is an fp32 product, saturate clamps to the format's finite range +-448 and
// keeps NaN, and the rounding is the hardware's (nearest, ties to even).
constexpr float kFp8Max = 448.0f;

__device__ inline float fp8_saturate(float y) { return y > kFp8Max ? kFp8Max : (y < -kFp8Max ? -kFp8Max : y); }

template <class E>
__global__ void __launch_bounds__(256)
pa_cache_scatter_fp8_kernel(const char* __restrict__ key, const char* __restrict__ value,
                            u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
                            const int* __restrict__ slot_mapping, int row_chunks, int64_t num_slots,
                            float inv_k, float inv_v) {
  const int t = blockIdx.x;
  const int chunk = blockIdx.y * blockDim.x + threadIdx.x;
  if (chunk >= row_chunks) return;
  const int slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t src = ((int64_t)t * row_chunks + chunk) * 16 * E::kBytes;
  const int64_t dst = (int64_t)slot * row_chunks + chunk;
  auto quantise = [&](const char* base, float inv) {
    float x[16];
    const u32x4* in = reinterpret_cast<const u32x4*>(base + src);
#pragma unroll
    for (int i = 0; i < E::kBytes; ++i) widen16<E>(in[i], x + i * (16 / E::kBytes));
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_saturate(x[4 * w] * inv), fp8_saturate(x[4 * w + 1] * inv), 0, false);
      out[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fp8_saturate(x[4 * w + 2] * inv),
                                                         fp8_saturate(x[4 * w + 3] * inv), lo, true);
    }
    return out;
  };
  k_cache[dst] = quantise(key, inv_k);
  v_cache[dst] = quantise(value, inv_v);
}

// ------------------------------------------------------------ block copies

// Grid (pairs, chunk groups): each thread moves kCopyPerThread 16-byte chunks
// of the K block and as many of the V block, all loads before all stores.
// Sources are read once (non-temporal loads: 110 -> 86 us for 4096 pairs of
// 32 KiB blocks); destinations are written with the default policy, since the
// decode that follows reads them (non-temporal stores measured slower).
constexpr int kCopyPerThread = 2;

__global__ void __launch_bounds__(256)
pa_copy_blocks_kernel(u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, const int* __restrict__ src,
                      const int* __restrict__ dst, int block_chunks, int num_blocks) {
  const int i = blockIdx.x;
  const int s = src[i], d = dst[i];
  if ((unsigned)s >= (unsigned)num_blocks || (unsigned)d >= (unsigned)num_blocks) return;
  const int c0 = blockIdx.y * blockDim.x * kCopyPerThread + threadIdx.x;
  const int64_t so = (int64_t)s * block_chunks, dof = (int64_t)d * block_chunks;
  u32x4 k[kCopyPerThread], v[kCopyPerThread];
#pragma unroll
  for (int j = 0; j < kCopyPerThread; ++j) {
    const int c = c0 + j * blockDim.x;
    if (c < block_chunks) {
      k[j] = __builtin_nontemporal_load(k_cache + so + c);
      v[j] = __builtin_nontemporal_load(v_cache + so + c);
    }
  }
#pragma unroll
  for (int j = 0; j < kCopyPerThread; ++j) {
    const int c = c0 + j * blockDim.x;
    if (c < block_chunks) {
      k_cache[dof + c] = k[j];
      v_cache[dof + c] = v[j];
    }
  }
}

// ------------------------------------------------------------ host side

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_FP8_E4M3 ? 1 : 2); }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Fixed split: a 256-byte header (the work-queue counter of the vector-ALU
// launch), then one partial record per (sequence, query head, partition).
constexpr size_t kQueueHeaderBytes = 256;
size_t split_workspace_bytes(int num_seqs, int num_heads, int head_size, int num_parts) {
  return kQueueHeaderBytes + (size_t)num_seqs * num_heads * num_parts * (head_size + kRecHead) * sizeof(float);
}

// Partitions per sequence of the fixed split: max_seq_len, or the table
// row's capacity when 0 is passed, in partition_size pieces.
int split_num_parts(int block_size, int max_blocks_per_seq, int max_seq_len, int partition_size) {
  const long long cap = (long long)max_blocks_per_seq * block_size;
  const int msl = max_seq_len > 0 ? max_seq_len : (int)(cap < 0x7fffffffLL ? cap : 0x7fffffffLL);
  return msl > 0 ? ceil_div(msl, partition_size) : 1;
}

// Balanced split: one 16-byte entry per sequence (where its records are),
// then two partial records per workgroup per query head.
size_t balanced_seq_bytes(int num_seqs) { return align256((size_t)num_seqs * 16); }
size_t balanced_workspace_bytes(int num_seqs, int num_heads, int head_size) {
  return balanced_seq_bytes(num_seqs) + (size_t)kSkWorkgroups * num_heads * 2 * (head_size + kRecHead) * sizeof(float);
}

// Balanced split of multi-token queries: 16 * tiles record rows per kv head
// instead of G.
size_t balanced_mq_workspace_bytes(int num_seqs, int num_kv_heads, int head_size, int tiles) {
  return balanced_seq_bytes(num_seqs) +
         (size_t)kSkWorkgroups * num_kv_heads * 2 * 16 * tiles * (head_size + kRecHead) * sizeof(float);
}

// Rows per wave of the balanced-split merges: four (16 lanes each) when the
// batch has enough sequences that each row has few records, else one.  Long
// contexts over few sequences leave dozens of records per row, which a whole
// wave reads 16 at a time (8 x 32k tokens: 5.7 us with one row per wave,
// about twice that with four).
constexpr int kMergeQuadMinSeqs = 64;
int merge_rows_per_wave(int num_seqs) { return num_seqs >= kMergeQuadMinSeqs ? 4 : 1; }

// Largest divisor of num_kv_heads that is at most `most` (8: one wave per kv
// head, two waves per SIMD): kv heads per workgroup.
int heads_per_workgroup(int num_kv_heads, int most = 8) {
  for (int d = most; d > 1; --d)
    if (num_kv_heads % d == 0) return d;
  return 1;
}

// Multi-token queries on the balanced split: 16-row tiles per kv head (the
// kv head's max_q * G (token, head) rows), at most kSkMaxTiles; one wave per
// kv head holds them all (kv heads per workgroup as in decode).
constexpr int kSkMaxTiles = 2;
int mq_tiles(int num_heads, int num_kv_heads, int max_q) {      // kSkMaxTiles + 1: more than the split takes
  const long long rows = (long long)max_q * (num_heads / num_kv_heads);
  if (rows > 16LL * kSkMaxTiles) return kSkMaxTiles + 1;
  return rows > 0 ? (int)((rows + 15) / 16) : 1;
}

struct Args {
  void* out; const void* query; const char* kc; const char* vc;
  const int* bt; const int* sl;
  int num_seqs, num_heads, num_kv_heads, max_blocks, num_blocks, max_seq_len;
  float qk_scale, v_scale;
  int part_tokens, num_parts;
  void* ws;
  bool stream_kv, fp8_kv;
  bool queue;   // vector-ALU launch with partitions: workgroups take items from a counter
  bool longest_first;   // vector-ALU launch without partitions: items ordered by length
};

// Sets the vector-ALU launch's work-queue counter to 0 (a kernel rather than a
// memset, so that the call can be captured in a graph).
__global__ void __launch_bounds__(64) pa_queue_reset_kernel(int* __restrict__ queue) {
  if (threadIdx.x == 0) queue[0] = 0;
}

// The sequences in decreasing order of their block count (ties in any order;
// out-of-contract lengths count none, counts from kOrderBuckets - 1 on count
// alike).  One workgroup: counts per block count in LDS, their running sums,
// then each sequence takes the next place of its count.
constexpr int kOrderBuckets = 4096;
__global__ void __launch_bounds__(1024)
pa_order_by_length_kernel(const int* __restrict__ seq_lens, int num_seqs, int max_blocks, int* __restrict__ order) {
  __shared__ int cnt[kOrderBuckets];           // index kOrderBuckets - 1 - blocks: longest first
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < kOrderBuckets; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  auto slot = [&](int s) {
    const int L = seq_lens[s];
    const long long nb = (L > 0 && (long long)L <= (long long)max_blocks * kBlockSize) ? ceil_div(L, kBlockSize) : 0;
    return kOrderBuckets - 1 - (int)(nb < kOrderBuckets - 1 ? nb : kOrderBuckets - 1);
  };
  for (int s = tid; s < num_seqs; s += blockDim.x) atomicAdd(&cnt[slot(s)], 1);
  __syncthreads();
  // exclusive running sums: thread t owns entries 4t .. 4t + 3
  static_assert(kOrderBuckets == 4 * 1024, "four entries per thread");
  int v[4], tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = cnt[4 * tid + j]; tot += v[j]; }
  int inc = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int base = inc - tot;
  for (int w2 = 0; w2 < wv; ++w2) base += wsum[w2];
#pragma unroll
  for (int j = 0; j < 4; ++j) { cnt[4 * tid + j] = base; base += v[j]; }
  __syncthreads();
  for (int s = tid; s < num_seqs; s += blockDim.x) order[atomicAdd(&cnt[slot(s)], 1)] = s;
}

// Workgroups of `kernel` (`threads` lanes, no dynamic LDS) the current device
// holds at once, found once per (kernel, workgroup size, device); 0 if the
// runtime cannot tell.
int resident_workgroups(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(kernel, threads, dev);
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  cache[key] = cus * per_cu;
  return cus * per_cu;
}

template <class E, class KV, int D, int G, bool NT>
int launch_mfma(const Args& a, hipStream_t st) {
  if (a.part_tokens > 0) {
    int hpw = heads_per_workgroup(a.num_kv_heads);
    long long items = (long long)a.num_seqs * a.num_parts * (a.num_kv_heads / hpw);
    if (items > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    const int groups = a.num_kv_heads / hpw;
    // Up to two items per CU: one round of at most one workgroup per CU,
    // workgroup b taking items b and b + grid (grid a multiple of the head
    // groups, so both are of its head group), the first item's record held
    // until the second has streamed.  More items: workgroups of up to
    // kMfmaQueueHeads kv heads, as many as the GPU holds, take them from the
    // work queue (the dispatcher's in-order deal over the XCDs left slots
    // empty with items of unequal length).
    const long long wgs = kSkWorkgroups >= groups ? kSkWorkgroups / groups * groups : groups;
    long long grid = items <= 2 * wgs ? (items < wgs ? items : wgs) : items;
    float* ws = reinterpret_cast<float*>(static_cast<char*>(a.ws) + kQueueHeaderBytes);
    int* queue = nullptr;
    auto k = pa_decode_mfma_kernel<E, KV, D, G, NT>;
    if (items > 2 * wgs) {
      hpw = heads_per_workgroup(a.num_kv_heads, kMfmaQueueHeads);
      items = (long long)a.num_seqs * a.num_parts * (a.num_kv_heads / hpw);
      if (items > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
      queue = static_cast<int*>(a.ws);
      int slots = resident_workgroups(reinterpret_cast<const void*>(k), 64 * hpw);
      if (slots <= 0) slots = kSkWorkgroups * 8 / hpw;
      grid = items < slots ? items : slots;
      hipLaunchKernelGGL(pa_queue_reset_kernel, dim3(1), dim3(64), 0, st, queue);
      if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * hpw), 0, st,
                       a.out, a.query, a.kc, a.vc, a.bt, a.sl, a.num_heads, a.num_kv_heads, a.max_blocks,
                       a.num_blocks, a.qk_scale, a.v_scale, a.part_tokens, a.num_parts, hpw, (int)items, ws, queue);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    hipLaunchKernelGGL((pa_reduce_kernel<E, D>), dim3((unsigned)(a.num_seqs * a.num_heads)), dim3(64), 0, st,
                       a.out, ws, a.sl, a.num_heads, a.max_blocks, a.part_tokens, a.num_parts);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const int hpw = heads_per_workgroup(a.num_kv_heads);
  const int groups = a.num_kv_heads / hpw;
  const int nwg = kSkWorkgroups / groups > 0 ? kSkWorkgroups / groups : 1;
  int4* ws_seq = static_cast<int4*>(a.ws);
  float* ws_rec = reinterpret_cast<float*>(static_cast<char*>(a.ws) + balanced_seq_bytes(a.num_seqs));
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL((pa_decode_sk_kernel<E, KV, D, G, NT>), dim3((unsigned)(groups * nwg)), dim3(64 * hpw), lds, st,
                     a.out, a.query, a.kc, a.vc, a.bt, a.sl, a.num_seqs, a.num_heads, a.num_kv_heads, a.max_blocks,
                     a.num_blocks, a.qk_scale, a.v_scale, hpw, nwg, ws_seq, ws_rec);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (merge_rows_per_wave(a.num_seqs) == 4)
    hipLaunchKernelGGL((pa_sk_merge_kernel<E, D, G, 4>), dim3((unsigned)(a.num_seqs * ceil_div(a.num_heads, 4))),
                       dim3(64), 0, st, a.out, ws_seq, ws_rec, a.num_heads, hpw, nwg);
  else
    hipLaunchKernelGGL((pa_sk_merge_kernel<E, D, G, 1>), dim3((unsigned)(a.num_seqs * a.num_heads)), dim3(64), 0, st,
                       a.out, ws_seq, ws_rec, a.num_heads, hpw, nwg);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// One single-wave workgroup per (sequence, kv head[, partition]); or, with
// partitions and a.queue, workgroups of up to kValuMaxHeadsPerWg kv heads, as
// many as the GPU holds at once, that take (sequence, partition, head group)
// items from a counter in the workspace header.
template <class E, class KV, int D, int G>
int launch_valu(const Args& a, hipStream_t st) {
  const bool queued = a.queue && a.part_tokens > 0;
  const int hpw = queued ? heads_per_workgroup(a.num_kv_heads, kValuMaxHeadsPerWg) : 1;
  const long long items = (long long)a.num_seqs * a.num_parts * (a.num_kv_heads / hpw);
  if (items > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  auto k = a.stream_kv ? pa_decode_valu_kernel<E, KV, D, G, true> : pa_decode_valu_kernel<E, KV, D, G, false>;
  long long grid = items;
  int* queue = nullptr;
  int* order = nullptr;
  float* ws = nullptr;
  if (a.part_tokens > 0) ws = reinterpret_cast<float*>(static_cast<char*>(a.ws) + kQueueHeaderBytes);
  if (a.longest_first && a.part_tokens == 0) {
    order = static_cast<int*>(a.ws);
    hipLaunchKernelGGL(pa_order_by_length_kernel, dim3(1), dim3(1024), 0, st, a.sl, a.num_seqs, a.max_blocks, order);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  if (queued) {
    queue = static_cast<int*>(a.ws);
    int slots = resident_workgroups(reinterpret_cast<const void*>(k), 64 * hpw);
    if (slots <= 0) slots = kSkWorkgroups * 4 * ValuOccupancy<E, KV, D, G>::kWaves / hpw;
    grid = items < slots ? items : slots;
    hipLaunchKernelGGL(pa_queue_reset_kernel, dim3(1), dim3(64), 0, st, queue);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * hpw), 0, st,
                     a.out, a.query, a.kc, a.vc, a.bt, a.sl, a.num_heads, a.num_kv_heads, a.max_blocks,
                     a.num_blocks, a.qk_scale, a.v_scale, a.part_tokens, a.num_parts, ws, (int)items, queue, order);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  if (a.part_tokens > 0) {
    hipLaunchKernelGGL((pa_reduce_kernel<E, D>), dim3((unsigned)(a.num_seqs * a.num_heads)), dim3(64), 0, st,
                       a.out, ws, a.sl, a.num_heads, a.max_blocks, a.part_tokens, a.num_parts);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

// One query head per kv head (no grouping) leaves the matrix-core tile 1/16
// dense; there the vector-ALU core runs.  Over 16-bit pools one workgroup per
// (sequence, kv head[, partition]); without partitions the sequences are
// first ordered longest first, so that the longest items (one wave streams a
// 2036-token sequence for ~230 us) start at once and short ones fill in
// behind them (13B-shaped batch, 64 seqs x 40 heads, lengths 128..2048: 234.2
// us, in the order given 251.5 us; fed from the work queue with 512-token
// partitions 262 us).  Over
// fp8 pools, where a wave's share of a block is half as large, the work queue
// with partitions wins: 142.1 us with the 256-token partitions chosen here
// (512: 144.9, 1024: 158) and 145.3 us with partition_size 512, against 150.4
// us for the balanced split on the matrix cores and 157.2 us for one
// workgroup per item.  Both need enough (sequence, kv head) items to keep
// every CU busy; fewer take the balanced split on the matrix cores.
constexpr long long kValuMhaMinItems = 1024;
constexpr int kValuPartTokens = 256;
constexpr bool kValuQueue16 = true;

// Partition size of the queue-fed vector-ALU launch for partition_size 0
// (0: the records would not fit at any size; the caller takes another path).
int valu_part_tokens(const Args& a, int head_size) {
  const size_t cap = balanced_workspace_bytes(a.num_seqs, a.num_heads, head_size);
  for (int pt = kValuPartTokens; pt <= (1 << 29); pt *= 2) {
    const int np = split_num_parts(kBlockSize, a.max_blocks, a.max_seq_len, pt);
    if (np <= 1 || split_workspace_bytes(a.num_seqs, a.num_heads, head_size, np) <= cap) return pt;
  }
  return 0;
}

// The queued vector-ALU launch with partitions the library picks, when those
// give enough (sequence, partition, kv head) items (an upper bound: the
// partitions max_seq_len needs, for every sequence).
bool queued_partitions(const Args& a, int head_size, Args& b) {
  b = a;
  b.queue = true;
  b.part_tokens = valu_part_tokens(a, head_size);
  if (b.part_tokens <= 0) return false;
  b.num_parts = split_num_parts(kBlockSize, a.max_blocks, a.max_seq_len, b.part_tokens);
  return (long long)a.num_seqs * b.num_parts * a.num_kv_heads >= kValuMhaMinItems;
}

template <class E, int D, int G>
int launch(const Args& a, hipStream_t st) {
  if constexpr (E::kBytes == 4) {
    return launch_valu<E, Kv16, D, G>(a, st);
  } else if (a.fp8_kv) {
    if constexpr (G == 1) {
      Args b = a;
      b.queue = true;
      if (a.part_tokens > 0) return launch_valu<E, KvFp8, D, G>(b, st);
      if (queued_partitions(a, D, b)) return launch_valu<E, KvFp8, D, G>(b, st);
    }
    return a.stream_kv ? launch_mfma<E, KvFp8, D, G, true>(a, st) : launch_mfma<E, KvFp8, D, G, false>(a, st);
  } else {
    if constexpr (G == 1) {
      if (a.part_tokens > 0) return launch_valu<E, Kv16, D, G>(a, st);
      Args b = a;
      if ((long long)a.num_seqs * a.num_kv_heads >= kValuMhaMinItems) {
        b.longest_first = true;
        return launch_valu<E, Kv16, D, G>(b, st);
      }
      if (kValuQueue16 && queued_partitions(a, D, b)) return launch_valu<E, Kv16, D, G>(b, st);
    }
    return a.stream_kv ? launch_mfma<E, Kv16, D, G, true>(a, st) : launch_mfma<E, Kv16, D, G, false>(a, st);
  }
}

template <class E, int D>
int dispatch_group(const Args& a, int group, hipStream_t st) {
  switch (group) {
    case 1: return launch<E, D, 1>(a, st);
    case 2: return launch<E, D, 2>(a, st);
    case 4: return launch<E, D, 4>(a, st);
    case 8: return launch<E, D, 8>(a, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <class E>
int dispatch_head(const Args& a, int head_size, int group, hipStream_t st) {
  switch (head_size) {
    case 64: return dispatch_group<E, 64>(a, group, st);
    case 128: return dispatch_group<E, 128>(a, group, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace
}  // namespace pa

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_CAPACITY: return "block table full";
    case PA_ERR_SCRATCH: return "request exceeds the library's fixed scratch buffer";
    default: return "unknown status";
  }
}

extern "C" size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_size,
                                           int max_seq_len, int partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_size <= 0 || max_seq_len < 0 || partition_size < 0) return 0;
  if (partition_size == 0) return pa::balanced_workspace_bytes(num_seqs, num_heads, head_size);
  const int np = max_seq_len > 0 ? pa::ceil_div(max_seq_len, partition_size) : 1;
  return pa::split_workspace_bytes(num_seqs, num_heads, head_size, np);
}

// Device memory of paged_attention_decode_noalloc: it stands in for the
// caller's workspace.  Each device the library runs on holds its own copy
// until the process ends; every call on a device shares it.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kScratchMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchMaxDevices];   // per device, found once with that device current
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (the host-side name
// of the array is only a stand-in, never a device address).  The stream, if
// not the null stream, must belong to the current device.
int scratch_address(void* stream, void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kScratchMaxDevices) return PA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return PA_ERR_HIP;
    if (sdev != dev) return PA_ERR_INVALID_ARG;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PA_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}


// Workspace bytes a decode call with these (already validated) sizes uses.
size_t decode_workspace_need(int num_seqs, int num_heads, int head_size, int block_size, int max_blocks_per_seq,
                             int max_seq_len, int partition_size, int dtype) {
  if (partition_size > 0)
    return split_workspace_bytes(num_seqs, num_heads, head_size,
                                 split_num_parts(block_size, max_blocks_per_seq, max_seq_len, partition_size));
  return dtype != PA_F32 ? balanced_workspace_bytes(num_seqs, num_heads, head_size) : 0;
}

int decode_impl(void* out, const void* query, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* seq_lens, int num_seqs, int num_heads,
                int num_kv_heads, int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                int max_seq_len, float scale, int dtype, int partition_size, unsigned flags, void* workspace,
                size_t workspace_bytes, void* stream, bool fp8_kv, float k_scale, float v_scale,
                bool noalloc = false) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 ||
      max_blocks_per_seq < 0 || num_blocks < 0 || max_seq_len < 0 || partition_size < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (flags & ~(unsigned)PA_FLAG_SHARED_BLOCKS) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  const int group = num_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % block_size != 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PA_ERR_INVALID_ARG;
  const int kv_bytes = fp8_kv ? 1 : elem_bytes(dtype);
  if ((long long)kBlockSize * num_kv_heads * head_size * kv_bytes > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;

  const size_t need = decode_workspace_need(num_seqs, num_heads, head_size, block_size, max_blocks_per_seq,
                                            max_seq_len, partition_size, dtype);
  if (partition_size == 0 && dtype != PA_F32 && num_seqs > kSkMaxSeqs) return PA_ERR_UNSUPPORTED;
  if (noalloc && need > 0) {                  // the library's scratch array in place of a workspace
    if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
    const int rc = scratch_address(stream, &workspace);
    if (rc != PA_OK) return rc;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }

  Args a{};
  a.out = out; a.query = query;
  a.kc = static_cast<const char*>(k_cache); a.vc = static_cast<const char*>(v_cache);
  a.bt = block_tables; a.sl = seq_lens;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.num_kv_heads = num_kv_heads;
  a.max_blocks = max_blocks_per_seq; a.num_blocks = num_blocks; a.max_seq_len = max_seq_len;
  a.qk_scale = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  a.v_scale = v_scale;
  a.fp8_kv = fp8_kv;
  a.part_tokens = 0; a.num_parts = 1;
  a.stream_kv = (flags & PA_FLAG_SHARED_BLOCKS) == 0;
  if (partition_size > 0) {
    a.part_tokens = partition_size;
    a.num_parts = split_num_parts(block_size, max_blocks_per_seq, max_seq_len, partition_size);
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return PA_ERR_WORKSPACE;
    a.ws = workspace;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PA_F32: return dispatch_head<ElemF32>(a, head_size, group, st);
    case PA_F16: return dispatch_head<ElemF16>(a, head_size, group, st);
    default: return dispatch_head<ElemBF16>(a, head_size, group, st);
  }
}

bool positive_finite(float x) { return x > 0.f && x <= 3.4028234663852886e38f; }

template <class E, class KV, int D, int G>
int launch_prefill(void* out, const void* query, const void* kc, const void* vc, const int32_t* bt,
                   const int32_t* sl, const int32_t* qs, int num_seqs, int num_heads, int num_kv_heads,
                   int max_blocks, int num_blocks, int max_query_len, float qk_scale, float v_scale, bool nt,
                   const int* order, hipStream_t st) {
  const int tiles = ceil_div(max_query_len * G, 16);
  if (tiles >= kPrefillLdsTiles) {
    // many query tiles per (sequence, kv head): the tiles of a workgroup share K/V through LDS.
    // Up to 8 tiles take workgroups of 8 (4 waves): 8B batch, 12 query tokens (3 tiles), 346 us
    // against 411 us with workgroups of 16; the chunked-prefill batch (128 tiles) 307 against 269 us.
    const int tpg = tiles <= kPfSmallGroupTiles ? kPfSmallGroupTiles : 16;
    const int gpp = ceil_div(tiles, tpg);
    const long long pairs = (long long)num_seqs * num_kv_heads;
    const long long grid = (pairs + 7) / 8 * 8 * gpp;
    if (grid > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    constexpr int TW = kPfTilesPerWave;
    if (tiles <= kPfOneTileWaveTiles) {
      // few tiles: workgroups of 4 waves with one tile each, so that fewer
      // waves only stage blocks (8B batch, 5 / 8 / 12 / 16 query tokens:
      // 268.4 / 276.6 / 285.4 / 292.6 us against 274.9 / 282.5 / 292.8 /
      // 298.6 us with two tiles per wave)
      auto k1 = nt ? pa_prefill_lds_kernel<E, KV, D, G, true, 1, 4> : pa_prefill_lds_kernel<E, KV, D, G, false, 1, 4>;
      const long long gpp1 = ceil_div(tiles, 4), grid1 = (pairs + 7) / 8 * 8 * gpp1;
      if (grid1 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
      hipLaunchKernelGGL(k1, dim3((unsigned)grid1), dim3(256), 0, st, out, query,
                         static_cast<const char*>(kc), static_cast<const char*>(vc), bt, sl, qs, num_seqs, num_heads,
                         num_kv_heads, max_blocks, num_blocks, (int)gpp1, qk_scale, v_scale, order);
      return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    auto k = tpg == 16 ? (nt ? pa_prefill_lds_kernel<E, KV, D, G, true, TW, 16> : pa_prefill_lds_kernel<E, KV, D, G, false, TW, 16>)
                       : (nt ? pa_prefill_lds_kernel<E, KV, D, G, true, TW, kPfSmallGroupTiles>
                             : pa_prefill_lds_kernel<E, KV, D, G, false, TW, kPfSmallGroupTiles>);
    hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(64 * tpg / TW), 0, st, out, query,
                       static_cast<const char*>(kc), static_cast<const char*>(vc), bt, sl, qs, num_seqs, num_heads,
                       num_kv_heads, max_blocks, num_blocks, gpp, qk_scale, v_scale, order);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const dim3 grid((unsigned)ceil_div(tiles, 4), (unsigned)num_seqs, (unsigned)num_kv_heads);
  auto k = nt ? pa_prefill_kernel<E, KV, D, G, true> : pa_prefill_kernel<E, KV, D, G, false>;
  hipLaunchKernelGGL(k, grid, dim3(256), 0, st, out, query, static_cast<const char*>(kc),
                     static_cast<const char*>(vc), bt, sl, qs, num_heads, num_kv_heads, max_blocks, num_blocks,
                     qk_scale, v_scale);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <class E, class KV, int D>
int prefill_group(int group, void* out, const void* query, const void* kc, const void* vc, const int32_t* bt,
                  const int32_t* sl, const int32_t* qs, int S, int Hq, int Hkv, int MB, int NB, int mq, float qks,
                  float vs, bool nt, const int* order, hipStream_t st) {
  switch (group) {
    case 1: return launch_prefill<E, KV, D, 1>(out, query, kc, vc, bt, sl, qs, S, Hq, Hkv, MB, NB, mq, qks, vs, nt, order, st);
    case 2: return launch_prefill<E, KV, D, 2>(out, query, kc, vc, bt, sl, qs, S, Hq, Hkv, MB, NB, mq, qks, vs, nt, order, st);
    case 4: return launch_prefill<E, KV, D, 4>(out, query, kc, vc, bt, sl, qs, S, Hq, Hkv, MB, NB, mq, qks, vs, nt, order, st);
    case 8: return launch_prefill<E, KV, D, 8>(out, query, kc, vc, bt, sl, qs, S, Hq, Hkv, MB, NB, mq, qks, vs, nt, order, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <class E, class KV, int D, int G>
int launch_mq_split(void* out, const void* query, const void* kc, const void* vc, const int32_t* bt,
                    const int32_t* sl, const int32_t* qs, int num_seqs, int num_heads, int num_kv_heads,
                    int max_blocks, int num_blocks, int max_q, float qk_scale, float v_scale, bool nt, void* ws,
                    hipStream_t st) {
  const int tiles = mq_tiles(num_heads, num_kv_heads, max_q);
  const int hpw = heads_per_workgroup(num_kv_heads, tiles == 2 && sk_wide<D, 2>() ? kSkWideHeads : 8);
  const int groups = num_kv_heads / hpw;
  const int nwg = kSkWorkgroups / groups > 0 ? kSkWorkgroups / groups : 1;
  int4* ws_seq = static_cast<int4*>(ws);
  float* ws_rec = reinterpret_cast<float*>(static_cast<char*>(ws) + balanced_seq_bytes(num_seqs));
  const size_t lds = (size_t)2 * (num_seqs + 1) * sizeof(int);
  // one wave per kv head holds all of its tiles, so each K/V line is read once
  auto k = tiles == 1 ? (nt ? pa_decode_sk_kernel<E, KV, D, G, true, true, 1> : pa_decode_sk_kernel<E, KV, D, G, false, true, 1>)
                      : (nt ? pa_decode_sk_kernel<E, KV, D, G, true, true, 2> : pa_decode_sk_kernel<E, KV, D, G, false, true, 2>);
  hipLaunchKernelGGL(k, dim3((unsigned)(groups * nwg)), dim3(64 * hpw), lds, st, out, query,
                     static_cast<const char*>(kc), static_cast<const char*>(vc), bt, sl, num_seqs, num_heads,
                     num_kv_heads, max_blocks, num_blocks, qk_scale, v_scale, hpw, nwg, ws_seq, ws_rec, qs);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  const int rpw = merge_rows_per_wave(num_seqs);
  const long long grid = (long long)num_seqs * num_kv_heads * ceil_div(max_q * G, rpw);
  auto mk = rpw == 4 ? pa_sk_merge_mq_kernel<E, D, G, 4> : pa_sk_merge_mq_kernel<E, D, G, 1>;
  hipLaunchKernelGGL(mk, dim3((unsigned)grid), dim3(64), 0, st, out, ws_seq, ws_rec, qs, num_heads, hpw, nwg, max_q,
                     16 * tiles);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Which path a multi-token call takes, and the workspace it needs.
// The many-tile kernel's grid runs the sequences longest first when there are
// at least kOrderMinSeqs of them (the order takes 4 bytes per sequence of the
// workspace): 8B batch, 256 sequences, 16 / 12 query tokens each: 293.7 /
// 288.0 us against 352.0 / 343.5 us in the order given.  A few sequences (a
// chunked prefill) gain nothing from it and would pay for the extra kernel.
// So ordered, it also beats the balanced split for two tiles per kv head
// once the (sequence, kv head) pairs fill the GPU (5 / 8 tokens: 274.3 /
// 282.3 us against 287.9 / 299.0 us), though three of its four waves then
// only stage blocks; smaller batches (few long sequences) keep the split.
constexpr int kOrderMinSeqs = 32;
constexpr long long kLdsTwoTileMinPairs = 1024;

bool prefill_uses_split(int num_seqs, int num_heads, int num_kv_heads, int max_q) {
  const int tiles = mq_tiles(num_heads, num_kv_heads, max_q);
  if (tiles > kSkMaxTiles || num_seqs > kSkMaxSeqs) return false;
  return !(tiles == 2 && num_seqs >= kOrderMinSeqs && (long long)num_seqs * num_kv_heads >= kLdsTwoTileMinPairs);
}

bool prefill_longest_first(int num_seqs, int num_heads, int num_kv_heads, int max_q) {
  return !prefill_uses_split(num_seqs, num_heads, num_kv_heads, max_q) &&
         ceil_div(max_q * (num_heads / num_kv_heads), 16) >= kPrefillLdsTiles && num_seqs >= kOrderMinSeqs;
}

size_t prefill_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_q) {
  if (prefill_uses_split(num_seqs, num_heads, num_kv_heads, max_q))
    return balanced_mq_workspace_bytes(num_seqs, num_kv_heads, head_size, mq_tiles(num_heads, num_kv_heads, max_q));
  return prefill_longest_first(num_seqs, num_heads, num_kv_heads, max_q) ? align256((size_t)num_seqs * 4) : 0;
}

int prefill_impl(void* out, const void* query, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start, int num_seqs,
                 int num_query_tokens, int num_heads, int num_kv_heads, int head_size, int block_size,
                 int max_blocks_per_seq, int num_blocks, int max_query_len, float scale, int dtype, unsigned flags,
                 void* workspace, size_t workspace_bytes, void* stream, bool fp8_kv, float k_scale,
                 float v_scale) {
  if (num_seqs < 0 || num_query_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0 || max_query_len < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (flags & ~(unsigned)PA_FLAG_SHARED_BLOCKS) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  const int group = num_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start) return PA_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PA_ERR_INVALID_ARG;
  const int kv_bytes = fp8_kv ? 1 : elem_bytes(dtype);
  if ((long long)kBlockSize * num_kv_heads * head_size * kv_bytes > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  const int mq = max_query_len > 0 ? max_query_len : num_query_tokens;
  const float qks = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  const bool nt = (flags & PA_FLAG_SHARED_BLOCKS) == 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (prefill_uses_split(num_seqs, num_heads, num_kv_heads, mq)) {
    const size_t need = balanced_mq_workspace_bytes(num_seqs, num_kv_heads, head_size,
                                                    mq_tiles(num_heads, num_kv_heads, mq));
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return PA_ERR_WORKSPACE;
#define PA_MQ(E, KV, D, G) launch_mq_split<E, KV, D, G>(out, query, k_cache, v_cache, block_tables, seq_lens, \
    query_start, num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, num_blocks, mq, qks, v_scale, nt, workspace, st)
#define PA_MQ_G(E, KV, D) (group == 1 ? PA_MQ(E, KV, D, 1) : group == 2 ? PA_MQ(E, KV, D, 2) : \
                           group == 4 ? PA_MQ(E, KV, D, 4) : PA_MQ(E, KV, D, 8))
    if (dtype == PA_F16) {
      if (fp8_kv) return head_size == 64 ? PA_MQ_G(ElemF16, KvFp8, 64) : PA_MQ_G(ElemF16, KvFp8, 128);
      return head_size == 64 ? PA_MQ_G(ElemF16, Kv16, 64) : PA_MQ_G(ElemF16, Kv16, 128);
    }
    if (fp8_kv) return head_size == 64 ? PA_MQ_G(ElemBF16, KvFp8, 64) : PA_MQ_G(ElemBF16, KvFp8, 128);
    return head_size == 64 ? PA_MQ_G(ElemBF16, Kv16, 64) : PA_MQ_G(ElemBF16, Kv16, 128);
#undef PA_MQ_G
#undef PA_MQ
  }
  int* order = nullptr;
  if (prefill_longest_first(num_seqs, num_heads, num_kv_heads, mq)) {
    const size_t need = align256((size_t)num_seqs * 4);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return PA_ERR_WORKSPACE;
    order = static_cast<int*>(workspace);
    hipLaunchKernelGGL(pa_order_by_length_kernel, dim3(1), dim3(1024), 0, st, seq_lens, num_seqs,
                       max_blocks_per_seq, order);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
#define PA_PREFILL(E, KV, D) prefill_group<E, KV, D>(group, out, query, k_cache, v_cache, block_tables, seq_lens, \
    query_start, num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, num_blocks, mq, qks, v_scale, nt, order, st)
  if (dtype == PA_F16) {
    if (fp8_kv) return head_size == 64 ? PA_PREFILL(ElemF16, KvFp8, 64) : PA_PREFILL(ElemF16, KvFp8, 128);
    return head_size == 64 ? PA_PREFILL(ElemF16, Kv16, 64) : PA_PREFILL(ElemF16, Kv16, 128);
  }
  if (fp8_kv) return head_size == 64 ? PA_PREFILL(ElemBF16, KvFp8, 64) : PA_PREFILL(ElemBF16, KvFp8, 128);
  return head_size == 64 ? PA_PREFILL(ElemBF16, Kv16, 64) : PA_PREFILL(ElemBF16, Kv16, 128);
#undef PA_PREFILL
}

template <class E>
void launch_scatter_fp8(const void* key, const void* value, void* k_cache, void* v_cache, const int32_t* slots,
                        int num_tokens, int row_chunks, int64_t num_slots, float inv_k, float inv_v,
                        hipStream_t st) {
  const int threads = row_chunks >= 256 ? 256 : (row_chunks + 63) / 64 * 64;
  const dim3 grid((unsigned)num_tokens, (unsigned)((row_chunks + threads - 1) / threads));
  hipLaunchKernelGGL(pa_cache_scatter_fp8_kernel<E>, grid, dim3(threads), 0, st, static_cast<const char*>(key),
                     static_cast<const char*>(value), static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                     slots, row_chunks, num_slots, inv_k, inv_v);
}

}  // namespace
}  // namespace pa

extern "C" int paged_attention_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int dtype, int partition_size,
                                      unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype == PA_FP8_E4M3) return PA_ERR_INVALID_ARG;
  return pa::decode_impl(out, query, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                         head_size, block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale, dtype,
                         partition_size, flags, workspace, workspace_bytes, stream, false, 1.0f, 1.0f);
}

extern "C" int paged_attention_decode_noalloc(void* out, const void* query, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              const int32_t* seq_lens, int num_seqs, int num_heads,
                                              int num_kv_heads, int head_size, int block_size,
                                              int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                                              int dtype, int partition_size, unsigned flags, void* stream) {
  if (dtype == PA_FP8_E4M3) return PA_ERR_INVALID_ARG;
  return pa::decode_impl(out, query, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                         head_size, block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale, dtype,
                         partition_size, flags, nullptr, 0, stream, false, 1.0f, 1.0f, true);
}

extern "C" int paged_attention_decode_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                          int block_size, int max_blocks_per_seq, int num_blocks,
                                          int max_seq_len, float scale, float k_scale, float v_scale, int dtype,
                                          int partition_size, unsigned flags, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (dtype != PA_F16 && dtype != PA_BF16) return dtype == PA_F32 ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
  if (!pa::positive_finite(k_scale) || !pa::positive_finite(v_scale)) return PA_ERR_INVALID_ARG;
  return pa::decode_impl(out, query, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                         head_size, block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale, dtype,
                         partition_size, flags, workspace, workspace_bytes, stream, true, k_scale, v_scale);
}

extern "C" int reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                                     const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_size,
                                     int block_size, int num_blocks, int dtype, float k_scale, float v_scale,
                                     void* stream) {
  using namespace pa;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (!positive_finite(k_scale) || !positive_finite(v_scale)) return PA_ERR_INVALID_ARG;
  const long long row_elems = (long long)num_kv_heads * head_size;
  if (row_elems % 16 != 0 || row_elems / 16 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PA_ERR_INVALID_ARG;
  const float inv_k = (float)(1.0 / (double)k_scale), inv_v = (float)(1.0 / (double)v_scale);
  const int chunks = (int)(row_elems / 16);
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PA_F32: launch_scatter_fp8<ElemF32>(key, value, k_cache, v_cache, slot_mapping, num_tokens, chunks, num_slots, inv_k, inv_v, st); break;
    case PA_F16: launch_scatter_fp8<ElemF16>(key, value, k_cache, v_cache, slot_mapping, num_tokens, chunks, num_slots, inv_k, inv_v, st); break;
    default: launch_scatter_fp8<ElemBF16>(key, value, k_cache, v_cache, slot_mapping, num_tokens, chunks, num_slots, inv_k, inv_v, st); break;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" int reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                 const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_size, int block_size, int num_blocks, int dtype, void* stream) {
  using namespace pa;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  const long long row_bytes = (long long)num_kv_heads * head_size * elem_bytes(dtype);
  if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PA_ERR_INVALID_ARG;
  const long long chunks = row_bytes / 16;
  if (chunks > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  const int threads = chunks >= 256 ? 256 : (int)((chunks + 63) / 64 * 64);
  const dim3 grid((unsigned)num_tokens, (unsigned)((chunks + threads - 1) / threads));
  hipLaunchKernelGGL(pa_cache_scatter_kernel, grid, dim3(threads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slot_mapping,
                     (int)chunks, (int64_t)num_blocks * block_size);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

extern "C" int copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int num_pairs,
                           int num_kv_heads, int head_size, int block_size, int num_blocks, int dtype,
                           void* stream) {
  using namespace pa;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_size <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3) return PA_ERR_INVALID_ARG;
  const long long block_bytes = (long long)block_size * num_kv_heads * head_size * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (block_bytes / 16 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src || !dst) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return PA_ERR_INVALID_ARG;
  const int chunks = (int)(block_bytes / 16);
  const int per_group = 256 * kCopyPerThread;
  const dim3 grid((unsigned)num_pairs, (unsigned)((chunks + per_group - 1) / per_group));
  hipLaunchKernelGGL(pa_copy_blocks_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), src, dst, chunks, num_blocks);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" size_t pa_prefill_workspace_size(int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                                            int head_size, int max_query_len) {
  if (num_seqs <= 0 || num_query_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      max_query_len < 0 || num_heads % num_kv_heads != 0)
    return 0;
  const int mq = max_query_len > 0 ? max_query_len : num_query_tokens;
  return pa::prefill_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, mq);
}

extern "C" int paged_attention_prefill(void* out, const void* query, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       const int32_t* query_start, int num_seqs, int num_query_tokens,
                                       int num_heads, int num_kv_heads, int head_size, int block_size,
                                       int max_blocks_per_seq, int num_blocks, int max_query_len, float scale,
                                       int dtype, unsigned flags, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return pa::prefill_impl(out, query, k_cache, v_cache, block_tables, seq_lens, query_start, num_seqs,
                          num_query_tokens, num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                          num_blocks, max_query_len, scale, dtype, flags, workspace, workspace_bytes, stream, false,
                          1.0f, 1.0f);
}

extern "C" int paged_attention_prefill_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           const int32_t* query_start, int num_seqs, int num_query_tokens,
                                           int num_heads, int num_kv_heads, int head_size, int block_size,
                                           int max_blocks_per_seq, int num_blocks, int max_query_len, float scale,
                                           float k_scale, float v_scale, int dtype, unsigned flags,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!pa::positive_finite(k_scale) || !pa::positive_finite(v_scale)) return PA_ERR_INVALID_ARG;
  return pa::prefill_impl(out, query, k_cache, v_cache, block_tables, seq_lens, query_start, num_seqs,
                          num_query_tokens, num_heads, num_kv_heads, head_size, block_size, max_blocks_per_seq,
                          num_blocks, max_query_len, scale, dtype, flags, workspace, workspace_bytes, stream, true,
                          k_scale, v_scale);
}
