// Host-side block manager of the paged KV cache: the C ABI pa_bm_* of
// include/pagedattn.h.
//
// What it does follows the devpress.csdn.net article on the vLLM
// architecture: section 1 (the KV-cache manager cuts GPU memory into
// fixed-size blocks kept in one global free pool, answers a sequence's
// requests for blocks, keeps the logical -> physical map, and uses reference
// counts for copy-on-write so blocks can be shared, e.g. by beam search) and
// section 2 (a scheduled request gets its blocks and table; a new token that
// needs a new block asks again).  The pool order follows the yangyitao.com
// vLLM book preface, "from OS to GPU" figure: freed blocks go straight to the
// next request, so the pool is a stack.
//
// Layout: one table (int32 physical ids) per sequence slot, reference counts
// per block, the free pool as a stack, and the queue of pending copies
// (shared source, fresh destination) that the caller hands to copy_blocks.
// Every operation checks everything it needs before changing anything, so a
// failed call leaves the manager as it was.  Not thread-safe: the caller
// serialises calls on one manager.

#include <stdint.h>

#include <new>
#include <utility>
#include <vector>

#include "pagedattn.h"

struct pa_block_manager {
  int num_blocks = 0, block_size = 0, max_seqs = 0, max_blocks_per_seq = 0;
  std::vector<int32_t> free_stack;                 // the next block handed out is back()
  std::vector<int32_t> ref;                        // reference count per block
  std::vector<std::vector<int32_t>> tables;        // per sequence id
  std::vector<int32_t> len;                        // tokens per sequence id, -1: no sequence
  std::vector<std::pair<int32_t, int32_t>> copies;
  std::vector<int32_t> scratch_block;              // per block: pending reference drops (batch check)
  std::vector<uint8_t> scratch_seq;                // per sequence: seen in the batch

  int blocks_for(int64_t tokens) const { return (int)((tokens + block_size - 1) / block_size); }
  bool live(int seq) const { return seq >= 0 && seq < max_seqs && len[seq] >= 0; }
  bool free_id(int seq) const { return seq >= 0 && seq < max_seqs && len[seq] < 0; }
  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  void write_slots(int seq, int first, int n, int32_t* slots) const {
    if (!slots) return;
    const std::vector<int32_t>& t = tables[seq];
    for (int i = 0; i < n; ++i) {
      const int tok = first + i;
      slots[i] = t[tok / block_size] * block_size + tok % block_size;
    }
  }
};

extern "C" int pa_bm_create(int num_blocks, int block_size, int max_seqs, int max_blocks_per_seq,
                            pa_block_manager** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0 || max_seqs < 0 || max_blocks_per_seq < 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)num_blocks * block_size > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;   // slots are int32
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return PA_ERR_INVALID_ARG;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_seqs = max_seqs;
    bm->max_blocks_per_seq = max_blocks_per_seq;
    bm->free_stack.resize(num_blocks);
    for (int i = 0; i < num_blocks; ++i) bm->free_stack[i] = num_blocks - 1 - i;   // block 0 first out
    bm->ref.assign(num_blocks, 0);
    bm->tables.resize(max_seqs);
    bm->len.assign(max_seqs, -1);
    bm->scratch_block.assign(num_blocks, 0);
    bm->scratch_seq.assign(max_seqs, 0);
  } catch (...) {
    delete bm;
    return PA_ERR_INVALID_ARG;
  }
  *out = bm;
  return PA_OK;
}

extern "C" void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

extern "C" int pa_bm_allocate(pa_block_manager* bm, int seq, int num_tokens, int32_t* slots) {
  if (!bm || !bm->free_id(seq) || num_tokens < 0) return PA_ERR_INVALID_ARG;
  const int nb = bm->blocks_for(num_tokens);
  if (nb > bm->max_blocks_per_seq) return PA_ERR_CAPACITY;
  if (nb > (int)bm->free_stack.size()) return PA_ERR_NO_BLOCKS;
  std::vector<int32_t>& t = bm->tables[seq];
  try {
    t.reserve(nb);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  t.clear();
  for (int i = 0; i < nb; ++i) t.push_back(bm->take());
  bm->len[seq] = num_tokens;
  bm->write_slots(seq, 0, num_tokens, slots);
  return PA_OK;
}

extern "C" int pa_bm_append_slots(pa_block_manager* bm, int seq, int num_tokens, int32_t* slots) {
  if (!bm || !bm->live(seq) || num_tokens < 0) return PA_ERR_INVALID_ARG;
  std::vector<int32_t>& t = bm->tables[seq];
  const int L = bm->len[seq];
  const int64_t new_len = (int64_t)L + num_tokens;
  if (new_len > 0x7fffffffLL) return PA_ERR_CAPACITY;
  const int need_blocks = bm->blocks_for(new_len);
  if (need_blocks > bm->max_blocks_per_seq) return PA_ERR_CAPACITY;
  const int grow = need_blocks - (int)t.size();
  // first write into a partly filled block that another sequence shares
  const bool cow = num_tokens > 0 && L % bm->block_size != 0 && bm->ref[t.back()] > 1;
  if (grow + (cow ? 1 : 0) > (int)bm->free_stack.size()) return PA_ERR_NO_BLOCKS;
  try {
    t.reserve(need_blocks);
    if (cow) bm->copies.reserve(bm->copies.size() + 1);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  if (cow) {
    const int32_t old = t.back();
    const int32_t fresh = bm->take();
    bm->ref[old] -= 1;
    t.back() = fresh;
    bm->copies.emplace_back(old, fresh);
  }
  for (int i = 0; i < grow; ++i) t.push_back(bm->take());
  bm->len[seq] = (int)new_len;
  bm->write_slots(seq, L, num_tokens, slots);
  return PA_OK;
}

extern "C" int pa_bm_append_batch(pa_block_manager* bm, const int32_t* seqs, int num_seqs, int32_t* slots) {
  if (!bm || num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!seqs) return PA_ERR_INVALID_ARG;
  // check the whole batch first, in this order: ids live and distinct, then
  // table capacity, then enough free blocks for the new blocks and copies
  // the appends need in order (a shared block copied for one sequence may be
  // private by the time a later sequence of the batch writes into it)
  int status = PA_OK;
  int marked = 0;
  for (; marked < num_seqs; ++marked) {
    const int s = seqs[marked];
    if (!bm->live(s) || bm->scratch_seq[s]) { status = PA_ERR_INVALID_ARG; break; }
    bm->scratch_seq[s] = 1;
  }
  for (int i = 0; i < marked; ++i) bm->scratch_seq[seqs[i]] = 0;
  if (status != PA_OK) return status;
  for (int i = 0; i < num_seqs; ++i) {
    const int L = bm->len[seqs[i]];
    if (L == 0x7fffffff || bm->blocks_for((int64_t)L + 1) > bm->max_blocks_per_seq) return PA_ERR_CAPACITY;
  }
  int64_t need = 0, copies = 0;
  for (int i = 0; i < num_seqs; ++i) {
    const int s = seqs[i];
    const int L = bm->len[s];
    if (L % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t b = bm->tables[s].back();
      if (bm->ref[b] - bm->scratch_block[b] > 1) {
        ++need;
        ++copies;
        bm->scratch_block[b] += 1;
      }
    }
  }
  for (int i = 0; i < num_seqs; ++i) {             // undo the scratch counts
    const int s = seqs[i];
    if (bm->len[s] % bm->block_size != 0) bm->scratch_block[bm->tables[s].back()] = 0;
  }
  if (need > (int64_t)bm->free_stack.size()) return PA_ERR_NO_BLOCKS;
  try {
    bm->copies.reserve(bm->copies.size() + (size_t)copies);
    for (int i = 0; i < num_seqs; ++i) bm->tables[seqs[i]].reserve(bm->tables[seqs[i]].size() + 1);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < num_seqs; ++i) {             // cannot fail now
    const int s = seqs[i];
    const int rc = pa_bm_append_slots(bm, s, 1, slots ? slots + i : nullptr);
    (void)rc;
  }
  return PA_OK;
}

extern "C" int pa_bm_fork(pa_block_manager* bm, int parent, int child) {
  if (!bm || !bm->live(parent) || !bm->free_id(child)) return PA_ERR_INVALID_ARG;
  try {
    bm->tables[child] = bm->tables[parent];
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t b : bm->tables[child]) bm->ref[b] += 1;
  bm->len[child] = bm->len[parent];
  return PA_OK;
}

extern "C" int pa_bm_free(pa_block_manager* bm, int seq) {
  if (!bm || !bm->live(seq)) return PA_ERR_INVALID_ARG;
  std::vector<int32_t>& t = bm->tables[seq];
  bool released = false;
  for (int32_t b : t) {
    if (--bm->ref[b] == 0) {
      bm->free_stack.push_back(b);                 // capacity num_blocks: never reallocates
      released = true;
    }
  }
  t.clear();
  bm->len[seq] = -1;
  if (released && !bm->copies.empty()) {           // a copy into a block nobody holds is dropped
    size_t k = 0;
    for (const auto& c : bm->copies)
      if (bm->ref[c.second] > 0) bm->copies[k++] = c;
    bm->copies.resize(k);
  }
  return PA_OK;
}

extern "C" int pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? (int)bm->free_stack.size() : PA_ERR_INVALID_ARG;
}

extern "C" int pa_bm_free_list(const pa_block_manager* bm, int32_t* blocks, int capacity) {
  if (!bm || capacity < 0 || (capacity > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  const int n = (int)bm->free_stack.size();
  if (capacity < n) return PA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) blocks[i] = bm->free_stack[i];
  return n;
}

extern "C" int pa_bm_ref_count(const pa_block_manager* bm, int block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID_ARG;
  return bm->ref[block];
}

extern "C" int pa_bm_seq_len(const pa_block_manager* bm, int seq) {
  if (!bm || seq < 0 || seq >= bm->max_seqs) return PA_ERR_INVALID_ARG;
  return bm->len[seq];
}

extern "C" int pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int num_seqs,
                                  int32_t* block_tables, int32_t* seq_lens) {
  if (!bm || num_seqs < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !block_tables || !seq_lens) return PA_ERR_INVALID_ARG;
  for (int i = 0; i < num_seqs; ++i)
    if (!bm->live(seqs[i])) return PA_ERR_INVALID_ARG;
  const int W = bm->max_blocks_per_seq;
  for (int i = 0; i < num_seqs; ++i) {
    const std::vector<int32_t>& t = bm->tables[seqs[i]];
    int32_t* row = block_tables + (int64_t)i * W;
    const int n = (int)t.size();
    for (int j = 0; j < n; ++j) row[j] = t[j];
    for (int j = n; j < W; ++j) row[j] = -1;
    seq_lens[i] = bm->len[seqs[i]];
  }
  return PA_OK;
}

extern "C" int pa_bm_num_copies(const pa_block_manager* bm) {
  return bm ? (int)bm->copies.size() : PA_ERR_INVALID_ARG;
}

extern "C" int pa_bm_take_copies(pa_block_manager* bm, int32_t* src, int32_t* dst, int capacity) {
  if (!bm || capacity < 0) return PA_ERR_INVALID_ARG;
  const int n = (int)bm->copies.size();
  if (n == 0) return 0;
  if (capacity < n || !src || !dst) return PA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    src[i] = bm->copies[i].first;
    dst[i] = bm->copies[i].second;
  }
  bm->copies.clear();
  return n;
}
