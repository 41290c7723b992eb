// Host-side block allocator: a free list of equal-sized physical blocks with
// reference counts, copy-on-write and per-sequence logical block tables.
//
// Page keys:
//   [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com)
//   [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn)
//
// [P3] section 二 describes the BlockManager (a free list, because every block
// has the same size there is nothing to split or coalesce; reference counts so
// that copy-on-write can share blocks) and the per-sequence BlockTable (logical
// block number -> physical block number, plus a token count).  [P1]
// "vLLM调度器与PagedAttention协同工作" adds on-demand allocation (a block is
// taken when a new token needs one) and prefix sharing by reference counts.
//
// Readings of the page's listing, whose operators were lost in extraction:
// allocation pops from the end of the free list (initially 0..N-1) and is all
// or nothing; a freed block is pushed back on the end (reused first); a
// reference dropped below zero is a double free, here detected before any
// count changes; copy-on-write keeps a sole owner's block and gives a writer of
// a shared block a fresh one.  The page has no method that adds a reference:
// pkv_incref and pkv_seq_fork provide it.
#include <algorithm>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Sequence {
  std::vector<int32_t> blocks;  // logical block -> physical block (host block when swapped)
  int64_t tokens = 0;
  bool swapped = false;         // blocks live in the host pool
};

}  // namespace

struct pkv_allocator {
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_list;  // the next block to leave is at the back
  std::vector<int32_t> refs;
  std::unordered_map<int32_t, Sequence> seqs;
  int32_t next_seq = 0;
  int64_t cow_copies = 0;
  // Host (swap) pool: blocks of the same size in pinned host memory.  A
  // swapped-out sequence owns its host blocks alone, so they need no counts.
  int num_host_blocks = 0;
  std::vector<int32_t> host_free;  // the next block to leave is at the back

  bool valid_id(int32_t id) const { return id >= 0 && id < num_blocks; }

  // Takes one block off the free list (caller checked it is not empty).
  int32_t pop_block() {
    int32_t b = free_list.back();
    free_list.pop_back();
    refs[b] = 1;
    return b;
  }

  void drop_ref(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
};

namespace {

int check_alloc(const pkv_allocator* a) {
  if (!a) return pkv::fail(PKV_ERR_INVALID_ARG, "allocator is NULL");
  return PKV_OK;
}

int find_seq(const pkv_allocator* a, int32_t seq, const Sequence** out) {
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  *out = &it->second;
  return PKV_OK;
}

// A sequence whose blocks are on the device (not swapped out).
int find_resident(const pkv_allocator* a, int32_t seq, const Sequence** out) {
  if (int rc = find_seq(a, seq, out)) return rc;
  if ((*out)->swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is swapped out", seq);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_allocator_create(int num_blocks, int block_size, pkv_allocator** out) {
  PKV_API_BEGIN
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_blocks (%d) and block_size (%d) must be positive",
                     num_blocks, block_size);
  // Slots (block * block_size + offset) are int32 in the slot mapping.
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_blocks * block_size (%lld) exceeds the int32 slot "
                     "range", static_cast<long long>(num_blocks) * block_size);
  auto* a = new pkv_allocator();
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->free_list.resize(num_blocks);
  for (int i = 0; i < num_blocks; ++i) a->free_list[i] = i;
  a->refs.assign(num_blocks, 0);
  *out = a;
  return PKV_OK;
  PKV_API_END
}

int pkv_allocator_destroy(pkv_allocator* a) {
  PKV_API_BEGIN
  delete a;
  return PKV_OK;
  PKV_API_END
}

int pkv_allocator_set_free_order(pkv_allocator* a, const int32_t* order, int n) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!order || n != a->num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "order must hold num_blocks (%d) ids", a->num_blocks);
  if (static_cast<int>(a->free_list.size()) != a->num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "set_free_order needs every block free");
  std::vector<char> seen(a->num_blocks, 0);
  for (int i = 0; i < n; ++i) {
    if (!a->valid_id(order[i]) || seen[order[i]])
      return pkv::fail(PKV_ERR_INVALID_ARG, "order is not a permutation (entry %d = %d)", i, order[i]);
    seen[order[i]] = 1;
  }
  a->free_list.assign(order, order + n);
  return PKV_OK;
  PKV_API_END
}

int pkv_allocate(pkv_allocator* a, int n, int32_t* out_ids) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (n < 0 || (n > 0 && !out_ids)) return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or NULL output");
  if (static_cast<size_t>(n) > a->free_list.size())
    return pkv::fail(PKV_ERR_OOM, "need %d blocks, %zu free", n, a->free_list.size());
  for (int i = 0; i < n; ++i) out_ids[i] = a->pop_block();
  return PKV_OK;
  PKV_API_END
}

int pkv_free(pkv_allocator* a, const int32_t* ids, int n) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (n < 0 || (n > 0 && !ids)) return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or NULL ids");
  // Validate the whole list (with multiplicity) before touching any count.
  std::unordered_map<int32_t, int> drops;
  for (int i = 0; i < n; ++i) {
    if (!a->valid_id(ids[i])) return pkv::fail(PKV_ERR_INVALID_ARG, "block id %d out of range", ids[i]);
    ++drops[ids[i]];
  }
  for (const auto& kv : drops)
    if (a->refs[kv.first] < kv.second)
      return pkv::fail(PKV_ERR_DOUBLE_FREE, "block %d freed more often than referenced", kv.first);
  for (int i = 0; i < n; ++i) a->drop_ref(ids[i]);
  return PKV_OK;
  PKV_API_END
}

int pkv_incref(pkv_allocator* a, const int32_t* ids, int n) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (n < 0 || (n > 0 && !ids)) return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or NULL ids");
  for (int i = 0; i < n; ++i) {
    if (!a->valid_id(ids[i])) return pkv::fail(PKV_ERR_INVALID_ARG, "block id %d out of range", ids[i]);
    if (a->refs[ids[i]] == 0) return pkv::fail(PKV_ERR_INVALID_ARG, "block %d is not allocated", ids[i]);
  }
  for (int i = 0; i < n; ++i) ++a->refs[ids[i]];
  return PKV_OK;
  PKV_API_END
}

int pkv_copy_on_write(pkv_allocator* a, int32_t id, int32_t* new_id, int* copied) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!new_id || !copied) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  if (!a->valid_id(id)) return pkv::fail(PKV_ERR_INVALID_ARG, "block id %d out of range", id);
  if (a->refs[id] == 0) return pkv::fail(PKV_ERR_INVALID_ARG, "block %d is not allocated", id);
  if (a->refs[id] == 1) {
    *new_id = id;
    *copied = 0;
    return PKV_OK;
  }
  if (a->free_list.empty()) return pkv::fail(PKV_ERR_OOM, "no free block for copy-on-write");
  *new_id = a->pop_block();
  --a->refs[id];  // still > 0: it was shared
  ++a->cow_copies;
  *copied = 1;
  return PKV_OK;
  PKV_API_END
}

int pkv_ref_count(const pkv_allocator* a, int32_t id, int* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  if (!a->valid_id(id)) return pkv::fail(PKV_ERR_INVALID_ARG, "block id %d out of range", id);
  *out = a->refs[id];
  return PKV_OK;
  PKV_API_END
}

int pkv_num_free(const pkv_allocator* a, int* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  *out = static_cast<int>(a->free_list.size());
  return PKV_OK;
  PKV_API_END
}

int pkv_usage_ratio(const pkv_allocator* a, double* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  *out = 1.0 - static_cast<double>(a->free_list.size()) / a->num_blocks;
  return PKV_OK;
  PKV_API_END
}

int pkv_free_list(const pkv_allocator* a, int32_t* out, int cap, int* n) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!n || (cap > 0 && !out)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  *n = static_cast<int>(a->free_list.size());
  if (cap < *n) return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d free blocks", cap, *n);
  std::copy(a->free_list.begin(), a->free_list.end(), out);
  return PKV_OK;
  PKV_API_END
}

int pkv_cow_count(const pkv_allocator* a, int64_t* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  *out = a->cow_copies;
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_create(pkv_allocator* a, int32_t* seq) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!seq) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  if (a->next_seq == INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence ids exhausted");
  *seq = a->next_seq++;
  a->seqs.emplace(*seq, Sequence());
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_fork(pkv_allocator* a, int32_t seq, int32_t* child) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!child) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  const Sequence* parent;
  if (int rc = find_resident(a, seq, &parent)) return rc;
  if (a->next_seq == INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence ids exhausted");
  Sequence copy = *parent;
  for (int32_t b : copy.blocks)
    if (b >= 0) ++a->refs[b];
  *child = a->next_seq++;
  a->seqs.emplace(*child, std::move(copy));
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_append_tokens(pkv_allocator* a, int32_t seq, int n, int32_t* slots_out,
                          int32_t* cow_pairs_out, int cow_cap, int* n_cow) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (n < 0 || (n > 0 && !slots_out)) return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or NULL slots");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  if (it->second.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is swapped out", seq);
  Sequence& s = it->second;
  const int64_t bs = a->block_size;
  if (s.tokens + n > static_cast<int64_t>(INT32_MAX) / 2)
    return pkv::fail(PKV_ERR_INVALID_ARG, "sequence too long");
  // Blocks this call needs: one copy if the partly filled last block is
  // shared and gets written, plus one per logical block boundary crossed.
  int64_t need = 0;
  const bool cow_first = n > 0 && s.tokens % bs != 0 && a->refs[s.blocks.back()] > 1;
  if (cow_first) ++need;
  need += (s.tokens + n + bs - 1) / bs - (s.tokens + bs - 1) / bs;
  if (need > static_cast<int64_t>(a->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "need %lld blocks, %zu free", static_cast<long long>(need),
                     a->free_list.size());
  if (cow_first && (cow_cap < 1 || !cow_pairs_out))
    return pkv::fail(PKV_ERR_INVALID_ARG, "a copy-on-write pair is needed but cow_cap < 1");
  int ncow = 0;
  for (int t = 0; t < n; ++t) {
    const int64_t off = s.tokens % bs;
    if (off == 0) {
      s.blocks.push_back(a->pop_block());
    } else if (a->refs[s.blocks.back()] > 1) {
      const int32_t old = s.blocks.back();
      const int32_t fresh = a->pop_block();
      --a->refs[old];
      ++a->cow_copies;
      s.blocks.back() = fresh;
      cow_pairs_out[2 * ncow] = old;
      cow_pairs_out[2 * ncow + 1] = fresh;
      ++ncow;
    }
    slots_out[t] = static_cast<int32_t>(s.blocks.back() * bs + off);
    ++s.tokens;
  }
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_trim_window(pkv_allocator* a, int32_t seq, int window, int32_t* released, int cap,
                        int* n_released) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (window <= 0 || !n_released || (cap > 0 && !released))
    return pkv::fail(PKV_ERR_INVALID_ARG, "window must be positive and n_released given");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  if (it->second.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is swapped out", seq);
  Sequence& s = it->second;
  // Blocks before the one holding token max(0, tokens - window) hold no token
  // of the window.
  const int64_t first_kept = std::max<int64_t>(0, s.tokens - window) / a->block_size;
  int count = 0;
  for (int64_t j = 0; j < first_kept; ++j) count += s.blocks[j] >= 0;
  *n_released = count;
  if (released && cap < count)
    return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d released blocks", cap, count);
  int k = 0;
  for (int64_t j = 0; j < first_kept; ++j) {
    const int32_t b = s.blocks[j];
    if (b < 0) continue;
    if (released) released[k] = b;
    ++k;
    a->drop_ref(b);
    s.blocks[j] = -1;
  }
  return PKV_OK;
  PKV_API_END
}

int pkv_allocator_set_host_pool(pkv_allocator* a, int num_host_blocks) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (num_host_blocks < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_host_blocks %d is negative", num_host_blocks);
  for (const auto& kv : a->seqs)
    if (kv.second.swapped)
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is swapped out", kv.first);
  a->num_host_blocks = num_host_blocks;
  a->host_free.resize(num_host_blocks);
  for (int i = 0; i < num_host_blocks; ++i) a->host_free[i] = i;
  return PKV_OK;
  PKV_API_END
}

int pkv_host_num_free(const pkv_allocator* a, int* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  *out = static_cast<int>(a->host_free.size());
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_swap_out(pkv_allocator* a, int32_t seq, int32_t* pairs, int cap, int* n_pairs) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!n_pairs || (cap > 0 && !pairs)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  Sequence& s = it->second;
  if (s.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is swapped out", seq);
  int need = 0;
  for (int32_t b : s.blocks) need += b >= 0;
  *n_pairs = need;
  if (need > static_cast<int>(a->host_free.size()))
    return pkv::fail(PKV_ERR_OOM, "need %d host blocks, %zu free", need, a->host_free.size());
  if (cap < need) return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d pairs", cap, need);
  int k = 0;
  for (int32_t& b : s.blocks) {
    if (b < 0) continue;
    const int32_t h = a->host_free.back();
    a->host_free.pop_back();
    pairs[2 * k] = b;
    pairs[2 * k + 1] = h;
    ++k;
    a->drop_ref(b);  // a block shared with other sequences stays theirs
    b = h;
  }
  s.swapped = true;
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_swap_in(pkv_allocator* a, int32_t seq, int32_t* pairs, int cap, int* n_pairs) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!n_pairs || (cap > 0 && !pairs)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  Sequence& s = it->second;
  if (!s.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d is not swapped out", seq);
  int need = 0;
  for (int32_t h : s.blocks) need += h >= 0;
  *n_pairs = need;
  if (need > static_cast<int>(a->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "need %d device blocks, %zu free", need, a->free_list.size());
  if (cap < need) return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d pairs", cap, need);
  int k = 0;
  for (int32_t& h : s.blocks) {
    if (h < 0) continue;
    const int32_t d = a->pop_block();
    pairs[2 * k] = h;
    pairs[2 * k + 1] = d;
    ++k;
    a->host_free.push_back(h);
    h = d;
  }
  s.swapped = false;
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_is_swapped(const pkv_allocator* a, int32_t seq, int* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  const Sequence* s;
  if (int rc = find_seq(a, seq, &s)) return rc;
  *out = s->swapped ? 1 : 0;
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_free(pkv_allocator* a, int32_t seq) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "no sequence %d", seq);
  for (int32_t b : it->second.blocks) {
    if (b < 0) continue;
    if (it->second.swapped)
      a->host_free.push_back(b);
    else
      a->drop_ref(b);
  }
  a->seqs.erase(it);
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_num_tokens(const pkv_allocator* a, int32_t seq, int* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  const Sequence* s;
  if (int rc = find_seq(a, seq, &s)) return rc;
  *out = static_cast<int>(s->tokens);
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_block_ids(const pkv_allocator* a, int32_t seq, int32_t* out, int cap, int* n) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!n || (cap > 0 && !out)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  const Sequence* s;
  if (int rc = find_seq(a, seq, &s)) return rc;
  *n = static_cast<int>(s->blocks.size());
  if (cap < *n) return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d blocks", cap, *n);
  std::copy(s->blocks.begin(), s->blocks.end(), out);
  return PKV_OK;
  PKV_API_END
}

int pkv_seq_physical_block(const pkv_allocator* a, int32_t seq, int token, int32_t* out) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL output");
  const Sequence* s;
  if (int rc = find_resident(a, seq, &s)) return rc;
  const int64_t idx = token / a->block_size;
  if (token < 0 || idx >= static_cast<int64_t>(s->blocks.size()) || s->blocks[idx] < 0)
    return pkv::fail(PKV_ERR_INDEX, "token %d: logical block %lld is not allocated", token,
                     static_cast<long long>(idx));
  *out = s->blocks[idx];
  return PKV_OK;
  PKV_API_END
}

int pkv_export_block_tables(const pkv_allocator* a, const int32_t* seqs, int n, int max_blocks,
                            int32_t pad, int32_t* out_tables, int32_t* out_lens) {
  PKV_API_BEGIN
  if (int rc = check_alloc(a)) return rc;
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !out_tables || !out_lens)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad count or NULL buffer");
  for (int i = 0; i < n; ++i) {
    const Sequence* s;
    if (int rc = find_resident(a, seqs[i], &s)) return rc;
    if (static_cast<int64_t>(s->blocks.size()) > max_blocks)
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d holds %zu blocks > max_blocks %d", seqs[i],
                       s->blocks.size(), max_blocks);
  }
  for (int i = 0; i < n; ++i) {
    const Sequence& s = a->seqs.find(seqs[i])->second;
    int32_t* row = out_tables + static_cast<int64_t>(i) * max_blocks;
    for (size_t j = 0; j < s.blocks.size(); ++j) row[j] = s.blocks[j] >= 0 ? s.blocks[j] : pad;
    std::fill(row + s.blocks.size(), row + max_blocks, pad);
    out_lens[i] = static_cast<int32_t>(s.tokens);
  }
  return PKV_OK;
  PKV_API_END
}

int pkv_validate_tables(const int32_t* tables, const int32_t* lens, int num_seqs, int max_blocks,
                        int block_size, int num_blocks, int sliding_window, int* bad_seq,
                        int* bad_block) {
  PKV_API_BEGIN
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0 || num_blocks < 0 || sliding_window < 0 ||
      (num_seqs > 0 && (!tables || !lens)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad shape or NULL buffer");
  if (bad_seq) *bad_seq = -1;
  if (bad_block) *bad_block = -1;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = lens[s];
    if (n < 0 || n > static_cast<int64_t>(max_blocks) * block_size) {
      if (bad_seq) *bad_seq = s;
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d: length %lld outside [0, %lld]", s,
                       static_cast<long long>(n), static_cast<long long>(max_blocks) * block_size);
    }
    const int64_t nb = (n + block_size - 1) / block_size;
    const int64_t first = sliding_window > 0 ? std::max<int64_t>(0, n - sliding_window) : 0;
    for (int64_t j = first / block_size; j < nb; ++j) {
      const int32_t b = tables[static_cast<int64_t>(s) * max_blocks + j];
      if (b < 0 || b >= num_blocks) {
        if (bad_seq) *bad_seq = s;
        if (bad_block) *bad_block = static_cast<int>(j);
        return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %d: block %lld = %d outside [0, %d)", s,
                         static_cast<long long>(j), b, num_blocks);
      }
    }
  }
  return PKV_OK;
  PKV_API_END
}

int pkv_find_shared_prefixes(const int32_t* tables, const int32_t* lens, int num_seqs,
                             int max_blocks, int block_size, int min_tokens, int min_group,
                             int32_t* groups_out, int cap, int* n_groups) {
  PKV_API_BEGIN
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0 || min_group < 1 || !n_groups ||
      (num_seqs > 0 && (!tables || !lens)) || (cap > 0 && !groups_out))
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad shape or NULL buffer");
  const int64_t unit = block_size > 16 ? block_size : 16;  // shared tokens are multiples of this
  const int64_t min_tok = std::max<int64_t>(min_tokens, unit);
  // Whole blocks of sequence s that its context covers and that hold a valid id.
  auto covered = [&](int s) {
    const int64_t n = std::min<int64_t>(std::max(lens[s], 0), static_cast<int64_t>(max_blocks) * block_size);
    return n / block_size;
  };
  auto entry = [&](int s, int64_t j) { return tables[static_cast<int64_t>(s) * max_blocks + j]; };
  int found = 0;
  int i = 0;
  while (i < num_seqs && found < 32) {
    int64_t common = covered(i);
    int64_t k = 0;
    while (k < common && entry(i, k) >= 0) ++k;
    common = k;
    int j = i + 1;
    for (; j < num_seqs; ++j) {
      int64_t c = std::min(common, covered(j));
      int64_t m = 0;
      while (m < c && entry(j, m) == entry(i, m)) ++m;
      if (m * block_size / unit * unit < min_tok) break;
      common = m;
    }
    const int64_t shared = common * block_size / unit * unit;
    if (j - i >= min_group && j - i >= 2 && shared >= min_tok) {
      if (found < cap) {
        groups_out[3 * found] = i;
        groups_out[3 * found + 1] = j - i;
        groups_out[3 * found + 2] = static_cast<int32_t>(shared);
      }
      ++found;
      i = j;
    } else {
      ++i;
    }
  }
  *n_groups = found;
  if (found > cap) return pkv::fail(PKV_ERR_INVALID_ARG, "capacity %d < %d groups", cap, found);
  return PKV_OK;
  PKV_API_END
}

}  // extern "C"
