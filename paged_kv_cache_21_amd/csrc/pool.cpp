// Host block pool: reference-counted physical blocks, fork, copy-on-write append
// planning, free.
//
// "The Reasoning Engine Meltdown", §5 "Paged Memory Management for Dynamic
// Trees": a fork points the child at the parent's pages and raises their counts;
// writes go to pages the writer owns (copy-on-write); pruning lowers the counts
// and a page at count 0 goes back to the free pool.  §6 fixes the error
// conventions: out-of-memory is reported before anything changes, a fork of an
// unknown parent is an error, freeing an unknown node does nothing.
// "Dismantling the Memory Wall", "PagedAttention ...": token t sits in logical
// block t / block_size, row t % block_size, and only the last block of a
// sequence is partly filled.
//
// The listing on the first page only copies on a capacity overflow and moves no
// data; this pool follows the prose instead: an append whose target block is
// shared and partly filled gets a fresh block holding a copy of the valid rows.
// Order is deterministic: a FIFO free list seeded by the caller, batches
// processed in the order given.
//
// Swap space ("Dismantling the Memory Wall", "Cross-Tier Memory Offloading":
// KV blocks that overflow the GPU move to CPU memory and come back before
// attention): host slots with their own FIFO list.  A swap-out moves the blocks
// a sequence holds alone to host slots and frees them on the device; blocks it
// shares stay on the device with its reference.  A swap-in takes device blocks
// for the host-resident entries.  Both are all-or-nothing and return the block
// copies that pkv_copy_blocks performs.
#include <algorithm>
#include <unordered_set>

#include "host_common.h"
#include "pool.h"

namespace {

int32_t blocks_for(int64_t tokens, int32_t block_size) {
  return static_cast<int32_t>((tokens + block_size - 1) / block_size);
}

}  // namespace

extern "C" {

pkv_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  pkv::clear_error();
  if (num_blocks < 0 || block_size <= 0) {
    pkv::fail(PKV_ERR_INVALID, "pkv_pool_create: num_blocks must be >= 0 and block_size > 0");
    return nullptr;
  }
  auto* p = new pkv_pool();
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        pkv::fail(PKV_ERR_INVALID, "pkv_pool_create: free_order is not a permutation of [0, num_blocks)");
        return nullptr;
      }
      seen[b] = 1;
      p->free_list.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_list.push_back(i);
  }
  return p;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status pkv_seq_alloc(pkv_pool* pool, int64_t seq, int32_t num_tokens) {
  pkv::clear_error();
  if (!pool) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc: null pool");
  if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc: num_tokens < 0");
  if (pool->seqs.count(seq)) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc: sequence %lld exists", (long long)seq);
  const int32_t need = blocks_for(num_tokens, pool->block_size);
  if (need > static_cast<int64_t>(pool->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "pkv_seq_alloc: requested %d blocks, only %zu free", need, pool->free_list.size());
  pkv_pool::Seq s;
  s.table.reserve(need);
  for (int32_t i = 0; i < need; ++i) {
    int32_t b = pool->free_list.front();
    pool->free_list.pop_front();
    pool->ref[b] = 1;
    s.table.push_back(b);
  }
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_alloc_prefix(pkv_pool* pool, int64_t seq, const int32_t* prefix_blocks, int32_t num_prefix_blocks,
                                int32_t num_tokens) {
  pkv::clear_error();
  if (!pool) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc_prefix: null pool");
  if (num_prefix_blocks < 0 || (num_prefix_blocks > 0 && !prefix_blocks))
    return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc_prefix: bad prefix");
  if (num_tokens < 0 || static_cast<int64_t>(num_prefix_blocks) * pool->block_size > num_tokens)
    return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc_prefix: num_tokens must cover the prefix blocks");
  if (pool->seqs.count(seq))
    return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc_prefix: sequence %lld exists", (long long)seq);
  for (int32_t i = 0; i < num_prefix_blocks; ++i) {
    const int32_t b = prefix_blocks[i];
    if (b < 0 || b >= pool->num_blocks || pool->ref[b] == 0)
      return pkv::fail(PKV_ERR_INVALID, "pkv_seq_alloc_prefix: prefix block %d is not allocated", b);
  }
  const int32_t need = blocks_for(num_tokens, pool->block_size) - num_prefix_blocks;
  if (need > static_cast<int64_t>(pool->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "pkv_seq_alloc_prefix: requested %d blocks, only %zu free", need,
                     pool->free_list.size());
  pkv_pool::Seq s;
  s.table.reserve(num_prefix_blocks + need);
  for (int32_t i = 0; i < num_prefix_blocks; ++i) {
    pool->ref[prefix_blocks[i]] += 1;
    s.table.push_back(prefix_blocks[i]);
  }
  for (int32_t i = 0; i < need; ++i) {
    const int32_t b = pool->free_list.front();
    pool->free_list.pop_front();
    pool->ref[b] = 1;
    s.table.push_back(b);
  }
  s.len = num_tokens;
  pool->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child) {
  pkv::clear_error();
  if (!pool) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_fork: null pool");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_seq_fork: parent %lld does not exist", (long long)parent);
  if (it->second.swapped) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_fork: parent %lld is swapped out", (long long)parent);
  if (pool->seqs.count(child)) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_fork: sequence %lld exists", (long long)child);
  pkv_pool::Seq s = it->second;  // copy of the table, partly filled tail included
  for (int32_t b : s.table) pool->ref[b] += 1;
  pool->seqs.emplace(child, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq) {
  pkv::clear_error();
  if (!pool) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_free: null pool");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return PKV_OK;  // unknown id: nothing to do
  const auto& s = it->second;
  for (size_t i = 0; i < s.table.size(); ++i) {
    const int32_t b = s.table[i];
    if (s.swapped && s.on_host[i])
      pool->host_free.push_back(b);
    else if (--pool->ref[b] == 0)
      pool->free_list.push_back(b);
  }
  pool->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_plan_append(pkv_pool* pool, const int64_t* seqs, int32_t n, int64_t* slot_out, int32_t* cow_src,
                           int32_t* cow_dst, int32_t* cow_rows, int32_t* num_cow, int32_t* row_cow_src) {
  pkv::clear_error();
  if (!pool || n < 0 || (n > 0 && (!seqs || !slot_out || !cow_src || !cow_dst || !cow_rows)) || !num_cow)
    return pkv::fail(PKV_ERR_INVALID, "pkv_plan_append: null argument or n < 0");
  const int32_t bs = pool->block_size;
  std::vector<pkv_pool::Seq*> ss(n);
  {
    std::unordered_set<int64_t> seen;
    seen.reserve(n * 2 + 1);
    for (int32_t i = 0; i < n; ++i) {
      auto it = pool->seqs.find(seqs[i]);
      if (it == pool->seqs.end())
        return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_plan_append: sequence %lld does not exist", (long long)seqs[i]);
      if (!seen.insert(seqs[i]).second)
        return pkv::fail(PKV_ERR_INVALID, "pkv_plan_append: sequence %lld appears twice", (long long)seqs[i]);
      if (it->second.swapped)
        return pkv::fail(PKV_ERR_INVALID, "pkv_plan_append: sequence %lld is swapped out", (long long)seqs[i]);
      if (it->second.len == INT32_MAX) return pkv::fail(PKV_ERR_INVALID, "pkv_plan_append: sequence too long");
      ss[i] = &it->second;
    }
  }
  // Capacity for the whole batch before touching anything.
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> dropped;  // count reductions earlier copies in this batch make
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = ss[i]->len, j = pos / bs, off = pos % bs;
    if (off == 0) {
      ++need;
    } else {
      const int32_t x = ss[i]->table[j];
      int32_t& d = dropped[x];
      if (pool->ref[x] + d > 1) {
        ++need;
        --d;
      }
    }
  }
  if (need > static_cast<int64_t>(pool->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "pkv_plan_append: batch needs %lld blocks, only %zu free", (long long)need,
                     pool->free_list.size());
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto& s = *ss[i];
    const int32_t pos = s.len, j = pos / bs, off = pos % bs;
    if (row_cow_src) row_cow_src[i] = -1;
    if (off == 0) {
      const int32_t y = pool->free_list.front();
      pool->free_list.pop_front();
      pool->ref[y] = 1;
      s.table.push_back(y);
    } else {
      const int32_t x = s.table[j];
      if (pool->ref[x] > 1) {
        const int32_t y = pool->free_list.front();
        pool->free_list.pop_front();
        pool->ref[y] = 1;
        if (row_cow_src) row_cow_src[i] = x;
        cow_src[nc] = x;
        cow_dst[nc] = y;
        cow_rows[nc] = off;
        ++nc;
        pool->ref[x] -= 1;
        s.table[j] = y;
      }
    }
    slot_out[i] = static_cast<int64_t>(s.table[j]) * bs + off;
    s.len = pos + 1;
  }
  *num_cow = nc;
  return PKV_OK;
}

pkv_status pkv_export_tables(const pkv_pool* pool, const int64_t* seqs, int32_t n, int32_t max_blocks,
                             int32_t* tables_out, int32_t* lens_out) {
  pkv::clear_error();
  if (!pool || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables_out || !lens_out)))
    return pkv::fail(PKV_ERR_INVALID, "pkv_export_tables: null argument or negative size");
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_export_tables: sequence %lld does not exist", (long long)seqs[i]);
    if (it->second.swapped)
      return pkv::fail(PKV_ERR_INVALID, "pkv_export_tables: sequence %lld is swapped out", (long long)seqs[i]);
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return pkv::fail(PKV_ERR_INVALID, "pkv_export_tables: sequence %lld has %zu blocks > max_blocks %d",
                       (long long)seqs[i], it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = pool->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    lens_out[i] = s.len;
  }
  return PKV_OK;
}

int32_t pkv_seq_table(const pkv_pool* pool, int64_t seq, int32_t* out, int32_t cap) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return -1;
  if (it->second.swapped) return -2;
  const auto& t = it->second.table;
  if (out)
    for (int32_t i = 0; i < cap && i < static_cast<int32_t>(t.size()); ++i) out[i] = t[i];
  return static_cast<int32_t>(t.size());
}

int32_t pkv_seq_len(const pkv_pool* pool, int64_t seq) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq);
  return it == pool->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->ref[block];
}

int32_t pkv_free_count(const pkv_pool* pool) { return pool ? static_cast<int32_t>(pool->free_list.size()) : -1; }

int32_t pkv_num_seqs(const pkv_pool* pool) { return pool ? static_cast<int32_t>(pool->seqs.size()) : -1; }

int32_t pkv_free_list(const pkv_pool* pool, int32_t* out, int32_t cap) {
  if (!pool) return -1;
  int32_t i = 0;
  if (out)
    for (auto it = pool->free_list.begin(); it != pool->free_list.end() && i < cap; ++it) out[i++] = *it;
  return static_cast<int32_t>(pool->free_list.size());
}

pkv_status pkv_pool_set_host_slots(pkv_pool* pool, int32_t num_host_slots, const int32_t* host_order) {
  pkv::clear_error();
  if (!pool || num_host_slots < 0) return pkv::fail(PKV_ERR_INVALID, "pkv_pool_set_host_slots: bad arguments");
  if (pool->num_host_slots != 0) return pkv::fail(PKV_ERR_INVALID, "pkv_pool_set_host_slots: already set");
  std::deque<int32_t> order;
  if (host_order) {
    std::vector<char> seen(num_host_slots, 0);
    for (int32_t i = 0; i < num_host_slots; ++i) {
      const int32_t h = host_order[i];
      if (h < 0 || h >= num_host_slots || seen[h])
        return pkv::fail(PKV_ERR_INVALID, "pkv_pool_set_host_slots: host_order is not a permutation");
      seen[h] = 1;
      order.push_back(h);
    }
  } else {
    for (int32_t i = 0; i < num_host_slots; ++i) order.push_back(i);
  }
  pool->num_host_slots = num_host_slots;
  pool->host_free = std::move(order);
  return PKV_OK;
}

pkv_status pkv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* device_blocks_out, int32_t* host_slots_out,
                            int32_t capacity, int32_t* num_copies) {
  pkv::clear_error();
  if (!pool || !num_copies || capacity < 0 || (capacity > 0 && (!device_blocks_out || !host_slots_out)))
    return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_out: null argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_seq_swap_out: sequence %lld does not exist", (long long)seq);
  auto& s = it->second;
  if (s.swapped) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_out: sequence %lld is swapped out", (long long)seq);
  int32_t alone = 0;
  for (int32_t b : s.table) alone += pool->ref[b] == 1;
  if (alone > capacity) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_out: capacity %d < %d copies", capacity, alone);
  if (alone > static_cast<int64_t>(pool->host_free.size()))
    return pkv::fail(PKV_ERR_OOM, "pkv_seq_swap_out: %d host slots needed, %zu free", alone, pool->host_free.size());
  s.on_host.assign(s.table.size(), 0);
  int32_t n = 0;
  for (size_t i = 0; i < s.table.size(); ++i) {
    const int32_t b = s.table[i];
    if (pool->ref[b] != 1) continue;
    const int32_t h = pool->host_free.front();
    pool->host_free.pop_front();
    device_blocks_out[n] = b;
    host_slots_out[n] = h;
    ++n;
    pool->ref[b] = 0;
    pool->free_list.push_back(b);
    s.table[i] = h;
    s.on_host[i] = 1;
  }
  s.swapped = true;
  *num_copies = n;
  return PKV_OK;
}

pkv_status pkv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* host_slots_out, int32_t* device_blocks_out,
                           int32_t capacity, int32_t* num_copies) {
  pkv::clear_error();
  if (!pool || !num_copies || capacity < 0 || (capacity > 0 && (!device_blocks_out || !host_slots_out)))
    return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_in: null argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end())
    return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_seq_swap_in: sequence %lld does not exist", (long long)seq);
  auto& s = it->second;
  if (!s.swapped) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_in: sequence %lld is not swapped out", (long long)seq);
  int32_t need = 0;
  for (uint8_t h : s.on_host) need += h;
  if (need > capacity) return pkv::fail(PKV_ERR_INVALID, "pkv_seq_swap_in: capacity %d < %d copies", capacity, need);
  if (need > static_cast<int64_t>(pool->free_list.size()))
    return pkv::fail(PKV_ERR_OOM, "pkv_seq_swap_in: %d device blocks needed, %zu free", need, pool->free_list.size());
  int32_t n = 0;
  for (size_t i = 0; i < s.table.size(); ++i) {
    if (!s.on_host[i]) continue;
    const int32_t y = pool->free_list.front();
    pool->free_list.pop_front();
    pool->ref[y] = 1;
    host_slots_out[n] = s.table[i];
    device_blocks_out[n] = y;
    ++n;
    pool->host_free.push_back(s.table[i]);
    s.table[i] = y;
  }
  s.on_host.clear();
  s.swapped = false;
  *num_copies = n;
  return PKV_OK;
}

int32_t pkv_seq_is_swapped(const pkv_pool* pool, int64_t seq) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq);
  return it == pool->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int32_t pkv_seq_placement(const pkv_pool* pool, int64_t seq, int32_t* ids_out, int8_t* on_host_out, int32_t cap) {
  if (!pool) return -1;
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return -1;
  const auto& s = it->second;
  for (int32_t i = 0; i < cap && i < static_cast<int32_t>(s.table.size()); ++i) {
    if (ids_out) ids_out[i] = s.table[i];
    if (on_host_out) on_host_out[i] = s.swapped ? static_cast<int8_t>(s.on_host[i]) : 0;
  }
  return static_cast<int32_t>(s.table.size());
}

int32_t pkv_host_free_count(const pkv_pool* pool) { return pool ? static_cast<int32_t>(pool->host_free.size()) : -1; }

int32_t pkv_host_free_list(const pkv_pool* pool, int32_t* out, int32_t cap) {
  if (!pool) return -1;
  int32_t i = 0;
  if (out)
    for (auto it = pool->host_free.begin(); it != pool->host_free.end() && i < cap; ++it) out[i++] = *it;
  return static_cast<int32_t>(pool->host_free.size());
}

}  // extern "C"
