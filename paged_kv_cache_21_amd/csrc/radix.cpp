// Prefix cache over paged KV blocks: a radix tree of token runs whose values
// are physical block ids held in the block pool, with per-node locks and leaf
// eviction.
//
// "Dismantling the Memory Wall", section "RadixAttention: The Tree of Life for
// Agentic Swarms": a compressed trie keeps the KV of finished requests; a new
// request takes the longest cached prefix and computes only the rest; a node
// carries children, parent, key, value, lock_ref and last_access_time; using a
// node locks it and its ancestors; under memory pressure least recently used
// unlocked leaves go first, so shared prefixes stay; a later turn of a
// conversation extends the leaf of the turn before.
// "RKSC - Reasoning-Aware KV Cache Sharing en Confident Early Exit", §2, C
// "RSBCM": the alternative policy removes the lowest importance
// branch_score / (depth + 1) first.
//
// Choices the pages leave open:
//  * the cache holds whole blocks: keys are compared in runs of block_size
//    tokens, so matches and splits fall on block boundaries and a partly
//    filled block is never cached;
//  * a match that ends inside a node splits it there (the new upper node takes
//    the matched blocks, the old node keeps its id and the rest), so a lock on
//    the returned node covers exactly the matched prefix;
//  * time is a logical clock, one tick per match or insert; ties go to the
//    smaller (older) node id;
//  * an insert keeps the tree's own blocks where the path is cached already,
//    adds the rest as one new leaf and takes one pool reference per adopted
//    block; path nodes take the current time and the larger score, a new leaf
//    takes the given score and depth;
//  * eviction removes whole leaves until the requested number of blocks went
//    back to the free list; removing a leaf drops the tree's reference on each
//    of its blocks in key order.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <tuple>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "host_common.h"
#include "pool.h"

namespace {

// Eviction order: smallest key first (omega is 0 under the LRU policy).
struct EvictKey {
  double omega;
  int64_t last_access;
  int64_t id;
  bool operator<(const EvictKey& o) const {
    return std::tie(omega, last_access, id) < std::tie(o.omega, o.last_access, o.id);
  }
};

struct Node {
  int64_t id = 0;
  Node* parent = nullptr;
  std::vector<int32_t> tokens;  // key: blocks.size() * block_size tokens
  std::vector<int32_t> blocks;  // value: physical block id of each key block
  int32_t lock_ref = 0;
  int64_t last_access = 0;
  double score = 0.0;
  int32_t depth = 0;
  std::unordered_multimap<uint64_t, Node*> children;  // by hash of the child's first key block
  bool queued = false;  // in the eviction order (an unlocked leaf), under `key`
  EvictKey key{};
};

uint64_t hash_block(const int32_t* t, int32_t n) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (int32_t i = 0; i < n; ++i) {
    h ^= static_cast<uint32_t>(t[i]);
    h *= 0x100000001b3ull;
    h ^= h >> 29;
  }
  return h;
}

}  // namespace

struct pkv_radix {
  pkv_pool* pool = nullptr;
  int32_t policy = PKV_EVICT_LRU;
  int32_t bs = 16;
  int64_t clock = 0;
  int64_t next_id = 1;
  std::unordered_map<int64_t, std::unique_ptr<Node>> nodes;
  Node* root = nullptr;
  std::map<EvictKey, Node*> order;  // unlocked leaves, next victim first
  int64_t cached = 0;               // blocks held by the tree

  bool evictable(const Node* n) const { return n != root && n->children.empty() && n->lock_ref == 0; }

  EvictKey key_of(const Node* n) const {
    const double omega = policy == PKV_EVICT_RSBCM ? n->score / static_cast<double>(n->depth + 1) : 0.0;
    return {omega, n->last_access, n->id};
  }

  void dequeue(Node* n) {
    if (n->queued) {
      order.erase(n->key);
      n->queued = false;
    }
  }

  // Call after a change to a node's time, score, lock or children.
  void requeue(Node* n) {
    dequeue(n);
    if (evictable(n)) {
      n->key = key_of(n);
      order.emplace(n->key, n);
      n->queued = true;
    }
  }

  size_t block_bytes() const { return static_cast<size_t>(bs) * sizeof(int32_t); }

  Node* find_child(Node* n, const int32_t* blk) const {
    auto range = n->children.equal_range(hash_block(blk, bs));
    for (auto it = range.first; it != range.second; ++it)
      if (std::memcmp(it->second->tokens.data(), blk, block_bytes()) == 0) return it->second;
    return nullptr;
  }

  void unlink_child(Node* parent, Node* child) {
    auto range = parent->children.equal_range(hash_block(child->tokens.data(), bs));
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == child) {
        parent->children.erase(it);
        return;
      }
  }

  void relink_child(Node* parent, Node* from, Node* to) {
    auto range = parent->children.equal_range(hash_block(from->tokens.data(), bs));
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == from) {
        it->second = to;
        return;
      }
  }

  // Blocks of `n`'s key equal to the query's blocks from `q` (at most `avail`);
  // the first block is known to match.
  int32_t common(const Node* n, const int32_t* q, int32_t avail) const {
    const int32_t nb = static_cast<int32_t>(n->blocks.size());
    int32_t m = 1;
    while (m < nb && m < avail &&
           std::memcmp(n->tokens.data() + static_cast<size_t>(m) * bs, q + static_cast<size_t>(m) * bs,
                       block_bytes()) == 0)
      ++m;
    return m;
  }

  // Split `n` after its first m blocks; returns the new upper node.
  Node* split(Node* n, int32_t m) {
    auto up = std::make_unique<Node>();
    Node* u = up.get();
    u->id = next_id++;
    u->parent = n->parent;
    u->tokens.assign(n->tokens.begin(), n->tokens.begin() + static_cast<size_t>(m) * bs);
    u->blocks.assign(n->blocks.begin(), n->blocks.begin() + m);
    u->lock_ref = n->lock_ref;
    u->last_access = n->last_access;
    u->score = n->score;
    u->depth = n->depth;
    relink_child(n->parent, n, u);
    n->tokens.erase(n->tokens.begin(), n->tokens.begin() + static_cast<size_t>(m) * bs);
    n->blocks.erase(n->blocks.begin(), n->blocks.begin() + m);
    u->children.emplace(hash_block(n->tokens.data(), bs), n);
    n->parent = u;
    nodes.emplace(u->id, std::move(up));
    return u;
  }

  Node* get(int64_t id) const {
    auto it = nodes.find(id);
    return it == nodes.end() ? nullptr : it->second.get();
  }

  void clear() {
    std::vector<int64_t> ids;
    ids.reserve(nodes.size());
    for (auto& kv : nodes)
      if (kv.first != 0) ids.push_back(kv.first);
    std::sort(ids.begin(), ids.end());
    for (int64_t id : ids)
      for (int32_t b : nodes[id]->blocks) pool->release(b);
    for (int64_t id : ids) nodes.erase(id);
    root->children.clear();
    order.clear();
    cached = 0;
  }
};

extern "C" {

pkv_radix* pkv_radix_create(pkv_pool* pool, int32_t policy) {
  pkv::clear_error();
  if (!pool) {
    pkv::fail(PKV_ERR_INVALID, "pkv_radix_create: null pool");
    return nullptr;
  }
  if (policy != PKV_EVICT_LRU && policy != PKV_EVICT_RSBCM) {
    pkv::fail(PKV_ERR_INVALID, "pkv_radix_create: unknown eviction policy %d", policy);
    return nullptr;
  }
  auto* r = new pkv_radix();
  r->pool = pool;
  r->policy = policy;
  r->bs = pool->block_size;
  auto root = std::make_unique<Node>();
  r->root = root.get();
  r->nodes.emplace(0, std::move(root));
  return r;
}

void pkv_radix_destroy(pkv_radix* r) {
  if (!r) return;
  r->clear();
  delete r;
}

pkv_status pkv_radix_clear(pkv_radix* r) {
  pkv::clear_error();
  if (!r) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_clear: null cache");
  r->clear();
  return PKV_OK;
}

pkv_status pkv_radix_match(pkv_radix* r, const int32_t* tokens, int32_t num_tokens, int32_t* matched_tokens,
                           int32_t* blocks_out, int32_t blocks_cap, int64_t* node_out) {
  pkv::clear_error();
  if (!r || num_tokens < 0 || (num_tokens > 0 && !tokens) || !matched_tokens || !node_out)
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_match: null argument or num_tokens < 0");
  const int32_t nb = num_tokens / r->bs;
  if (blocks_out && blocks_cap < nb)
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_match: blocks_cap %d < %d full blocks", blocks_cap, nb);
  r->clock += 1;
  Node* node = r->root;
  int32_t i = 0;
  while (i < nb) {
    const int32_t* q = tokens + static_cast<size_t>(i) * r->bs;
    Node* c = r->find_child(node, q);
    if (!c) break;
    const int32_t m = r->common(c, q, nb - i);
    if (m < static_cast<int32_t>(c->blocks.size())) c = r->split(c, m);
    c->last_access = r->clock;
    r->requeue(c);
    if (blocks_out) std::memcpy(blocks_out + i, c->blocks.data(), sizeof(int32_t) * m);
    i += m;
    node = c;
  }
  *matched_tokens = i * r->bs;
  *node_out = node->id;
  return PKV_OK;
}

pkv_status pkv_radix_insert(pkv_radix* r, const int32_t* tokens, int32_t num_tokens, const int32_t* blocks,
                            int32_t num_blocks, double score, int32_t depth, int64_t* node_out,
                            int32_t* adopted_out) {
  pkv::clear_error();
  if (!r || num_tokens < 0 || (num_tokens > 0 && !tokens) || num_blocks < 0 || (num_blocks > 0 && !blocks))
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_insert: null argument or negative size");
  const int32_t nb = num_tokens / r->bs;
  if (num_blocks < nb)
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_insert: %d block ids for %d full blocks", num_blocks, nb);
  if (depth < 0) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_insert: depth < 0");
  if (!std::isfinite(score)) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_insert: score is not finite");
  for (int32_t k = 0; k < nb; ++k)
    if (blocks[k] < 0 || blocks[k] >= r->pool->num_blocks || r->pool->ref[blocks[k]] == 0)
      return pkv::fail(PKV_ERR_INVALID, "pkv_radix_insert: block %d is not allocated", blocks[k]);
  r->clock += 1;
  Node* node = r->root;
  int32_t i = 0, adopted = 0;
  while (i < nb) {
    const int32_t* q = tokens + static_cast<size_t>(i) * r->bs;
    Node* c = r->find_child(node, q);
    if (c) {
      const int32_t m = r->common(c, q, nb - i);
      if (m < static_cast<int32_t>(c->blocks.size())) c = r->split(c, m);
      c->last_access = r->clock;
      c->score = std::max(c->score, score);
      r->requeue(c);
      node = c;
      i += m;
      continue;
    }
    auto leaf = std::make_unique<Node>();
    Node* l = leaf.get();
    l->id = r->next_id++;
    l->parent = node;
    l->tokens.assign(q, tokens + static_cast<size_t>(nb) * r->bs);
    l->blocks.assign(blocks + i, blocks + nb);
    l->last_access = r->clock;
    l->score = score;
    l->depth = depth;
    for (int32_t b : l->blocks) r->pool->retain(b);
    node->children.emplace(hash_block(q, r->bs), l);
    r->nodes.emplace(l->id, std::move(leaf));
    r->requeue(node);
    r->requeue(l);
    adopted = nb - i;
    r->cached += adopted;
    node = l;
    i = nb;
  }
  if (node_out) *node_out = node->id;
  if (adopted_out) *adopted_out = adopted;
  return PKV_OK;
}

pkv_status pkv_radix_lock(pkv_radix* r, int64_t node) {
  pkv::clear_error();
  if (!r) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_lock: null cache");
  Node* n = r->get(node);
  if (!n) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_lock: node %lld does not exist", (long long)node);
  for (; n != r->root; n = n->parent) {
    n->lock_ref += 1;
    r->requeue(n);
  }
  return PKV_OK;
}

pkv_status pkv_radix_unlock(pkv_radix* r, int64_t node) {
  pkv::clear_error();
  if (!r) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_unlock: null cache");
  Node* n = r->get(node);
  if (!n) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_unlock: node %lld does not exist", (long long)node);
  for (Node* p = n; p != r->root; p = p->parent)
    if (p->lock_ref == 0) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_unlock: node %lld is not locked", (long long)node);
  for (; n != r->root; n = n->parent) {
    n->lock_ref -= 1;
    r->requeue(n);
  }
  return PKV_OK;
}

pkv_status pkv_radix_set_score(pkv_radix* r, int64_t node, double score) {
  pkv::clear_error();
  if (!r) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_set_score: null cache");
  if (!std::isfinite(score)) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_set_score: score is not finite");
  Node* n = r->get(node);
  if (!n) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_set_score: node %lld does not exist", (long long)node);
  if (n == r->root) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_set_score: the root has no score");
  n->score = score;
  r->requeue(n);
  for (Node* p = n->parent; p != r->root; p = p->parent) {
    p->score = std::max(p->score, score);
    r->requeue(p);
  }
  return PKV_OK;
}

pkv_status pkv_radix_evict(pkv_radix* r, int32_t num_blocks, int32_t* released_out, int64_t* evicted_out,
                           int32_t evicted_cap, int32_t* num_evicted_out) {
  pkv::clear_error();
  if (!r || num_blocks < 0 || evicted_cap < 0 || (evicted_cap > 0 && !evicted_out))
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_evict: null argument or negative size");
  int32_t released = 0, evicted = 0;
  while (released < num_blocks && !r->order.empty()) {
    Node* v = r->order.begin()->second;
    r->dequeue(v);
    for (int32_t b : v->blocks)
      if (r->pool->release(b)) ++released;
    Node* parent = v->parent;
    r->unlink_child(parent, v);
    r->cached -= static_cast<int64_t>(v->blocks.size());
    if (evicted < evicted_cap) evicted_out[evicted] = v->id;
    ++evicted;
    r->nodes.erase(v->id);
    r->requeue(parent);
  }
  if (released_out) *released_out = released;
  if (num_evicted_out) *num_evicted_out = evicted;
  return PKV_OK;
}

int32_t pkv_radix_num_nodes(const pkv_radix* r) { return r ? static_cast<int32_t>(r->nodes.size()) : -1; }

int32_t pkv_radix_cached_blocks(const pkv_radix* r) { return r ? static_cast<int32_t>(r->cached) : -1; }

int32_t pkv_radix_evictable_blocks(const pkv_radix* r) {
  if (!r) return -1;
  int64_t n = 0;
  for (auto& kv : r->nodes)
    if (kv.second.get() != r->root && kv.second->lock_ref == 0) n += static_cast<int64_t>(kv.second->blocks.size());
  return static_cast<int32_t>(n);
}

int32_t pkv_radix_node_ids(const pkv_radix* r, int64_t* out, int32_t cap) {
  if (!r) return -1;
  std::vector<int64_t> ids;
  ids.reserve(r->nodes.size());
  for (auto& kv : r->nodes) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  if (out)
    for (int32_t i = 0; i < cap && i < static_cast<int32_t>(ids.size()); ++i) out[i] = ids[i];
  return static_cast<int32_t>(ids.size());
}

pkv_status pkv_radix_node_info(const pkv_radix* r, int64_t node, int64_t* parent, int32_t* lock_ref,
                               int64_t* last_access, double* score, int32_t* depth, int32_t* num_blocks,
                               int32_t* blocks_out, int32_t blocks_cap, int32_t* tokens_out, int32_t tokens_cap) {
  pkv::clear_error();
  if (!r) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_node_info: null cache");
  const Node* n = r->get(node);
  if (!n) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_node_info: node %lld does not exist", (long long)node);
  const int32_t nb = static_cast<int32_t>(n->blocks.size());
  if ((blocks_out && blocks_cap < nb) || (tokens_out && tokens_cap < nb * r->bs))
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_node_info: output too small for %d blocks", nb);
  if (parent) *parent = n->parent ? n->parent->id : -1;
  if (lock_ref) *lock_ref = n->lock_ref;
  if (last_access) *last_access = n->last_access;
  if (score) *score = n->score;
  if (depth) *depth = n->depth;
  if (num_blocks) *num_blocks = nb;
  if (blocks_out && nb) std::memcpy(blocks_out, n->blocks.data(), sizeof(int32_t) * nb);
  if (tokens_out && nb) std::memcpy(tokens_out, n->tokens.data(), sizeof(int32_t) * n->tokens.size());
  return PKV_OK;
}

pkv_status pkv_radix_admit(pkv_radix* r, const int32_t* tokens, const int64_t* offsets, int32_t n,
                           const int64_t* seqs, int32_t* matched_out, int64_t* node_out, int32_t* num_admitted) {
  pkv::clear_error();
  if (!r || n < 0 || (n > 0 && (!tokens || !offsets || !seqs || !matched_out || !node_out)) || !num_admitted)
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_admit: null argument or n < 0");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = offsets[i + 1] - offsets[i];
    if (offsets[i] < 0 || len < 1 || len > INT32_MAX)
      return pkv::fail(PKV_ERR_INVALID, "pkv_radix_admit: request %d has %lld tokens", i, (long long)len);
    if (r->pool->seqs.count(seqs[i]))
      return pkv::fail(PKV_ERR_INVALID, "pkv_radix_admit: sequence %lld exists", (long long)seqs[i]);
  }
  {
    std::unordered_set<int64_t> seen(seqs, seqs + n);
    if (static_cast<int32_t>(seen.size()) != n) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_admit: repeated sequence id");
  }
  thread_local std::vector<int32_t> blocks;
  int32_t done = 0;
  for (; done < n; ++done) {
    const int32_t* t = tokens + offsets[done];
    const int32_t len = static_cast<int32_t>(offsets[done + 1] - offsets[done]);
    blocks.resize(static_cast<size_t>(len / r->bs) + 1);
    int32_t m = 0;
    int64_t node = 0;
    pkv_radix_match(r, t, len - 1, &m, blocks.data(), static_cast<int32_t>(blocks.size()), &node);
    pkv_radix_lock(r, node);
    const int32_t cached = m / r->bs;
    const int32_t need = (len + r->bs - 1) / r->bs - cached;
    const int32_t free_now = static_cast<int32_t>(r->pool->free_list.size());
    if (need > free_now) pkv_radix_evict(r, need - free_now, nullptr, nullptr, 0, nullptr);
    if (pkv_seq_alloc_prefix(r->pool, seqs[done], blocks.data(), cached, len) != PKV_OK) {
      pkv_radix_unlock(r, node);
      break;
    }
    matched_out[done] = m;
    node_out[done] = node;
  }
  pkv::clear_error();
  *num_admitted = done;
  return PKV_OK;
}

pkv_status pkv_radix_finish(pkv_radix* r, const int32_t* tokens, const int64_t* offsets, int32_t n,
                            const int64_t* seqs, const int64_t* nodes, const double* scores, const int32_t* depths) {
  pkv::clear_error();
  if (!r || n < 0 || (n > 0 && (!tokens || !offsets || !seqs || !nodes)))
    return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: null argument or n < 0");
  // Check everything first, so that a bad entry changes nothing.
  std::unordered_map<int64_t, int32_t> unlocks;
  {
    std::unordered_set<int64_t> seen(seqs, seqs + n);
    if (static_cast<int32_t>(seen.size()) != n) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: repeated sequence id");
  }
  for (int32_t i = 0; i < n; ++i) {
    auto it = r->pool->seqs.find(seqs[i]);
    if (it == r->pool->seqs.end())
      return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_finish: sequence %lld does not exist", (long long)seqs[i]);
    if (it->second.swapped)
      return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: sequence %lld is swapped out", (long long)seqs[i]);
    const int64_t len = offsets[i + 1] - offsets[i];
    if (offsets[i] < 0 || len < 0 || len > it->second.len)
      return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: request %d: %lld tokens for a %d-token sequence", i,
                       (long long)len, it->second.len);
    if (scores && !std::isfinite(scores[i])) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: score not finite");
    if (depths && depths[i] < 0) return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: depth < 0");
    Node* nd = r->get(nodes[i]);
    if (!nd) return pkv::fail(PKV_ERR_NOT_FOUND, "pkv_radix_finish: node %lld does not exist", (long long)nodes[i]);
    for (Node* p = nd; p != r->root; p = p->parent)
      if (p->lock_ref < ++unlocks[p->id])
        return pkv::fail(PKV_ERR_INVALID, "pkv_radix_finish: node %lld is not locked", (long long)nodes[i]);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& seq = r->pool->seqs.find(seqs[i])->second;
    const std::vector<int32_t> table = seq.table;
    pkv_radix_insert(r, tokens + offsets[i], static_cast<int32_t>(offsets[i + 1] - offsets[i]), table.data(),
                     static_cast<int32_t>(table.size()), scores ? scores[i] : 0.0, depths ? depths[i] : 0, nullptr,
                     nullptr);
    pkv_radix_unlock(r, nodes[i]);
    pkv_seq_free(r->pool, seqs[i]);
  }
  return PKV_OK;
}

}  // extern "C"
