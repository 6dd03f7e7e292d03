// Cascade planner: find the blocks that several block tables share and lay out
// the shared-prefix work.
//
// "Dismantling the Memory Wall", "RadixAttention": cached prefixes form a tree
// of token runs, and a request that matches a prefix references the cached KV
// instead of holding its own copy.  "The Reasoning Engine Meltdown", §5: a
// forked branch points at its parent's physical pages.  With block tables built
// that way, rows that share a prefix hold the same physical id at the same
// logical index.  The planner walks a trie over (logical index, physical id)
// of the rows' *full* blocks: every maximal run of blocks on which the same set
// of at least `min_members` rows agrees becomes a node; a row's blocks after
// its last node are its own remainder.  Partly filled blocks are never put in
// a node (an append may still write them), so a plan stays valid while rows
// only grow by appends.
#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "host_common.h"
#include "launch.h"
#include "plan.h"

namespace {

struct Group {
  std::vector<int32_t> rows;
  int32_t start;  // first logical block index not yet known to be shared by all rows
};

void build_image(pkv_plan* p) {
  auto& im = p->image;
  im.clear();
  p->off_row_info = im.size();
  im.insert(im.end(), p->row_info.begin(), p->row_info.end());
  p->off_nodes = im.size();
  for (const auto& n : p->nodes) {
    im.push_back(n.block_off);
    im.push_back(n.num_blocks);
    im.push_back(n.member_off);
    im.push_back(n.num_members);
    im.push_back(n.pieces);
    im.push_back(n.piece_blocks);
  }
  p->off_blocks = im.size();
  im.insert(im.end(), p->node_blocks.begin(), p->node_blocks.end());
  p->off_members = im.size();
  im.insert(im.end(), p->node_members.begin(), p->node_members.end());
  p->off_items = im.size();
  im.insert(im.end(), p->items.begin(), p->items.end());
  if (im.empty()) im.push_back(0);
}

// Token pieces.  A node's work is (64-row tiles) x (KV heads) x (blocks); the
// chip wants a few work-groups per CU.  Long nodes are cut into pieces of about
// `target` blocks so the item count lands near kTargetItems, but never below
// kMinPieceBlocks blocks per piece: every piece costs each member row one more
// fp32 partial per query head, written and read back once.
void split_pieces(pkv_plan* p) {
  constexpr int64_t kTargetItems = 1024;
  constexpr int32_t kMinPieceBlocks = 32;
  constexpr int32_t kMaxPieceBlocks = 64;
  const int rows_per_item = pkv::kCascadeRowsPerItem;
  int64_t work = 0;
  for (const auto& n : p->nodes) {
    const int64_t tiles = (static_cast<int64_t>(n.num_members) * p->group + rows_per_item - 1) / rows_per_item;
    work += tiles * p->num_kv_heads * n.num_blocks;
  }
  const int64_t target = std::max<int64_t>(kMinPieceBlocks, (work + kTargetItems - 1) / kTargetItems);
  for (auto& n : p->nodes) {
    // at most kMaxPieceBlocks blocks per piece: the cascade kernel keeps a piece's
    // block ids in one 64-lane register
    n.pieces = static_cast<int32_t>(std::max<int64_t>(
        std::max<int64_t>(1, n.num_blocks / target), (n.num_blocks + kMaxPieceBlocks - 1) / kMaxPieceBlocks));
    n.piece_blocks = (n.num_blocks + n.pieces - 1) / n.pieces;
    n.pieces = (n.num_blocks + n.piece_blocks - 1) / n.piece_blocks;
  }
}

// Partial slots: along each row's path, node pieces take consecutive slots.
// path[b] lists (node, member entry) pairs, root first.
void assign_slots(pkv_plan* p, const std::vector<std::vector<std::pair<int32_t, int32_t>>>& path) {
  p->max_depth = 0;
  for (int32_t b = 0; b < p->batch; ++b) {
    int32_t used = 0;
    for (const auto& [node, entry] : path[b]) {
      p->node_members[2 * entry + 1] = used;
      used += p->nodes[node].pieces;
    }
    p->row_info[2 * b + 1] = used;
    p->max_depth = std::max(p->max_depth, used);
  }
}

// Work items: one per (node, KV head, 64-row tile, piece).  Work-group i runs on
// XCD i % 8, and each XCD has its own L2, so all tiles of one (node, head, piece)
// go to the same XCD queue: the tiles after the first find the piece's K/V in
// that L2.  Clusters are dealt to the least-loaded queue (load = blocks x tiles);
// queues are interleaved into launch order and padded with idle items.
void build_items(pkv_plan* p) {
  constexpr int kXcds = 8;
  const int rows_per_item = pkv::kCascadeRowsPerItem;
  struct Cluster {
    int32_t node, head, tiles, piece;
    int64_t load;
  };
  std::vector<Cluster> clusters;
  for (int32_t n = 0; n < static_cast<int32_t>(p->nodes.size()); ++n) {
    const auto& nd = p->nodes[n];
    const int32_t rows = nd.num_members * p->group;
    const int32_t tiles = (rows + rows_per_item - 1) / rows_per_item;
    for (int32_t pc = 0; pc < nd.pieces; ++pc) {
      const int32_t blocks = std::min(nd.piece_blocks, nd.num_blocks - pc * nd.piece_blocks);
      for (int32_t h = 0; h < p->num_kv_heads; ++h)
        clusters.push_back({n, h, tiles, pc, static_cast<int64_t>(blocks) * tiles});
    }
  }
  std::stable_sort(clusters.begin(), clusters.end(),
                   [](const Cluster& x, const Cluster& y) { return x.load > y.load; });
  std::vector<std::vector<int32_t>> queues(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (const auto& c : clusters) {
    int q = 0;
    for (int i = 1; i < kXcds; ++i)
      if (load[i] < load[q]) q = i;
    load[q] += c.load;
    for (int32_t t = 0; t < c.tiles; ++t) {
      queues[q].push_back(c.node);
      queues[q].push_back(c.head);
      queues[q].push_back(t * rows_per_item);
      queues[q].push_back(c.piece);
    }
  }
  size_t longest = 0;
  for (const auto& q : queues) longest = std::max(longest, q.size() / 4);
  p->items.clear();
  if (clusters.empty()) return;
  for (size_t k = 0; k < longest; ++k)
    for (int q = 0; q < kXcds; ++q) {
      if (k < queues[q].size() / 4) {
        p->items.insert(p->items.end(), queues[q].begin() + 4 * k, queues[q].begin() + 4 * k + 4);
      } else {
        p->items.insert(p->items.end(), {-1, 0, 0, 0});
      }
    }
}

}  // namespace

extern "C" {

pkv_plan* pkv_plan_build(const int32_t* block_tables, const int32_t* seq_lens, int32_t batch,
                         int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t min_members) {
  pkv::clear_error();
  if (batch < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || min_members < 2 || (batch > 0 && (!block_tables || !seq_lens))) {
    pkv::fail(PKV_ERR_INVALID, "pkv_plan_build: invalid arguments");
    return nullptr;
  }
  auto* p = new pkv_plan();
  p->batch = batch;
  p->max_blocks = max_blocks_per_seq;
  p->block_size = block_size;
  p->num_q_heads = num_q_heads;
  p->num_kv_heads = num_kv_heads;
  p->group = num_q_heads / num_kv_heads;
  p->row_info.assign(2 * static_cast<size_t>(batch), 0);

  std::vector<int32_t> full(batch);
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0 || static_cast<int64_t>(seq_lens[b]) > static_cast<int64_t>(max_blocks_per_seq) * block_size) {
      delete p;
      pkv::fail(PKV_ERR_INVALID, "pkv_plan_build: seq_lens[%d] = %d outside [0, max_blocks*block_size]", b, seq_lens[b]);
      return nullptr;
    }
    full[b] = seq_lens[b] / block_size;
  }
  auto id_at = [&](int32_t row, int32_t j) { return block_tables[static_cast<int64_t>(row) * max_blocks_per_seq + j]; };

  std::vector<std::vector<std::pair<int32_t, int32_t>>> path(batch);  // (node, member entry), root first
  std::vector<Group> stack;
  {
    Group g;
    for (int32_t b = 0; b < batch; ++b)
      if (full[b] > 0) g.rows.push_back(b);
    g.start = 0;
    if (static_cast<int32_t>(g.rows.size()) >= min_members) stack.push_back(std::move(g));
  }
  while (!stack.empty()) {
    Group g = std::move(stack.back());
    stack.pop_back();
    int32_t i = g.start;
    for (;;) {  // extend while every row has a full block at i with the same id
      bool same = true;
      const int32_t id0 = full[g.rows[0]] > i ? id_at(g.rows[0], i) : -1;
      for (int32_t r : g.rows) {
        if (full[r] <= i || id_at(r, i) != id0) {
          same = false;
          break;
        }
      }
      if (!same) break;
      ++i;
    }
    if (i > g.start) {
      pkv_plan::Node n;
      n.block_off = static_cast<int32_t>(p->node_blocks.size());
      n.num_blocks = i - g.start;
      n.member_off = static_cast<int32_t>(p->node_members.size() / 2);
      n.num_members = static_cast<int32_t>(g.rows.size());
      for (int32_t j = g.start; j < i; ++j) p->node_blocks.push_back(id_at(g.rows[0], j));
      for (int32_t r : g.rows) {
        path[r].emplace_back(static_cast<int32_t>(p->nodes.size()), static_cast<int32_t>(p->node_members.size() / 2));
        p->node_members.push_back(r);
        p->node_members.push_back(0);  // slot, assigned once pieces are known
        p->row_info[2 * r] = i * block_size;
      }
      p->nodes.push_back(n);
    }
    // split by the id at i; groups keep the rows' order
    std::vector<std::pair<int32_t, int32_t>> by_id;
    for (int32_t r : g.rows)
      if (full[r] > i) by_id.emplace_back(id_at(r, i), r);
    std::stable_sort(by_id.begin(), by_id.end(),
                     [](const std::pair<int32_t, int32_t>& x, const std::pair<int32_t, int32_t>& y) {
                       return x.first < y.first;
                     });
    std::vector<Group> children;
    for (size_t s = 0; s < by_id.size();) {
      size_t e = s;
      while (e < by_id.size() && by_id[e].first == by_id[s].first) ++e;
      if (static_cast<int32_t>(e - s) >= min_members) {
        Group c;
        c.start = i;
        for (size_t k = s; k < e; ++k) c.rows.push_back(by_id[k].second);
        children.push_back(std::move(c));
      }
      s = e;
    }
    for (auto it = children.rbegin(); it != children.rend(); ++it) stack.push_back(std::move(*it));
  }
  split_pieces(p);
  assign_slots(p, path);
  build_items(p);
  build_image(p);
  return p;
}

void pkv_plan_destroy(pkv_plan* plan) { delete plan; }

size_t pkv_plan_device_bytes(const pkv_plan* plan) { return plan ? plan->image.size() * sizeof(int32_t) : 0; }

int32_t pkv_plan_num_nodes(const pkv_plan* plan) { return plan ? static_cast<int32_t>(plan->nodes.size()) : -1; }

pkv_status pkv_plan_node(const pkv_plan* plan, int32_t node, int32_t* num_blocks, int32_t* num_members,
                         int32_t* blocks_out, int32_t* members_out) {
  pkv::clear_error();
  if (!plan || node < 0 || node >= static_cast<int32_t>(plan->nodes.size()))
    return pkv::fail(PKV_ERR_INVALID, "pkv_plan_node: bad plan or node index");
  const auto& n = plan->nodes[node];
  if (num_blocks) *num_blocks = n.num_blocks;
  if (num_members) *num_members = n.num_members;
  if (blocks_out) std::memcpy(blocks_out, plan->node_blocks.data() + n.block_off, sizeof(int32_t) * n.num_blocks);
  if (members_out)
    for (int32_t k = 0; k < n.num_members; ++k) members_out[k] = plan->node_members[2 * (n.member_off + k)];
  return PKV_OK;
}

int32_t pkv_plan_node_pieces(const pkv_plan* plan, int32_t node) {
  if (!plan || node < 0 || node >= static_cast<int32_t>(plan->nodes.size())) return -1;
  return plan->nodes[node].pieces;
}

pkv_status pkv_plan_row(const pkv_plan* plan, int32_t row, int32_t* shared_tokens, int32_t* depth) {
  pkv::clear_error();
  if (!plan || row < 0 || row >= plan->batch) return pkv::fail(PKV_ERR_INVALID, "pkv_plan_row: bad plan or row");
  if (shared_tokens) *shared_tokens = plan->row_info[2 * row];
  if (depth) *depth = plan->row_info[2 * row + 1];
  return PKV_OK;
}

}  // extern "C"
