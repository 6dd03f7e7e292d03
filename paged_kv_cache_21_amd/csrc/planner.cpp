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
//
// The extend plan (several new query tokens per row, each attending causally
// to its row's cache) uses the same nodes, with one member entry per query
// token instead of per row, plus one private node per row covering the rest of
// its blocks (the partly filled last block included); every entry carries the
// last token it may attend to, so one matrix-core kernel serves both.
#include <algorithm>
#include <climits>
#include <cstring>
#include <utility>
#include <vector>

#include "host_common.h"
#include "launch.h"
#include "plan.h"

static_assert(pkv_plan::kItemHeadInts == pkv::kItemHeadInts && pkv_plan::kItemFirstIds == pkv::kItemFirstIds &&
                  pkv_plan::kItemMemberInts == pkv::kItemMemberInts,
              "work-item record layout shared by the planner and the matrix-core kernel");

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
    im.insert(im.end(), {n.block_off, n.num_blocks, n.member_off, n.num_members, n.pieces, n.piece_blocks,
                         n.start_tok, n.valid_tokens});
  }
  p->off_blocks = im.size();
  im.insert(im.end(), p->node_blocks.begin(), p->node_blocks.end());
  p->off_members = im.size();
  im.insert(im.end(), p->node_members.begin(), p->node_members.end());
  p->off_items = im.size();
  im.insert(im.end(), p->items.begin(), p->items.end());
  while (im.size() % 4) im.push_back(0);
  p->off_item_recs = im.size();
  const int32_t per_tile = p->rows_per_item / p->group;  // member rows of a tile
  p->item_ints = pkv_plan::kItemHeadInts + pkv_plan::kItemMemberInts * per_tile;
  for (size_t it = 0; it + 4 <= p->items.size(); it += 4) {
    const int32_t node = p->items[it], head = p->items[it + 1], row0 = p->items[it + 2], piece = p->items[it + 3];
    const size_t base = im.size();
    im.resize(base + p->item_ints, 0);
    int32_t* r = im.data() + base;
    if (node < 0) {  // idle item: no blocks, no member rows
      r[0] = -1;
      for (int32_t j = 0; j < pkv_plan::kItemFirstIds; ++j) r[8 + j] = -1;
      for (int32_t li = 0; li < per_tile; ++li) {
        r[pkv_plan::kItemHeadInts + pkv_plan::kItemMemberInts * li] = -1;
        r[pkv_plan::kItemHeadInts + pkv_plan::kItemMemberInts * li + 2] = -1;
      }
      continue;
    }
    const auto& n = p->nodes[node];
    const int32_t pb0 = piece * n.piece_blocks;
    const int32_t nblk = std::min(n.piece_blocks, n.num_blocks - pb0);
    r[0] = head;
    r[1] = row0;
    r[2] = piece;
    r[3] = n.block_off + pb0;
    r[4] = nblk;
    r[5] = n.num_members * p->group;
    r[6] = n.start_tok + pb0 * p->block_size;
    r[7] = n.valid_tokens - pb0 * p->block_size;
    for (int32_t j = 0; j < pkv_plan::kItemFirstIds; ++j) r[8 + j] = j < nblk ? p->node_blocks[n.block_off + pb0 + j] : -1;
    for (int32_t li = 0; li < per_tile; ++li) {
      int32_t* e = r + pkv_plan::kItemHeadInts + pkv_plan::kItemMemberInts * li;
      const int32_t m = row0 / p->group + li;  // member index inside the node
      if (m < n.num_members) {
        const int32_t* mrec = &p->node_members[pkv_plan::kMemberInts * (n.member_off + m)];
        e[0] = mrec[0];
        e[1] = mrec[1] + piece;
        e[2] = mrec[2];
      } else {
        e[0] = -1;
        e[2] = -1;
      }
    }
  }
  if (im.empty()) im.push_back(0);
}

int32_t member_limit(const pkv_plan* p, int32_t entry) { return p->node_members[pkv_plan::kMemberInts * entry + 2]; }

// Pieces of node n that the members of 64-row tile t need: the pieces starting at
// or before the latest token any of the tile's members may attend to (pieces
// past it would be fully masked for every member, so no work item runs them).
int32_t tile_pieces(const pkv_plan* p, int32_t n, int32_t t) {
  const auto& nd = p->nodes[n];
  const int32_t per_tile = p->rows_per_item / p->group;  // member entries per tile
  const int32_t e0 = t * per_tile, e1 = std::min(nd.num_members, e0 + per_tile);
  int32_t lim = INT_MIN;
  for (int32_t e = e0; e < e1; ++e) lim = std::max(lim, member_limit(p, nd.member_off + e));
  if (lim == INT_MAX) return nd.pieces;
  const int64_t span = static_cast<int64_t>(lim) - nd.start_tok;  // latest attended token, node-local
  if (span < 0) return 0;
  return static_cast<int32_t>(std::min<int64_t>(nd.pieces, span / (static_cast<int64_t>(nd.piece_blocks) * p->block_size) + 1));
}

// Token pieces.  A node's work is (64-row tiles) x (KV heads) x (blocks); the
// chip wants a few work-groups per CU.  Long nodes are cut into pieces of about
// `target` blocks so the item count lands near kTargetItems, but never below
// kMinPieceBlocks blocks per piece: every piece costs each member row one more
// fp32 partial per query head, written and read back once.
void split_pieces(pkv_plan* p) {
  // items the chip runs at once: one work-group of the 256-row instance per CU, about
  // four of the smaller ones; aim at two rounds
  const int64_t kTargetItems = p->rows_per_item >= 128 ? 512 : 1024;
  constexpr int32_t kMinPieceBlocks = 32;
  constexpr int32_t kMaxPieceBlocks = pkv::kCascadeMaxPieceBlocks;
  const int rows_per_item = p->rows_per_item;
  int64_t work = 0;
  for (const auto& n : p->nodes) {
    const int64_t tiles = (static_cast<int64_t>(n.num_members) * p->group + rows_per_item - 1) / rows_per_item;
    work += tiles * p->num_kv_heads * n.num_blocks;
  }
  const int64_t target = std::max<int64_t>(kMinPieceBlocks, (work + kTargetItems - 1) / kTargetItems);
  for (auto& n : p->nodes) {
    // at most kMaxPieceBlocks blocks per piece: the cascade kernel keeps a piece's
    // block ids in four 64-lane registers
    n.pieces = static_cast<int32_t>(std::max<int64_t>(
        std::max<int64_t>(1, n.num_blocks / target), (n.num_blocks + kMaxPieceBlocks - 1) / kMaxPieceBlocks));
    n.piece_blocks = (n.num_blocks + n.pieces - 1) / n.pieces;
    n.pieces = (n.num_blocks + n.piece_blocks - 1) / n.piece_blocks;
    p->max_piece_blocks_ = std::max(p->max_piece_blocks_, n.piece_blocks);
  }
}

// Partial slots: every query row's node pieces take consecutive slots, nodes in
// creation order (root first along each path).
void assign_slots(pkv_plan* p) {
  std::vector<int32_t> used(p->num_query_rows, 0);
  const int32_t per_tile = p->rows_per_item / p->group;
  for (int32_t n = 0; n < static_cast<int32_t>(p->nodes.size()); ++n) {
    const auto& nd = p->nodes[n];
    for (int32_t e = 0; e < nd.num_members; ++e) {
      int32_t* rec = &p->node_members[pkv_plan::kMemberInts * (nd.member_off + e)];
      rec[1] = used[rec[0]];
      used[rec[0]] += tile_pieces(p, n, e / per_tile);
    }
  }
  p->max_depth = 0;
  for (int32_t r = 0; r < p->num_query_rows; ++r) {
    p->row_info[2 * r + 1] = used[r];
    p->max_depth = std::max(p->max_depth, used[r]);
  }
}

// Work items: one per (node, KV head, 64-row tile, piece).  Work-group i runs on
// XCD i % 8, and each XCD has its own L2, so all tiles of one (node, head, piece)
// go to the same XCD queue: the tiles after the first find the piece's K/V in
// that L2.  Clusters are dealt to the least-loaded queue (load = blocks x tiles);
// queues are interleaved into launch order and padded with idle items.
void build_items(pkv_plan* p) {
  constexpr int kXcds = 8;
  const int rows_per_item = p->rows_per_item;
  struct Cluster {
    int32_t node, head, tiles, piece;
    int64_t load;
  };
  std::vector<Cluster> clusters;
  struct Tiles {
    std::vector<int32_t> first_rows;
  };
  std::vector<std::vector<Tiles>> per_piece;  // [node][piece]: tiles that need the piece
  for (int32_t n = 0; n < static_cast<int32_t>(p->nodes.size()); ++n) {
    const auto& nd = p->nodes[n];
    const int32_t rows = nd.num_members * p->group;
    const int32_t tiles = (rows + rows_per_item - 1) / rows_per_item;
    per_piece.emplace_back(nd.pieces);
    for (int32_t t = 0; t < tiles; ++t) {
      const int32_t np = tile_pieces(p, n, t);
      for (int32_t pc = 0; pc < np; ++pc) per_piece[n][pc].first_rows.push_back(t * rows_per_item);
    }
    for (int32_t pc = 0; pc < nd.pieces; ++pc) {
      const int32_t blocks = std::min(nd.piece_blocks, nd.num_blocks - pc * nd.piece_blocks);
      const int32_t nt = static_cast<int32_t>(per_piece[n][pc].first_rows.size());
      if (nt == 0) continue;
      for (int32_t h = 0; h < p->num_kv_heads; ++h)
        clusters.push_back({n, h, nt, pc, static_cast<int64_t>(blocks) * nt});
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
    for (int32_t first_row : per_piece[c.node][c.piece].first_rows) {
      queues[q].push_back(c.node);
      queues[q].push_back(c.head);
      queues[q].push_back(first_row);
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

// The trie walk shared by both plans.  rows_in: rows taking part; full[b]: full
// blocks of row b; add_members(r): append row r's member entries (query row,
// slot placeholder, limit) to node_members; covered[r] receives the tokens of row
// r covered by nodes.
template <class AddMembers>
void build_shared_nodes(pkv_plan* p, const int32_t* block_tables, const std::vector<int32_t>& rows_in,
                        const std::vector<int32_t>& full, int32_t min_members, AddMembers add_members,
                        std::vector<int32_t>& covered) {
  const int32_t max_blocks = p->max_blocks, block_size = p->block_size;
  auto id_at = [&](int32_t row, int32_t j) { return block_tables[static_cast<int64_t>(row) * max_blocks + j]; };
  std::vector<Group> stack;
  {
    Group g;
    for (int32_t b : rows_in)
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
      n.member_off = static_cast<int32_t>(p->node_members.size() / pkv_plan::kMemberInts);
      n.start_tok = g.start * block_size;
      n.valid_tokens = n.num_blocks * block_size;
      for (int32_t j = g.start; j < i; ++j) p->node_blocks.push_back(id_at(g.rows[0], j));
      for (int32_t r : g.rows) {
        add_members(r);
        covered[r] = i * block_size;
      }
      n.num_members = static_cast<int32_t>(p->node_members.size() / pkv_plan::kMemberInts) - n.member_off;
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
}

pkv_plan* new_plan(pkv_plan::Kind kind, int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                   int32_t num_q_heads, int32_t num_kv_heads) {
  auto* p = new pkv_plan();
  p->kind = kind;
  p->batch = batch;
  p->max_blocks = max_blocks_per_seq;
  p->block_size = block_size;
  p->num_q_heads = num_q_heads;
  p->num_kv_heads = num_kv_heads;
  p->group = num_q_heads / num_kv_heads;
  // the extend pass is compute-bound: register blocking two 16-row blocks per wave
  // pays there; a decode cascade keeps more resident waves with one
  p->rows_per_item = kind == pkv_plan::kExtend ? pkv::kExtendRowsPerItem : pkv::kCascadeRowsPerItem;
  return p;
}

void finish_plan(pkv_plan* p, const std::vector<int32_t>& covered_per_query_row) {
  // A decode plan whose every node has at least 128 query rows takes 128-row work
  // items (two 16-row blocks per wave share each LDS operand; two work-groups per
  // CU); one with smaller nodes keeps 64-row items, four work-groups per CU, so the
  // many small items still overlap (tree search 79 -> 74 us with 128 rows, radix tree
  // 68 -> 93 us).
  if (p->kind == pkv_plan::kDecode && !p->nodes.empty()) {
    int32_t min_rows = INT32_MAX;
    for (const auto& n : p->nodes) min_rows = std::min(min_rows, n.num_members * p->group);
    p->rows_per_item = min_rows >= 2 * pkv::kCascadeRowsPerItem ? 2 * pkv::kCascadeRowsPerItem
                                                                  : pkv::kCascadeRowsPerItem;
  }
  p->row_info.assign(2 * static_cast<size_t>(p->num_query_rows), 0);
  for (int32_t r = 0; r < p->num_query_rows; ++r) p->row_info[2 * r] = covered_per_query_row[r];
  split_pieces(p);
  assign_slots(p);
  build_items(p);
  build_image(p);
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
  std::vector<int32_t> full(batch), rows(batch);
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0 || static_cast<int64_t>(seq_lens[b]) > static_cast<int64_t>(max_blocks_per_seq) * block_size) {
      pkv::fail(PKV_ERR_INVALID, "pkv_plan_build: seq_lens[%d] = %d outside [0, max_blocks*block_size]", b, seq_lens[b]);
      return nullptr;
    }
    full[b] = seq_lens[b] / block_size;
    rows[b] = b;
  }
  pkv_plan* p = new_plan(pkv_plan::kDecode, batch, max_blocks_per_seq, block_size, num_q_heads, num_kv_heads);
  p->num_query_rows = batch;
  std::vector<int32_t> covered(batch, 0);
  build_shared_nodes(
      p, block_tables, rows, full, min_members,
      [&](int32_t r) { p->node_members.insert(p->node_members.end(), {r, 0, INT_MAX}); }, covered);
  for (int32_t b = 0; b < batch; ++b) p->last_tokens_own &= seq_lens[b] == 0 || covered[b] < seq_lens[b];
  finish_plan(p, covered);
  return p;
}

pkv_plan* pkv_plan_build_extend(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_lens,
                                int32_t batch, int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t min_members) {
  pkv::clear_error();
  if (batch < 0 || max_blocks_per_seq < 0 || block_size <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || min_members < 2 ||
      (batch > 0 && (!block_tables || !seq_lens || !q_lens))) {
    pkv::fail(PKV_ERR_INVALID, "pkv_plan_build_extend: invalid arguments");
    return nullptr;
  }
  std::vector<int32_t> full(batch, 0), q_start(batch + 1, 0), rows;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t len = seq_lens[b], ql = q_lens[b];
    if (len < 0 || static_cast<int64_t>(len) > static_cast<int64_t>(max_blocks_per_seq) * block_size || ql < 0 ||
        ql > len) {
      pkv::fail(PKV_ERR_INVALID, "pkv_plan_build_extend: row %d: need 0 <= q_lens <= seq_lens <= max_blocks*block_size",
                b);
      return nullptr;
    }
    if (static_cast<int64_t>(q_start[b]) + ql > (1 << 28)) {
      pkv::fail(PKV_ERR_INVALID, "pkv_plan_build_extend: too many query tokens");
      return nullptr;
    }
    q_start[b + 1] = q_start[b] + ql;
    if (ql > 0) {
      rows.push_back(b);
      full[b] = len / block_size;
    }
  }
  pkv_plan* p = new_plan(pkv_plan::kExtend, batch, max_blocks_per_seq, block_size, num_q_heads, num_kv_heads);
  p->num_query_rows = q_start[batch];
  auto add_members = [&](int32_t r) {
    const int32_t first_pos = seq_lens[r] - q_lens[r];
    for (int32_t i = 0; i < q_lens[r]; ++i) p->node_members.insert(p->node_members.end(), {q_start[r] + i, 0, first_pos + i});
  };
  std::vector<int32_t> covered(batch, 0);
  build_shared_nodes(p, block_tables, rows, full, min_members, add_members, covered);
  // one private node per row over the rest of its blocks
  for (int32_t r : rows) {
    const int32_t len = seq_lens[r];
    if (len <= covered[r]) continue;
    pkv_plan::Node n;
    n.block_off = static_cast<int32_t>(p->node_blocks.size());
    const int32_t j0 = covered[r] / block_size, j1 = (len + block_size - 1) / block_size;
    n.num_blocks = j1 - j0;
    n.member_off = static_cast<int32_t>(p->node_members.size() / pkv_plan::kMemberInts);
    n.start_tok = covered[r];
    n.valid_tokens = len - covered[r];
    for (int32_t j = j0; j < j1; ++j) p->node_blocks.push_back(block_tables[static_cast<int64_t>(r) * max_blocks_per_seq + j]);
    add_members(r);
    n.num_members = q_lens[r];
    p->nodes.push_back(n);
  }
  std::vector<int32_t> covered_q(p->num_query_rows, 0);
  for (int32_t r : rows)
    for (int32_t i = 0; i < q_lens[r]; ++i) covered_q[q_start[r] + i] = covered[r];
  finish_plan(p, covered_q);
  return p;
}

void pkv_plan_destroy(pkv_plan* plan) { delete plan; }

size_t pkv_plan_device_bytes(const pkv_plan* plan) { return plan ? plan->image.size() * sizeof(int32_t) : 0; }

int32_t pkv_plan_num_nodes(const pkv_plan* plan) { return plan ? static_cast<int32_t>(plan->nodes.size()) : -1; }

int32_t pkv_plan_num_query_rows(const pkv_plan* plan) { return plan ? plan->num_query_rows : -1; }

int32_t pkv_plan_rows_per_item(const pkv_plan* plan) { return plan ? plan->rows_per_item : -1; }

int64_t pkv_plan_item_records(const pkv_plan* plan, int32_t* ints_per_item) {
  if (!plan) return -1;
  if (ints_per_item) *ints_per_item = plan->item_ints;
  return static_cast<int64_t>(plan->off_item_recs);
}

int64_t pkv_plan_image(const pkv_plan* plan, int32_t* out, int64_t capacity, int64_t* offsets) {
  if (!plan) return -1;
  const int64_t n = static_cast<int64_t>(plan->image.size());
  if (out && capacity >= n) std::memcpy(out, plan->image.data(), sizeof(int32_t) * n);
  if (offsets) {
    offsets[0] = static_cast<int64_t>(plan->off_row_info);
    offsets[1] = static_cast<int64_t>(plan->off_nodes);
    offsets[2] = static_cast<int64_t>(plan->off_blocks);
    offsets[3] = static_cast<int64_t>(plan->off_members);
    offsets[4] = static_cast<int64_t>(plan->off_items);
    offsets[5] = plan->max_depth;
  }
  return n;
}

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
    for (int32_t k = 0; k < n.num_members; ++k)
      members_out[k] = plan->node_members[pkv_plan::kMemberInts * (n.member_off + k)];
  return PKV_OK;
}

int32_t pkv_plan_node_pieces(const pkv_plan* plan, int32_t node) {
  if (!plan || node < 0 || node >= static_cast<int32_t>(plan->nodes.size())) return -1;
  return plan->nodes[node].pieces;
}

pkv_status pkv_plan_row(const pkv_plan* plan, int32_t row, int32_t* shared_tokens, int32_t* depth) {
  pkv::clear_error();
  if (!plan || row < 0 || row >= plan->num_query_rows) return pkv::fail(PKV_ERR_INVALID, "pkv_plan_row: bad plan or row");
  if (shared_tokens) *shared_tokens = plan->row_info[2 * row];
  if (depth) *depth = plan->row_info[2 * row + 1];
  return PKV_OK;
}

}  // extern "C"
