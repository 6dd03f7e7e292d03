// Host representation of a cascade / extend plan and its device image.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

struct pkv_plan {
  enum Kind { kDecode = 0, kExtend = 1 };
  Kind kind = kDecode;
  int32_t batch = 0;
  int32_t max_blocks = 0;
  int32_t block_size = 0;
  int32_t num_q_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t group = 0;
  // Query rows: decode, one per sequence (row b); extend, one per new token, in
  // (sequence, token) order.
  int32_t num_query_rows = 0;
  int32_t rows_per_item = 64;  // query rows of a cascade work item (tile), set by the plan's kind

  struct Node {
    int32_t block_off, num_blocks, member_off, num_members;
    int32_t pieces = 1, piece_blocks = 0;  // token split of the node across work-groups
    int32_t start_tok = 0;                 // logical index of the node's first token in its rows
    int32_t valid_tokens = 0;              // tokens of the node holding data (the rest are masked, values zeroed)
  };
  static constexpr int kNodeInts = 8;
  static constexpr int kMemberInts = 3;
  std::vector<Node> nodes;
  std::vector<int32_t> node_blocks;   // physical ids, concatenated per node
  // (query row, partial slot of piece 0, last token the query row may attend to), concatenated per node
  std::vector<int32_t> node_members;
  std::vector<int32_t> row_info;  // per query row: (tokens covered by nodes, partial slots used)
  int32_t max_depth = 0;
  // decode: every row's last token lies past its nodes (so a token appended there is
  // read by the split pass, which the fused append needs)
  bool last_tokens_own = true;
  std::vector<int32_t> items;  // (node, kv head, first member row, piece) in launch order; node -1 = idle

  // Self-contained work-item records, the form the matrix-core kernel reads: per item a
  // header of kItemHeadInts ints (kv head or -1 = idle, first tile row, piece, index of
  // the piece's first id in node_blocks, blocks in the piece, query rows of the node,
  // logical position of the piece's first token, tokens of the piece holding data, the
  // ids of the piece's first kItemFirstIds blocks or -1, zero padding), then one entry
  // of kItemMemberInts ints per member row of the tile (query row or -1 past the node's
  // members, partial slot of this piece, last attended position or INT32_MAX, 0).
  // Everything an item needs before its first K/V loads is one read away.
  static constexpr int kItemHeadInts = 16;
  static constexpr int kItemFirstIds = 4;
  static constexpr int kItemMemberInts = 4;
  int32_t item_ints = 0;  // ints per record: kItemHeadInts + kItemMemberInts * rows_per_item / group

  // device image: one int32 array holding, in order, row_info, nodes, node_blocks, node_members,
  // items, then (from a multiple of 4 ints) the item records
  std::vector<int32_t> image;
  size_t off_row_info = 0, off_nodes = 0, off_blocks = 0, off_members = 0, off_items = 0, off_item_recs = 0;
  const int32_t* device = nullptr;  // bound by pkv_plan_upload

  int32_t num_items() const { return static_cast<int32_t>(items.size() / 4); }
  int32_t max_piece_blocks_ = 0;  // largest piece over the nodes, set with the pieces
  int32_t max_piece_blocks() const { return max_piece_blocks_; }
};
