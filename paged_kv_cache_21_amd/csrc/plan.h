// Host representation of a cascade plan and its device image.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

struct pkv_plan {
  int32_t batch = 0;
  int32_t max_blocks = 0;
  int32_t block_size = 0;
  int32_t num_q_heads = 0;
  int32_t num_kv_heads = 0;
  int32_t group = 0;

  struct Node {
    int32_t block_off, num_blocks, member_off, num_members;
    int32_t pieces = 1, piece_blocks = 0;  // token split of the node across work-groups
  };
  std::vector<Node> nodes;
  std::vector<int32_t> node_blocks;   // physical ids, concatenated per node
  std::vector<int32_t> node_members;  // (row, partial slot) pairs, concatenated per node
  std::vector<int32_t> row_info;      // (shared tokens, depth) per row
  int32_t max_depth = 0;
  std::vector<int32_t> items;  // (node, kv head, first row, piece) in launch order; node -1 = idle

  // device image: one int32 array holding, in order, row_info, nodes, node_blocks, node_members, items
  std::vector<int32_t> image;
  size_t off_row_info = 0, off_nodes = 0, off_blocks = 0, off_members = 0, off_items = 0;
  const int32_t* device = nullptr;  // bound by pkv_plan_upload

  int32_t num_items() const { return static_cast<int32_t>(items.size() / 4); }
};
