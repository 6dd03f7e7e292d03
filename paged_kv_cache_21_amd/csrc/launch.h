// Kernel launch interface between the C-ABI dispatch (capi.cpp) and the HIP
// translation units.  Plain structs of pointers and sizes; no HIP types beyond
// hipStream_t / hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Block copies: for i < n and array k < num_arrays, block dst_ids[i] of dst[k]
// gets block src_ids[i] of src[k] (block_bytes[k] bytes, a multiple of 16).
// Pointers are device addresses (for pinned host memory, its device mapping).
struct CopyArgs {
  char* dst[4];
  const char* src[4];
  int64_t block_bytes[4];
  int32_t num_arrays;
  int64_t dst_blocks;
  int64_t src_blocks;
  const int32_t* dst_ids;
  const int32_t* src_ids;
  int32_t n;
  int32_t max_workgroups;  // 0: one work-group per (block, array) item
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

struct AppendArgs {
  uint16_t* k_pages;  // 16-bit pages; FP8 pages: byte arrays (cast)
  uint16_t* v_pages;
  float* k_scales;    // FP8 pages: [num_blocks][num_kv_heads][block_size] (else null)
  float* v_scales;
  int32_t num_kv_heads;
  int32_t head_dim;
  int64_t num_blocks;
  int32_t block_size;
  int32_t row_elems;  // num_kv_heads * head_dim
  const uint16_t* k_new;
  const uint16_t* v_new;
  int32_t num_tokens;
  const int64_t* slot_mapping;
  const int32_t* cow_src;
  const int32_t* cow_dst;
  const int32_t* cow_rows;
  int32_t num_cow;
};

// Split-K decode over each row's own tokens [shared_tokens_b, len_b), with the
// work spread evenly over a fixed number of persistent waves.
//
// Work order: rows b, then KV heads, then the row's own blocks j; a row-head
// "segment" (b, h) holds n_b = ceil((len_b - shared_b) / 16) blocks and spans
// n_b + kSegUnits positions of the order (the extra positions hold no block and
// stand for the segment's fixed cost).  With T the total number of positions and W
// waves, wave w takes the blocks at positions [w*c, (w+1)*c),
// c = max(min_chunk, ceil(T / W)).  Partial k of segment (b, h) comes from wave
// floor(S_bh / c) + k (S_bh = the position of the segment's block 0) and goes to
// partial slot depth_b + k; the wave that starts a segment also stores its partial
// count.
struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* row_info;  // [batch][2] = (shared tokens, depth) from a cascade plan, or null
  const float* k_scales;    // FP8 pages: [num_blocks][num_kv_heads][16] per-row scales (else null)
  const float* v_scales;
  float* acc;
  float2* ml;
  int32_t* counts;  // [batch][num_kv_heads] partials per segment (written for non-empty segments)
  // fused append (16-bit pages; null otherwise): each row's new token [batch][num_kv_heads][D]
  // and its last block's copy-on-write source (-1: none)
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* cow_src;
  int64_t num_blocks;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t slots;
  int32_t min_chunk;  // c >= min_chunk bounds the partials per segment
  int32_t num_waves;  // W
  float scale_log2;
  int32_t* status;    // optional device word: PKV_STATUS_BAD_BLOCK is or-ed in for block ids out of range
};

// Merge of all partials of a query row into the normalised output.  Decode:
// rows are sequences, counts holds each (row, KV head)'s split pieces.  Extend:
// rows are query tokens, seq_lens and counts are null (node partials only).
struct MergeArgs {
  const int32_t* seq_lens;
  const int32_t* row_info;  // per row: (tokens covered by nodes, node partial slots)
  const int32_t* counts;
  const float* acc;
  const float2* ml;
  float* out;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t slots;
  int32_t* status;  // optional device word: PKV_STATUS_LEN_CLAMPED is or-ed in for lengths outside [0, limit]
  // One-launch append (k_new non-null): after every read of the call, each row's new token
  // (token len - 1) and, when its last block was copied on write, rows [0, its row) of the
  // copy's source are written into the row's own last block (16-bit pages).
  uint16_t* k_pages = nullptr;
  uint16_t* v_pages = nullptr;
  const int32_t* block_tables = nullptr;
  const uint16_t* k_new = nullptr;  // [batch][num_kv_heads][D]
  const uint16_t* v_new = nullptr;
  const int32_t* cow_src = nullptr;  // per row: copy-on-write source of the last block, or -1
  int64_t num_blocks = 0;
};

// Shared-prefix (cascade) pass over the plan's work items.
struct CascadeArgs {
  const uint16_t* q;
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  // [num_items][item_ints] self-contained work items: header (kv head or -1 = idle, first
  // tile row, piece, index of the piece's first id in node_blocks, blocks in the piece,
  // query rows of the node, logical position of the piece's first token, tokens of the
  // piece holding data, ids of the piece's first kItemFirstIds blocks or -1, padding),
  // then kItemMemberInts ints per member row of the tile (query row or -1, partial slot
  // of this piece, last token position it attends to or INT_MAX, 0)
  const int32_t* item_recs;
  int32_t item_ints;
  const int32_t* node_blocks;   // physical block ids
  float* acc;
  float2* ml;
  int64_t num_blocks;
  int32_t num_items;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t slots;
  int32_t max_piece_blocks;  // largest piece of the plan (selects the kernel instance)
  float scale_log2;
  int32_t rows_per_item;     // query rows per work item: kCascadeRowsPerItem or kExtendRowsPerItem
  const float* k_scales;     // FP8 pages: [num_blocks][num_kv_heads][16] per-row scales (else null)
  const float* v_scales;
  int32_t* status;           // optional device word: PKV_STATUS_BAD_BLOCK for node block ids out of range
};

#ifndef PKV_CASCADE_ROWS
#define PKV_CASCADE_ROWS 64
#endif
constexpr int kCascadeRowsPerItem = PKV_CASCADE_ROWS;  // decode plans: 4 waves x (rows / 64) blocks of 16 rows
#ifndef PKV_EXTEND_ROWS
#define PKV_EXTEND_ROWS 128
#endif
constexpr int kExtendRowsPerItem = PKV_EXTEND_ROWS;  // extend plans: 4 waves x 2 x 16 rows
constexpr int kCascadeMaxPieceBlocks = 256;  // blocks of one work item's token piece
constexpr int kItemHeadInts = 16;       // header ints of a work-item record
constexpr int kItemFirstIds = 4;        // block ids of a piece's first two chunks in the header
constexpr int kItemMemberInts = 4;      // ints per member entry of a work-item record

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
// FP8 pages: quantize each new token's head vectors; src_dtype 0 f16, 1 bf16 for k_new / v_new.
hipError_t launch_kv_append_fp8(int src_dtype, const AppendArgs& a, hipStream_t stream);
// dtype: 0 f16, 1 bf16 (q and pages); 2 FP8 pages with f16 q, 3 FP8 pages with bf16 q.
// Returns hipErrorInvalidValue for shapes not built.
hipError_t launch_decode_split(int dtype, int head_dim, int group, const SplitArgs& a, hipStream_t stream);
// Waves the split kernel runs as for these shapes on the current device (all resident at once).
int decode_split_waves(int dtype, int head_dim, int group, bool fused);
hipError_t launch_merge(int head_dim, const MergeArgs& a, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int grid, hipStream_t stream);
hipError_t launch_cascade(int dtype, int head_dim, int group, const CascadeArgs& a, hipStream_t stream);

// Size of the fixed per-device scratch the no-allocation decode uses in place of a
// caller workspace, and its device address on the current device (taken once per
// device; an error if the runtime cannot resolve it).
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_address(void** out);

}  // namespace pkv
