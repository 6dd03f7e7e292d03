// C-ABI entry points for the device operations: argument checks on the host,
// workspace layout, kernel dispatch, optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "host_common.h"
#include "launch.h"
#include "plan.h"

namespace pkv {

namespace {
thread_local std::string g_error;
}

void set_error_message(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
}

void clear_error() { g_error.clear(); }

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// kernel timing

struct Timing {
  std::mutex mu;
  bool on = false;
  struct Pending {
    int kernel;
    hipEvent_t start, stop;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> spare;
  double total_ms[PKV_NUM_KERNELS] = {};
  int64_t count[PKV_NUM_KERNELS] = {};
};

Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.spare.empty()) {
    hipEvent_t e = t.spare.back();
    t.spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
pkv_status launch(int kernel, const char* what, hipStream_t stream, F&& f) {
  Timing& t = timing();
  hipEvent_t start = nullptr, stop = nullptr;
  if (t.on) {
    std::lock_guard<std::mutex> lk(t.mu);
    start = take_event(t);
    stop = take_event(t);
    if (start) (void)hipEventRecord(start, stream);
  }
  const hipError_t err = f();
  if (t.on && start && stop) {
    (void)hipEventRecord(stop, stream);
    std::lock_guard<std::mutex> lk(t.mu);
    t.pending.push_back({kernel, start, stop});
  }
  if (err != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// split-K sizing shared by the workspace query and the decode call

// Smallest share of blocks a wave of the split kernel takes; bounds the number
// of partials a (row, KV head) segment can produce.
#ifndef PKV_MIN_CHUNK
#define PKV_MIN_CHUNK 8
#endif

struct DecodeLayout {
  int32_t slots;       // partial slots per row: cascade nodes + split pieces
  size_t ml_offset;    // bytes
  size_t counts_offset;
  size_t bytes;
};

// Workspace: fp32 partials acc [batch][slots][Hq][D], (m, l) pairs [batch][slots][Hq],
// partial counts int32 [batch][Hkv].  A (row, head) segment of n blocks is cut
// into at most ceil(n / PKV_MIN_CHUNK) + 1 pieces by the split kernel.
DecodeLayout decode_layout(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_seq_len, const pkv_plan* plan) {
  DecodeLayout L{};
  const int32_t min_shared = [&] {
    if (!plan || plan->batch == 0) return 0;
    int32_t m = plan->row_info[0];
    for (int32_t b = 1; b < plan->batch; ++b) m = std::min(m, plan->row_info[2 * b]);
    return m;
  }();
  const int64_t span = std::max<int64_t>(0, static_cast<int64_t>(max_seq_len) - min_shared);
  const int64_t max_nb = (span + 15) / 16;
  const int64_t pieces = max_nb > 0 ? (max_nb + PKV_MIN_CHUNK - 1) / PKV_MIN_CHUNK + 1 : 0;
  L.slots = static_cast<int32_t>(pieces + (plan ? plan->max_depth : 0));
  const size_t recs = static_cast<size_t>(batch) * L.slots * num_q_heads;
  const size_t acc_bytes = recs * head_dim * sizeof(float);
  L.ml_offset = (acc_bytes + 255) & ~static_cast<size_t>(255);
  L.counts_offset = (L.ml_offset + recs * sizeof(float2) + 255) & ~static_cast<size_t>(255);
  L.bytes = L.counts_offset + static_cast<size_t>(batch) * num_kv_heads * sizeof(int32_t);
  return L;
}

bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

}  // namespace
}  // namespace pkv

using pkv::fail;

extern "C" {

const char* pkv_last_error(void) { return pkv::g_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

pkv_status pkv_kv_append(void* k_pages, void* v_pages, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, const void* k_new, const void* v_new, int32_t num_tokens,
                         const int64_t* slot_mapping, const int32_t* cow_src, const int32_t* cow_dst,
                         const int32_t* cow_rows, int32_t num_cow, void* stream) {
  pkv::clear_error();
  if (dtype != PKV_F16 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: dtype %d", dtype);
  if (num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_tokens < 0 || num_cow < 0)
    return fail(PKV_ERR_INVALID, "pkv_kv_append: negative or zero size");
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if ((row_elems * 2) % 16 != 0 || row_elems > (1 << 24))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append: num_kv_heads*head_dim*2 must be a multiple of 16 bytes");
  if (num_tokens > 0 && (!k_pages || !v_pages || !k_new || !v_new || !slot_mapping))
    return fail(PKV_ERR_INVALID, "pkv_kv_append: null pointer");
  if (num_cow > 0 && (!k_pages || !v_pages || !cow_src || !cow_dst || !cow_rows))
    return fail(PKV_ERR_INVALID, "pkv_kv_append: null copy-on-write pointer");
  if (!pkv::aligned16(k_pages) || !pkv::aligned16(v_pages) || !pkv::aligned16(k_new) || !pkv::aligned16(v_new))
    return fail(PKV_ERR_INVALID, "pkv_kv_append: page and token pointers must be 16-byte aligned");
  if (static_cast<int64_t>(num_tokens) + num_cow > 0x7fffffff) return fail(PKV_ERR_INVALID, "pkv_kv_append: too many work items");
  pkv::AppendArgs a{static_cast<uint16_t*>(k_pages),
                    static_cast<uint16_t*>(v_pages),
                    nullptr,
                    nullptr,
                    num_kv_heads,
                    head_dim,
                    num_blocks,
                    block_size,
                    static_cast<int32_t>(row_elems),
                    static_cast<const uint16_t*>(k_new),
                    static_cast<const uint16_t*>(v_new),
                    num_tokens,
                    slot_mapping,
                    cow_src,
                    cow_dst,
                    cow_rows,
                    num_cow};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return pkv::launch(PKV_KERNEL_APPEND, "kv_append", s, [&] { return pkv::launch_kv_append(a, s); });
}

pkv_status pkv_kv_append_fp8(void* k_pages, void* v_pages, float* k_scales, float* v_scales, int64_t num_blocks,
                             int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                             const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                             const int32_t* cow_src, const int32_t* cow_dst, const int32_t* cow_rows, int32_t num_cow,
                             void* stream) {
  pkv::clear_error();
  if (src_dtype != PKV_F16 && src_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append_fp8: source dtype %d", src_dtype);
  if (num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || num_tokens < 0 || num_cow < 0)
    return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: negative or zero size");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append_fp8: head_dim %d (built: 64, 128)", head_dim);
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (row_elems > (1 << 24)) return fail(PKV_ERR_UNSUPPORTED, "pkv_kv_append_fp8: token row too large");
  if ((num_tokens > 0 || num_cow > 0) && (!k_pages || !v_pages || !k_scales || !v_scales))
    return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: null page or scale pointer");
  if (num_tokens > 0 && (!k_new || !v_new || !slot_mapping)) return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: null pointer");
  if (num_cow > 0 && (!cow_src || !cow_dst || !cow_rows))
    return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: null copy-on-write pointer");
  if (!pkv::aligned16(k_pages) || !pkv::aligned16(v_pages) || !pkv::aligned16(k_new) || !pkv::aligned16(v_new) ||
      ((reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) & 3u))
    return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: pages and tokens must be 16-byte, scales 4-byte aligned");
  if (static_cast<int64_t>(num_tokens) + num_cow > 0x7fffffff)
    return fail(PKV_ERR_INVALID, "pkv_kv_append_fp8: too many work items");
  pkv::AppendArgs a{static_cast<uint16_t*>(k_pages),
                    static_cast<uint16_t*>(v_pages),
                    k_scales,
                    v_scales,
                    num_kv_heads,
                    head_dim,
                    num_blocks,
                    block_size,
                    static_cast<int32_t>(row_elems),
                    static_cast<const uint16_t*>(k_new),
                    static_cast<const uint16_t*>(v_new),
                    num_tokens,
                    slot_mapping,
                    cow_src,
                    cow_dst,
                    cow_rows,
                    num_cow};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return pkv::launch(PKV_KERNEL_APPEND, "kv_append_fp8", s, [&] { return pkv::launch_kv_append_fp8(src_dtype, a, s); });
}

size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_seq_len, const pkv_plan* plan) {
  pkv::clear_error();
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0) {
    fail(PKV_ERR_INVALID, "pkv_decode_workspace_bytes: invalid sizes");
    return 0;
  }
  if (plan && (plan->kind != pkv_plan::kDecode || plan->batch != batch)) {
    fail(PKV_ERR_INVALID, "pkv_decode_workspace_bytes: plan not a decode plan for batch %d", batch);
    return 0;
  }
  return pkv::decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, plan).bytes;
}

}  // extern "C"

namespace {

// Shared body of the 16-bit and FP8 decode calls.  kdtype: kernel type code (0 f16,
// 1 bf16, 2 FP8 pages with f16 q, 3 FP8 pages with bf16 q).
pkv_status decode_impl(int kdtype, const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, const void* k_pages, const void* v_pages, const float* k_scales,
                       const float* v_scales, int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float scale,
                       const pkv_plan* plan, void* workspace, size_t workspace_bytes, float* out, int32_t* status,
                       void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                       const int32_t* cow_src = nullptr) {
  const int dtype = kdtype;
  const bool fused = k_new != nullptr;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
      max_seq_len < 0)
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: negative or zero size");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn: head_dim %d (built: 64, 128)", head_dim);
  if (block_size != 16) return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn: block_size %d (built: 16)", block_size);
  if (!pkv::supported_group(group))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn: GQA group %d (built: 1, 2, 4, 8)", group);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: scale is not finite");
  if (plan) {
    if (plan->kind != pkv_plan::kDecode)
      return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: plan was built by pkv_plan_build_extend");
    if (plan->batch != batch || plan->group != group || plan->num_kv_heads != num_kv_heads ||
        plan->block_size != block_size || plan->max_blocks != max_blocks_per_seq)
      return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: plan was built for different shapes");
    if (!plan->device) return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: plan not uploaded (pkv_plan_upload)");
    // the shared nodes attend to every token they cover; a max_seq_len below that would
    // clamp a row's own part but not its shared part
    int32_t covered = 0;
    for (int32_t b = 0; b < plan->batch; ++b) covered = std::max(covered, plan->row_info[2 * b]);
    if (max_seq_len < covered)
      return fail(PKV_ERR_INVALID,
                  "pkv_paged_decode_attn: max_seq_len %d is below the %d tokens the plan's shared nodes cover",
                  max_seq_len, covered);
  }
  const pkv::DecodeLayout L = pkv::decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, plan);
  if (batch == 0) return PKV_OK;
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: the pool must hold at least one block");
  if (!q || !k_pages || !v_pages || !block_tables || !seq_lens || !out)
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: null pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pages) || !pkv::aligned16(v_pages) || !pkv::aligned16(out))
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: q, pages and out must be 16-byte aligned");
  if (workspace_bytes < L.bytes || (L.bytes > 0 && !workspace))
    return fail(PKV_ERR_WORKSPACE, "pkv_paged_decode_attn: workspace of %zu bytes, %zu needed", workspace_bytes,
                L.bytes);
  if (!pkv::aligned16(workspace)) return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn: workspace must be 16-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  float* acc = static_cast<float*>(workspace);
  float2* ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + L.ml_offset);
  const float scale_log2 = scale * 1.4426950408889634f;
  const int32_t* row_info = plan ? plan->device + plan->off_row_info : nullptr;

  if (plan && plan->num_items() > 0) {
    pkv::CascadeArgs c{};
    c.q = static_cast<const uint16_t*>(q);
    c.k_pages = static_cast<const uint16_t*>(k_pages);
    c.v_pages = static_cast<const uint16_t*>(v_pages);
    c.item_recs = plan->device + plan->off_item_recs;
    c.item_ints = plan->item_ints;
    c.node_blocks = plan->device + plan->off_blocks;
    c.acc = acc;
    c.ml = ml;
    c.num_blocks = num_blocks;
    c.num_items = plan->num_items();
    c.num_q_heads = num_q_heads;
    c.num_kv_heads = num_kv_heads;
    c.slots = L.slots;
    c.max_piece_blocks = plan->max_piece_blocks();
    c.scale_log2 = scale_log2;
    c.rows_per_item = plan->rows_per_item;
    c.k_scales = k_scales;
    c.v_scales = v_scales;
    c.status = status;
    pkv_status st = pkv::launch(PKV_KERNEL_CASCADE, "cascade", s,
                                [&] { return pkv::launch_cascade(dtype, head_dim, group, c, s); });
    if (st != PKV_OK) return st;
  }
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + L.counts_offset);
  if (L.slots > (plan ? plan->max_depth : 0)) {
    const int waves = pkv::decode_split_waves(dtype, head_dim, group, fused);
    pkv::SplitArgs sa{static_cast<const uint16_t*>(q),
                      static_cast<const uint16_t*>(k_pages),
                      static_cast<const uint16_t*>(v_pages),
                      block_tables,
                      seq_lens,
                      row_info,
                      k_scales,
                      v_scales,
                      acc,
                      ml,
                      counts,
                      static_cast<const uint16_t*>(k_new),
                      static_cast<const uint16_t*>(v_new),
                      cow_src,
                      num_blocks,
                      batch,
                      num_q_heads,
                      num_kv_heads,
                      max_blocks_per_seq,
                      max_seq_len,
                      L.slots,
                      PKV_MIN_CHUNK,
                      waves,
                      scale_log2,
                      status};
    pkv_status st = pkv::launch(PKV_KERNEL_DECODE_SPLIT, "decode_split", s,
                                [&] { return pkv::launch_decode_split(dtype, head_dim, group, sa, s); });
    if (st != PKV_OK) return st;
  }
  pkv::MergeArgs ma{seq_lens, row_info, counts, acc, ml, out, batch, num_q_heads, num_kv_heads, max_blocks_per_seq,
                    max_seq_len, L.slots, status};
  if (fused) {  // the merge writes the new tokens (and copied rows) once every read is done
    ma.k_pages = static_cast<uint16_t*>(const_cast<void*>(k_pages));
    ma.v_pages = static_cast<uint16_t*>(const_cast<void*>(v_pages));
    ma.block_tables = block_tables;
    ma.k_new = static_cast<const uint16_t*>(k_new);
    ma.v_new = static_cast<const uint16_t*>(v_new);
    ma.cow_src = cow_src;
    ma.num_blocks = num_blocks;
  }
  return pkv::launch(PKV_KERNEL_MERGE, "merge", s, [&] { return pkv::launch_merge(head_dim, ma, s); });
}

}  // namespace

extern "C" {

pkv_status pkv_paged_decode_attn(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, const void* k_pages, const void* v_pages,
                                 int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                 const pkv_plan* plan, void* workspace, size_t workspace_bytes, float* out,
                                 int32_t* status, void* stream) {
  pkv::clear_error();
  if (dtype != PKV_F16 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn: dtype %d", dtype);
  return decode_impl(dtype, q, batch, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, nullptr, nullptr,
                     num_blocks, block_size, block_tables, max_blocks_per_seq, seq_lens, max_seq_len, scale, plan,
                     workspace, workspace_bytes, out, status, stream);
}

pkv_status pkv_paged_decode_attn_append(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t dtype, void* k_pages, void* v_pages,
                                        int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                        const void* k_new, const void* v_new, const int32_t* cow_src, float scale,
                                        const pkv_plan* plan, void* workspace, size_t workspace_bytes, float* out,
                                        int32_t* status, void* stream) {
  pkv::clear_error();
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn_append: dtype %d", dtype);
  if (batch > 0 && (!k_new || !v_new || !cow_src))
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_append: null new-token or copy-on-write pointer");
  if (!pkv::aligned16(k_new) || !pkv::aligned16(v_new))
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_append: k_new and v_new must be 16-byte aligned");
  if (plan && !plan->last_tokens_own)
    return fail(PKV_ERR_INVALID,
                "pkv_paged_decode_attn_append: the plan puts some row's last token in a shared node "
                "(build it from the tables after the append)");
  if (batch == 0) return PKV_OK;
  return decode_impl(dtype, q, batch, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, nullptr, nullptr,
                     num_blocks, block_size, block_tables, max_blocks_per_seq, seq_lens, max_seq_len, scale, plan,
                     workspace, workspace_bytes, out, status, stream, k_new, v_new, cow_src);
}

pkv_status pkv_paged_decode_attn_fp8(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t q_dtype, const void* k_pages, const void* v_pages,
                                     const float* k_scales, const float* v_scales, int64_t num_blocks,
                                     int32_t block_size, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len, float scale, const pkv_plan* plan,
                                     void* workspace, size_t workspace_bytes, float* out, int32_t* status,
                                     void* stream) {
  pkv::clear_error();
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn_fp8: q dtype %d", q_dtype);
  if (batch > 0 && (!k_scales || !v_scales)) return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_fp8: null scales");
  if ((reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) & 15u)
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_fp8: scales must be 16-byte aligned");
  return decode_impl(2 + q_dtype, q, batch, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, k_scales, v_scales,
                     num_blocks, block_size, block_tables, max_blocks_per_seq, seq_lens, max_seq_len, scale, plan,
                     workspace, workspace_bytes, out, status, stream);
}

pkv_status pkv_paged_decode_attn_noalloc(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t dtype, const void* k_pages, const void* v_pages,
                                         int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                         float scale, const pkv_plan* plan, float* out, int32_t* status,
                                         void* stream) {
  pkv::clear_error();
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_decode_attn_noalloc: dtype %d", dtype);
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_noalloc: invalid sizes");
  if (plan && (plan->kind != pkv_plan::kDecode || plan->batch != batch))
    return fail(PKV_ERR_INVALID, "pkv_paged_decode_attn_noalloc: plan not a decode plan for batch %d", batch);
  const size_t need = pkv::decode_layout(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, plan).bytes;
  if (need > pkv::kScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "pkv_paged_decode_attn_noalloc: these sizes need %zu bytes of scratch; the fixed scratch holds %zu "
                "(use pkv_paged_decode_attn with a workspace)",
                need, pkv::kScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = pkv::scratch_address(&scratch);
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "pkv_paged_decode_attn_noalloc: scratch address: %s", hipGetErrorString(e));
  return decode_impl(dtype, q, batch, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, nullptr, nullptr,
                     num_blocks, block_size, block_tables, max_blocks_per_seq, seq_lens, max_seq_len, scale, plan,
                     scratch, pkv::kScratchBytes, out, status, stream);
}

size_t pkv_extend_workspace_bytes(const pkv_plan* plan, int32_t head_dim) {
  pkv::clear_error();
  if (!plan || plan->kind != pkv_plan::kExtend || head_dim <= 0) {
    fail(PKV_ERR_INVALID, "pkv_extend_workspace_bytes: needs an extend plan and head_dim > 0");
    return 0;
  }
  const size_t recs = static_cast<size_t>(plan->num_query_rows) * std::max(plan->max_depth, 1) * plan->num_q_heads;
  const size_t ml_offset = (recs * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return ml_offset + recs * sizeof(float2);
}

namespace {

// kdtype: 0 f16, 1 bf16 pages; 2 / 3 FP8 pages with f16 / bf16 queries (scales given)
pkv_status extend_impl(int kdtype, const void* q, int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, const void* k_pages, const void* v_pages, const float* k_scales,
                       const float* v_scales, int64_t num_blocks, int32_t block_size, float scale,
                       const pkv_plan* plan, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  const int dtype = kdtype;
  if (!plan || plan->kind != pkv_plan::kExtend)
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: needs a plan from pkv_plan_build_extend");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || num_blocks < 0)
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: invalid head counts or pool size");
  if (plan->num_query_rows != num_query_rows || plan->num_q_heads != num_q_heads ||
      plan->num_kv_heads != num_kv_heads || plan->block_size != block_size)
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: plan was built for different shapes");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_extend_attn: head_dim %d (built: 64, 128)", head_dim);
  if (block_size != 16) return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_extend_attn: block_size %d (built: 16)", block_size);
  const int32_t group = num_q_heads / num_kv_heads;
  if (!pkv::supported_group(group))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_extend_attn: GQA group %d (built: 1, 2, 4, 8)", group);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: scale is not finite");
  if (!plan->device) return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: plan not uploaded (pkv_plan_upload)");
  if (num_query_rows == 0) return PKV_OK;
  if (num_blocks < 1) return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: the pool must hold at least one block");
  if (!q || !k_pages || !v_pages || !out) return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: null pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pages) || !pkv::aligned16(v_pages) || !pkv::aligned16(out))
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: q, pages and out must be 16-byte aligned");
  const size_t need = pkv_extend_workspace_bytes(plan, head_dim);
  if (workspace_bytes < need || !workspace)
    return fail(PKV_ERR_WORKSPACE, "pkv_paged_extend_attn: workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (!pkv::aligned16(workspace)) return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn: workspace must be 16-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t slots = std::max(plan->max_depth, 1);
  const size_t recs = static_cast<size_t>(num_query_rows) * slots * num_q_heads;
  float* acc = static_cast<float*>(workspace);
  float2* ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                         ((recs * head_dim * sizeof(float) + 255) & ~static_cast<size_t>(255)));
  const float scale_log2 = scale * 1.4426950408889634f;
  if (plan->num_items() > 0) {
    pkv::CascadeArgs c{};
    c.q = static_cast<const uint16_t*>(q);
    c.k_pages = static_cast<const uint16_t*>(k_pages);
    c.v_pages = static_cast<const uint16_t*>(v_pages);
    c.item_recs = plan->device + plan->off_item_recs;
    c.item_ints = plan->item_ints;
    c.node_blocks = plan->device + plan->off_blocks;
    c.acc = acc;
    c.ml = ml;
    c.num_blocks = num_blocks;
    c.num_items = plan->num_items();
    c.num_q_heads = num_q_heads;
    c.num_kv_heads = num_kv_heads;
    c.slots = slots;
    c.max_piece_blocks = plan->max_piece_blocks();
    c.scale_log2 = scale_log2;
    c.rows_per_item = plan->rows_per_item;
    c.k_scales = k_scales;
    c.v_scales = v_scales;
    c.status = nullptr;
    pkv_status st = pkv::launch(PKV_KERNEL_CASCADE, "cascade", s,
                                [&] { return pkv::launch_cascade(dtype, head_dim, group, c, s); });
    if (st != PKV_OK) return st;
  }
  pkv::MergeArgs ma{nullptr, plan->device + plan->off_row_info, nullptr, acc, ml, out, num_query_rows, num_q_heads,
                    num_kv_heads, 0, 0, slots, nullptr};
  return pkv::launch(PKV_KERNEL_MERGE, "merge", s, [&] { return pkv::launch_merge(head_dim, ma, s); });
}

}  // namespace

pkv_status pkv_paged_extend_attn(const void* q, int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, const void* k_pages, const void* v_pages,
                                 int64_t num_blocks, int32_t block_size, float scale, const pkv_plan* plan,
                                 void* workspace, size_t workspace_bytes, float* out, void* stream) {
  pkv::clear_error();
  if (dtype != PKV_F16 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_extend_attn: dtype %d", dtype);
  return extend_impl(dtype, q, num_query_rows, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, nullptr,
                     nullptr, num_blocks, block_size, scale, plan, workspace, workspace_bytes, out, stream);
}

pkv_status pkv_paged_extend_attn_fp8(const void* q, int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t q_dtype, const void* k_pages, const void* v_pages,
                                     const float* k_scales, const float* v_scales, int64_t num_blocks,
                                     int32_t block_size, float scale, const pkv_plan* plan, void* workspace,
                                     size_t workspace_bytes, float* out, void* stream) {
  pkv::clear_error();
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_paged_extend_attn_fp8: q dtype %d", q_dtype);
  if (num_query_rows > 0 && (!k_scales || !v_scales))
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn_fp8: null scales");
  if ((reinterpret_cast<uintptr_t>(k_scales) | reinterpret_cast<uintptr_t>(v_scales)) & 15u)
    return fail(PKV_ERR_INVALID, "pkv_paged_extend_attn_fp8: scales must be 16-byte aligned");
  return extend_impl(2 + q_dtype, q, num_query_rows, num_q_heads, num_kv_heads, head_dim, k_pages, v_pages, k_scales,
                     v_scales, num_blocks, block_size, scale, plan, workspace, workspace_bytes, out, stream);
}

pkv_status pkv_plan_upload(pkv_plan* plan, void* device_buf, size_t bytes, void* stream) {
  pkv::clear_error();
  if (!plan || !device_buf) return fail(PKV_ERR_INVALID, "pkv_plan_upload: null argument");
  const size_t need = plan->image.size() * sizeof(int32_t);
  if (bytes < need) return fail(PKV_ERR_INVALID, "pkv_plan_upload: buffer of %zu bytes, %zu needed", bytes, need);
  const hipError_t e = hipMemcpyAsync(device_buf, plan->image.data(), need, hipMemcpyHostToDevice,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_plan_upload: %s", hipGetErrorString(e));
  plan->device = static_cast<const int32_t*>(device_buf);
  return PKV_OK;
}

pkv_status pkv_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  pkv::clear_error();
  if (bytes < 0 || grid < 0 || (bytes > 0 && (!buf || !sink)))
    return fail(PKV_ERR_INVALID, "pkv_stream_read: invalid arguments");
  if (!pkv::aligned16(buf)) return fail(PKV_ERR_INVALID, "pkv_stream_read: buffer must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = pkv::launch_stream_read(buf, bytes, sink, grid > 0 ? grid : 2048, s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_stream_read: %s", hipGetErrorString(e));
  return PKV_OK;
}

namespace {

// Device address of a block array: device memory as is, pinned host memory through
// its device mapping; anything else (pageable host memory) is refused.
bool device_address(const void* p, const char** where, char** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    *where = "memory unknown to HIP (pageable host memory?)";
    return false;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = static_cast<char*>(const_cast<void*>(p));
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    // the mapping of the allocation's base; keep p's offset inside it
    const char* host_base = static_cast<const char*>(attr.hostPointer ? attr.hostPointer : p);
    *out = static_cast<char*>(attr.devicePointer) + (static_cast<const char*>(p) - host_base);
    return true;
  }
  *where = "host memory without a device mapping";
  return false;
}

}  // namespace

pkv_status pkv_copy_blocks(int32_t num_arrays, void* const* dst, const void* const* src, const int64_t* block_bytes,
                           int64_t dst_blocks, int64_t src_blocks, const int32_t* dst_ids, const int32_t* src_ids,
                           int32_t n, int32_t max_workgroups, void* stream) {
  pkv::clear_error();
  if (num_arrays < 1 || num_arrays > 4 || !dst || !src || !block_bytes || n < 0 || dst_blocks < 0 || src_blocks < 0 ||
      max_workgroups < 0)
    return fail(PKV_ERR_INVALID, "pkv_copy_blocks: invalid arguments (1..4 arrays, n >= 0)");
  if (n > 0 && (!dst_ids || !src_ids)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks: null id arrays");
  if (n == 0) return PKV_OK;
  pkv::CopyArgs a{};
  a.num_arrays = num_arrays;
  for (int32_t k = 0; k < num_arrays; ++k) {
    if (!dst[k] || !src[k] || block_bytes[k] <= 0 || block_bytes[k] % 16 != 0)
      return fail(PKV_ERR_INVALID, "pkv_copy_blocks: array %d: null pointer or block_bytes not a positive multiple of 16", k);
    if (!pkv::aligned16(dst[k]) || !pkv::aligned16(src[k]))
      return fail(PKV_ERR_INVALID, "pkv_copy_blocks: array %d is not 16-byte aligned", k);
    const char* why = nullptr;
    char* p = nullptr;
    if (!device_address(dst[k], &why, &p)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks: destination %d: %s", k, why);
    a.dst[k] = p;
    if (!device_address(src[k], &why, &p)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks: source %d: %s", k, why);
    a.src[k] = p;
    a.block_bytes[k] = block_bytes[k];
  }
  for (int32_t k = 0; k < 2; ++k) {  // id arrays are read by the kernel: device memory or pinned host memory
    const char* why = nullptr;
    char* p = nullptr;
    if (!device_address(k == 0 ? static_cast<const void*>(dst_ids) : static_cast<const void*>(src_ids), &why, &p))
      return fail(PKV_ERR_INVALID, "pkv_copy_blocks: %s ids: %s", k == 0 ? "destination" : "source", why);
    (k == 0 ? a.dst_ids : a.src_ids) = reinterpret_cast<const int32_t*>(p);
  }
  a.dst_blocks = dst_blocks;
  a.src_blocks = src_blocks;
  a.n = n;
  a.max_workgroups = max_workgroups;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return pkv::launch(PKV_KERNEL_COPY, "pkv_copy_blocks", s, [&] { return pkv::launch_copy_blocks(a, s); });
}

pkv_status pkv_copy_blocks_memcpy(int32_t num_arrays, void* const* dst, const void* const* src,
                               const int64_t* block_bytes, int64_t dst_blocks, int64_t src_blocks,
                               const int32_t* dst_ids, const int32_t* src_ids, int32_t n, void* stream) {
  pkv::clear_error();
  if (num_arrays < 1 || num_arrays > 4 || !dst || !src || !block_bytes || n < 0 || dst_blocks < 0 || src_blocks < 0)
    return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: invalid arguments (1..4 arrays, n >= 0)");
  if (n > 0 && (!dst_ids || !src_ids)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: null id arrays");
  for (int32_t i = 0; i < n; ++i)
    if (dst_ids[i] < 0 || dst_ids[i] >= dst_blocks || src_ids[i] < 0 || src_ids[i] >= src_blocks)
      return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: entry %d (%d <- %d) out of range", i, dst_ids[i], src_ids[i]);
  for (int32_t k = 0; k < num_arrays; ++k) {
    if (!dst[k] || !src[k] || block_bytes[k] <= 0)
      return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: array %d: null pointer or block_bytes <= 0", k);
    const char* why = nullptr;
    char* p = nullptr;
    if (!device_address(dst[k], &why, &p)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: destination %d: %s", k, why);
    if (!device_address(src[k], &why, &p)) return fail(PKV_ERR_INVALID, "pkv_copy_blocks_memcpy: source %d: %s", k, why);
  }
  if (n == 0) return PKV_OK;
  // runs of consecutive (dst, src) ids become one copy each
  std::vector<void*> dsts, srcs;
  std::vector<size_t> sizes;
  for (int32_t i = 0; i < n;) {
    int32_t r = 1;
    while (i + r < n && dst_ids[i + r] == dst_ids[i] + r && src_ids[i + r] == src_ids[i] + r) ++r;
    for (int32_t k = 0; k < num_arrays; ++k) {
      dsts.push_back(static_cast<char*>(dst[k]) + static_cast<int64_t>(dst_ids[i]) * block_bytes[k]);
      srcs.push_back(static_cast<char*>(const_cast<void*>(src[k])) + static_cast<int64_t>(src_ids[i]) * block_bytes[k]);
      sizes.push_back(static_cast<size_t>(r) * static_cast<size_t>(block_bytes[k]));
    }
    i += r;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return pkv::launch(PKV_KERNEL_COPY, "pkv_copy_blocks_memcpy", s, [&] {
    for (size_t c = 0; c < sizes.size(); ++c) {
      const hipError_t e = hipMemcpyAsync(dsts[c], srcs[c], sizes[c], hipMemcpyDefault, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

pkv_status pkv_timing_enable(int32_t on) {
  pkv::clear_error();
  auto& t = pkv::timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return PKV_OK;
}

pkv_status pkv_timing_reset(void) {
  pkv::clear_error();
  auto& t = pkv::timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& p : t.pending) {
    (void)hipEventSynchronize(p.stop);
    t.spare.push_back(p.start);
    t.spare.push_back(p.stop);
  }
  t.pending.clear();
  for (int k = 0; k < PKV_NUM_KERNELS; ++k) {
    t.total_ms[k] = 0;
    t.count[k] = 0;
  }
  return PKV_OK;
}

pkv_status pkv_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  pkv::clear_error();
  if (kernel < 0 || kernel >= PKV_NUM_KERNELS) return fail(PKV_ERR_INVALID, "pkv_timing_read: kernel id %d", kernel);
  auto& t = pkv::timing();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& p : t.pending) {
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_timing_read: %s", hipGetErrorString(e));
    t.total_ms[p.kernel] += ms;
    t.count[p.kernel] += 1;
    t.spare.push_back(p.start);
    t.spare.push_back(p.stop);
  }
  t.pending.clear();
  if (total_ms) *total_ms = t.total_ms[kernel];
  if (launches) *launches = t.count[kernel];
  return PKV_OK;
}

}  // extern "C"
