// Split-K paged decode attention, the partial-result merge, and the append /
// copy-on-write kernel, for gfx950 (wave64).
//
// Attention as defined in "The Reasoning Engine Meltdown", §2.1: the decode
// query of each row attends to all of the row's cached keys and values,
// softmax(scale * q K^T) V.  The cache is paged as in "Dismantling the Memory
// Wall", "PagedAttention: The Virtual Memory Analogy for GPUs": token t of a
// row is row t % 16 of physical block block_table[t / 16].  The softmax is
// evaluated online (running max m and sum l per query head, rescaled when the
// max grows) so a row's tokens can be split into independent chunks whose
// partials (m, l, acc) are merged exactly afterwards:
//   M = max_i m_i,  o = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
// Scores are kept in log2 units (scale * log2(e) folded into one multiply) so
// every exponential is a single v_exp_f32.
#include "device_common.h"
#include "launch.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Split-K partial attention.
//
// One wave per work unit (row b, KV head, chunk s of split_len tokens).  The
// group's G query heads share every K/V load.  Lanes are split into 64/LPT
// "token rows" of LPT lanes: each token row reads one token's K (and V) row of
// head_dim elements as LPT x (D/LPT) contiguous bytes with 16-byte loads, so a
// wave-wide load instruction covers 64/LPT whole tokens.  The q.k dot product
// is a per-lane dot2 chain plus a DPP sum over the LPT lanes; each token row
// keeps its own online-softmax state, and the token rows are merged once at
// the end of the unit with lane shuffles.  The next block's K/V loads are
// issued before the current block is consumed.
template <class DT, int D, int G, int LPT>
__global__ __launch_bounds__(64) void decode_split_kernel(SplitArgs a) {
  constexpr int ROWS = 64 / LPT;      // token rows per wave
  constexpr int VPL = D / (8 * LPT);  // 16-byte vectors per token per lane
  constexpr int TPB = 16 / ROWS;      // tokens per lane per 16-token block
  static_assert(VPL >= 1 && TPB >= 1 && ROWS * TPB == 16, "unsupported lane split");

  const int lane = threadIdx.x;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int Hkv = a.num_kv_heads;
  const int hkv = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % a.batch;
  const int s = rest / a.batch;

  int len = a.seq_lens[b];
  len = min(len, a.max_seq_len);
  len = min(len, a.max_blocks * 16);
  int begin = 0, depth = 0;
  if (a.row_info) {
    begin = a.row_info[2 * b];
    depth = a.row_info[2 * b + 1];
  }
  const int t0 = begin + s * a.split_len;  // multiple of 16
  if (t0 >= len) return;
  const int t1 = min(t0 + a.split_len, len);

  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;  // elements between consecutive tokens
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;

  // q of the G heads, restricted to this lane's dims: vector v holds dims (v*LPT + c)*8 .. +8
  u32x4 qv[G][VPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint16_t* qh = a.q + (static_cast<int64_t>(b) * a.num_q_heads + hkv * G + h) * D;
#pragma unroll
    for (int v = 0; v < VPL; ++v) qv[h][v] = ld16(qh + (v * LPT + c) * 8);
  }

  float m[G], l[G], acc[G][VPL * 8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VPL * 8; ++e) acc[h][e] = 0.f;
  }

  const int jb_first = t0 >> 4;
  const int jb_last = (t1 - 1) >> 4;

  u32x4 kc[TPB][VPL], vc[TPB][VPL];
  bool ok_c;
  auto load_block = [&](int jb, u32x4(&kk)[TPB][VPL], u32x4(&vv)[TPB][VPL]) -> bool {
    const int phys = bt[jb];
    const bool ok = phys >= 0 && static_cast<int64_t>(phys) < a.num_blocks;
    const int64_t base = ok ? (static_cast<int64_t>(phys) * 16) * tok_stride + static_cast<int64_t>(hkv) * D : 0;
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int64_t off = base + static_cast<int64_t>(r + i * ROWS) * tok_stride + (v * LPT + c) * 8;
        if (ok) {
          kk[i][v] = ld16(a.k_pages + off);
          vv[i][v] = ld16(a.v_pages + off);
        } else {
          kk[i][v] = u32x4{0, 0, 0, 0};
          vv[i][v] = u32x4{0, 0, 0, 0};
        }
      }
    }
    return ok;
  };

  ok_c = load_block(jb_first, kc, vc);
  for (int jb = jb_first; jb <= jb_last; ++jb) {
    u32x4 kn[TPB][VPL], vn[TPB][VPL];
    bool ok_n = false;
    if (jb < jb_last) ok_n = load_block(jb + 1, kn, vn);

    // scores of this lane's tokens for the G heads
    float sc[TPB][G];
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          x = DT::dot2(kc[i][v].x, qv[h][v].x, x);
          x = DT::dot2(kc[i][v].y, qv[h][v].y, x);
          x = DT::dot2(kc[i][v].z, qv[h][v].z, x);
          x = DT::dot2(kc[i][v].w, qv[h][v].w, x);
        }
        sc[i][h] = x;
      }
    }
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      const int tok = jb * 16 + r + i * ROWS;
      const bool valid = ok_c && tok < t1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float x = group_sum<LPT>(sc[i][h]) * a.scale_log2;
        sc[i][h] = valid ? x : kNegInf;
      }
    }

    // online softmax, per token row
    float mx[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = m[h];
#pragma unroll
      for (int i = 0; i < TPB; ++i) mx[h] = fmaxf(mx[h], sc[i][h]);
      grow |= mx[h] > m[h];
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = mx[h] > m[h] ? exp2_diff(m[h], mx[h]) : 1.f;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VPL * 8; ++e) acc[h][e] *= alpha;
        m[h] = mx[h];
      }
    }
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
      float vf[VPL * 8];
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        vf[v * 8 + 0] = DT::lo(vc[i][v].x);
        vf[v * 8 + 1] = DT::hi(vc[i][v].x);
        vf[v * 8 + 2] = DT::lo(vc[i][v].y);
        vf[v * 8 + 3] = DT::hi(vc[i][v].y);
        vf[v * 8 + 4] = DT::lo(vc[i][v].z);
        vf[v * 8 + 5] = DT::hi(vc[i][v].z);
        vf[v * 8 + 6] = DT::lo(vc[i][v].w);
        vf[v * 8 + 7] = DT::hi(vc[i][v].w);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = m[h] == kNegInf ? 0.f : fast_exp2(sc[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < VPL * 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }

    if (jb < jb_last) {
#pragma unroll
      for (int i = 0; i < TPB; ++i) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          kc[i][v] = kn[i][v];
          vc[i][v] = vn[i][v];
        }
      }
      ok_c = ok_n;
    }
  }

  // merge the token rows (lanes c, c+LPT, c+2LPT, ... hold the same dims)
#pragma unroll
  for (int dist = LPT; dist < 64; dist *= 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor_f32(m[h], dist);
      const float lo_ = shfl_xor_f32(l[h], dist);
      const float mn = fmaxf(m[h], mo);
      const float fa = exp2_diff(m[h], mn);
      const float fb = exp2_diff(mo, mn);
      l[h] = l[h] * fa + lo_ * fb;
#pragma unroll
      for (int e = 0; e < VPL * 8; ++e) {
        const float ao = shfl_xor_f32(acc[h][e], dist);
        acc[h][e] = acc[h][e] * fa + ao * fb;
      }
      m[h] = mn;
    }
  }

  if (r == 0) {
    const int slot = depth + s;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t rec = (static_cast<int64_t>(b) * a.slots + slot) * a.num_q_heads + hkv * G + h;
      float* dst = a.acc + rec * D;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        float4* d4 = reinterpret_cast<float4*>(dst + (v * LPT + c) * 8);
        d4[0] = make_float4(acc[h][v * 8 + 0], acc[h][v * 8 + 1], acc[h][v * 8 + 2], acc[h][v * 8 + 3]);
        d4[1] = make_float4(acc[h][v * 8 + 4], acc[h][v * 8 + 5], acc[h][v * 8 + 6], acc[h][v * 8 + 7]);
      }
      if (c == 0) a.ml[rec] = make_float2(m[h], l[h]);
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per (row, query head) combines the row's node partials and
// split partials; rows with no tokens get 0.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x % a.num_q_heads;
  const int b = blockIdx.x / a.num_q_heads;
  int len = a.seq_lens[b];
  len = min(len, a.max_seq_len);
  len = min(len, a.max_blocks * 16);
  int begin = 0, depth = 0;
  if (a.row_info) {
    begin = a.row_info[2 * b];
    depth = a.row_info[2 * b + 1];
  }
  const int nsplit = len > begin ? (len - begin + a.split_len - 1) / a.split_len : 0;
  const int np = min(depth + nsplit, a.slots);
  const int64_t rec0 = static_cast<int64_t>(b) * a.slots * a.num_q_heads + h;

  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ml[rec0 + static_cast<int64_t>(p) * a.num_q_heads].x);
  float L = 0.f;
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int p = 0; p < np; ++p) {
    const int64_t rec = rec0 + static_cast<int64_t>(p) * a.num_q_heads;
    const float2 ml = a.ml[rec];
    const float w = exp2_diff(ml.x, M);
    L = fmaf(w, ml.y, L);
    const float* src = a.acc + rec * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = fmaf(w, src[e], o[e]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* dst = a.out + (static_cast<int64_t>(b) * a.num_q_heads + h) * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) dst[e] = o[e] * inv;
}

// ---------------------------------------------------------------------------
// Append with copy-on-write, one launch.  Work-groups [0, num_cow) copy rows
// [0, rows) of a source block into a fresh block ("The Reasoning Engine
// Meltdown", §5: writes land only in pages the writer owns); the remaining
// work-groups write one new token each into its slot.  A plan from the host
// pool never lets a token write touch a row a copy reads or writes, so the two
// kinds of work-group do not race.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int64_t vec_per_row = a.row_elems / 8;  // 16-byte vectors per token row
  if (static_cast<int>(blockIdx.x) < a.num_cow) {
    const int cidx = blockIdx.x;
    const int src = a.cow_src[cidx], dst = a.cow_dst[cidx], rows = a.cow_rows[cidx];
    if (src < 0 || dst < 0 || static_cast<int64_t>(src) >= a.num_blocks || static_cast<int64_t>(dst) >= a.num_blocks ||
        rows <= 0 || rows > a.block_size)
      return;
    const int64_t n = static_cast<int64_t>(rows) * vec_per_row;
    const int64_t sbase = static_cast<int64_t>(src) * a.block_size * vec_per_row;
    const int64_t dbase = static_cast<int64_t>(dst) * a.block_size * vec_per_row;
    const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_pages);
    const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_pages);
    u32x4* kd = reinterpret_cast<u32x4*>(a.k_pages);
    u32x4* vd = reinterpret_cast<u32x4*>(a.v_pages);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      kd[dbase + i] = ks[sbase + i];
      vd[dbase + i] = vs[sbase + i];
    }
    return;
  }
  const int t = blockIdx.x - a.num_cow;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0 || slot >= a.num_blocks * a.block_size) return;
  const u32x4* kn = reinterpret_cast<const u32x4*>(a.k_new) + static_cast<int64_t>(t) * vec_per_row;
  const u32x4* vn = reinterpret_cast<const u32x4*>(a.v_new) + static_cast<int64_t>(t) * vec_per_row;
  u32x4* kd = reinterpret_cast<u32x4*>(a.k_pages) + slot * vec_per_row;
  u32x4* vd = reinterpret_cast<u32x4*>(a.v_pages) + slot * vec_per_row;
  for (int64_t i = threadIdx.x; i < vec_per_row; i += blockDim.x) {
    kd[i] = kn[i];
    vd[i] = vn[i];
  }
}

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(a.num_cow) + a.num_tokens;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

namespace {

template <class DT, int D, int G>
hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  constexpr int LPT = D == 128 ? 16 : 8;
  const int64_t grid = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.max_splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_split_kernel<DT, D, G, LPT>), dim3(static_cast<unsigned>(grid)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <class DT, int D>
hipError_t launch_split_g(int group, const SplitArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_split_t<DT, D, 1>(a, stream);
    case 2: return launch_split_t<DT, D, 2>(a, stream);
    case 4: return launch_split_t<DT, D, 4>(a, stream);
    case 8: return launch_split_t<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_split_d(int head_dim, int group, const SplitArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_split_g<DT, 64>(group, a, stream);
    case 128: return launch_split_g<DT, 128>(group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_split(int dtype, int head_dim, int group, const SplitArgs& a, hipStream_t stream) {
  return dtype == 1 ? launch_split_d<BF16>(head_dim, group, a, stream) : launch_split_d<F16>(head_dim, group, a, stream);
}

hipError_t launch_merge(int head_dim, const MergeArgs& a, hipStream_t stream) {
  const int64_t grid = static_cast<int64_t>(a.batch) * a.num_q_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(64), 0, stream, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
