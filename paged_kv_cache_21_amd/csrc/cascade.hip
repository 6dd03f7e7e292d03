// Shared-prefix ("cascade") decode pass on the gfx950 matrix cores.
//
// When many rows' block tables point at the same physical blocks — branches of
// one search tree forked from a common prefix ("The Reasoning Engine Meltdown",
// §5: children point at the parent's pages; "Dismantling the Memory Wall",
// "RadixAttention": one cached copy of a shared prefix serves every request
// that matches it) — the rows' queries against that prefix form a dense
// product: Q_n [rows x d] against K_n [tokens x d].  This pass reads each
// shared block once per KV head and work item and evaluates it for up to 64
// query rows at a time with MFMA:
//
//   S^T = K_n Q_n^T        (v_mfma_f32_16x16x32, K from LDS as the A operand,
//                           the queries held in registers as the B operand)
//   online softmax down each column of S^T (one column per query row)
//   O^T += V_n^T P^T       (V staged transposed in LDS as the A operand; P^T comes
//                           straight out of the S^T accumulator layout)
//
// For bf16 (and FP8) pages P is fed to the matrix core as two 16-bit terms,
// p = p_hi + p_lo, so the product keeps ~16 bits of the fp32 weights rather than 8;
// for f16 pages one f16 term (11 bits) is exact enough.
//
// Each (query row, query head) gets one partial (m, l, acc) per node piece, in
// the same log2-scaled form as the split-K partials, and the merge kernel
// combines them with the row's own remainder.
//
// The same kernel runs the multi-token (extend) pass: a query row is then one
// new token of a sequence, which may attend only to the tokens up to its own
// position (causal; "Dismantling the Memory Wall", "Chunked Prefill": a prompt
// is processed in slices, each slice's tokens attending to everything cached
// before them; the verification pass of "RKSC", §1: a generated branch is
// scored by one forward pass over its tokens).  Every member entry carries the
// last token position it may attend to; scores past it are masked, and the
// values of tokens past a node's valid length are zeroed.
#include <climits>

#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

}  // namespace

// One f16 weight term in the PV products of f16 pages (see the kernel): 1, or two
// 16-bit terms for every page type: 0.
#ifndef PKV_CASCADE_F16P
#define PKV_CASCADE_F16P 1
#endif

// Work-group: 4 waves, 64 x RB query rows (16 x RB per wave), one token piece of
// one node for one KV head.  Row rho of a node is (member rho / G, query head
// hkv*G + rho % G).  Tokens are processed in chunks of 32 (two blocks): the
// work-group stages K [32 x D] and V^T [D x 32] in LDS, each wave evaluates its
// 16 rows.  Pipeline: two LDS buffers and a two-chunk register ring, so chunk
// c is evaluated while chunk c+1 is written to the other LDS buffer and chunks
// c+2, c+3 are in flight from memory; one barrier per chunk.
//
// MFMA 16x16x32 operand layout used (lane l, element j of 8): A row l % 16,
// k = 8*(l / 16) + j; B column l % 16, same k; accumulator element j of lane l
// is (row 4*(l / 16) + j, column l % 16).  A contraction index may be permuted
// freely as long as A and B agree; the PV product uses the token order the S^T
// accumulator leaves in each lane.
// NW: 64-block windows of block ids held per lane (1 when every piece of the plan
// has at most 64 blocks; up to kCascadeMaxPieceBlocks / 64 otherwise).
// RB: 16-row blocks per wave (64 * RB rows per work item).  Each K / V^T operand
// read from LDS then feeds RB products; the registers it costs lower the
// occupancy (3 waves per SIMD at RB = 1, 2 at RB = 2).
template <class DT, int D, int G, int NW, int RB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 3 : RB == 2 ? 2 : 1))) void
cascade_kernel(CascadeArgs a) {
  // FP8 pages: E4M3 codes widened to the 16-bit type of q on their way into LDS
  // (exact), the per-token K scale applied to each score and the V scale folded
  // into each weight
  using CT = typename is_fp8<DT>::compute;
  constexpr bool Q8 = is_fp8<DT>::value;
  constexpr int EB = Q8 ? 1 : 2;  // bytes per page element
  typedef typename std::conditional<Q8, u32x2, u32x4>::type KV;  // 8 page elements
  constexpr int KPITCH = D + 8;   // K row pitch in LDS (elements); the pad spreads rows over banks
  constexpr int VPITCH = D + 16;  // V row pitch (elements): the transpose reads of a half-wave
                                  // (8 rows x 32 bytes) then land in distinct banks
  constexpr int NKS = D / 32;    // k-steps of the QK product
  constexpr int NDT = D / 16;    // 16-wide d tiles of the PV product
  constexpr int KVEC = 32 * D / 8;             // 16-byte vectors per K chunk
  constexpr int KVEC_PER_THREAD = KVEC / 256;  // 1 (D=64) or 2 (D=128)
  static_assert(KVEC_PER_THREAD >= 1, "unsupported head_dim");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][32 * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][32 * VPITCH];
  // f16 pages: the weights enter the PV products as one f16 term (11 significant bits,
  // exact enough); bf16 and FP8 pages as two 16-bit terms.  (Staging bf16 V a second
  // time as f16 for one term, with the two-term path kept for chunks beyond the f16
  // range, measured much slower: the copy and the registers cost more than the products.)
  constexpr bool P16 = PKV_CASCADE_F16P != 0 && !Q8 && std::is_same<CT, F16>::value;
  // FP8: the chunk's 32 K scales, then its 32 V scales (zero for tokens without data)
  __shared__ __attribute__((aligned(16))) float sc_lds[2][Q8 ? 64 : 1];

  // The work item's record holds everything needed before the first K/V loads (the
  // piece's first block ids, its member rows), so they issue one read after launch.
  // The header is read through the constant address space (scalar loads: the record is
  // never written while the kernel runs).  An idle item has no blocks and no member rows.
  typedef const int32_t __attribute__((address_space(4))) const_i32;
  const int item = blockIdx.x;
  const int32_t* irec = a.item_recs + static_cast<int64_t>(item) * a.item_ints;
  const_i32* hrec = (const_i32*)(irec);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 15;  // MFMA row / column index
  const int lgrp = lane >> 4;  // MFMA k group
  // this lane's member entries, one per row block (query row -1 past the node's members):
  // at a fixed place in the record, so they load alongside the header
  int my_b[RB], my_slot[RB], my_limit_raw[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int32_t* mrec = irec + kItemHeadInts + kItemMemberInts * ((wave * 16 * RB + rb * 16 + lrow) / G);
    my_b[rb] = mrec[0];
    my_slot[rb] = mrec[1];
    my_limit_raw[rb] = mrec[2];
  }
  const int hkv = max(hrec[0], 0);  // -1 (idle item) reads as head 0
  const int row0 = hrec[1];
  const int blk_start = hrec[3];  // the piece's first id in node_blocks
  const int nblk = hrec[4];
  const int R = hrec[5];
  const int piece_tok0 = hrec[6];   // logical position of the piece's first token
  const int piece_valid = hrec[7];  // tokens of the piece holding data (may exceed the piece)
  const int Hkv = a.num_kv_heads;
  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;

  const bool wave_active = row0 + wave * 16 * RB < R;

  // K and V take the same thread mapping: vector i of thread tid is token
  // (tid + 256 i) / (D / 8) of the chunk, 8-element column (tid + 256 i) % (D / 8)
  struct Stage {
    KV k[KVEC_PER_THREAD];
    KV v[KVEC_PER_THREAD];
    f32x4 sc;  // FP8, threads 0..15: four scales of the chunk
  };
  const int nchunks = (nblk + 1) / 2;
  // Per-thread element offsets inside a block (32-bit: a block is 16 * Hkv * D
  // elements); per chunk only the two block bases change, and those are uniform.
  const int64_t blk_stride = 16 * tok_stride;
  uint32_t koff[KVEC_PER_THREAD];  // bytes
  // token in the chunk's second block: the same for a whole wave (a wave's 64 vectors
  // cover 512 / D consecutive tokens of one block), so each load takes one block base
  // for the wave and a 32-bit offset per lane
  bool khi[KVEC_PER_THREAD];
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int i = 0; i < KVEC_PER_THREAD; ++i) {
    const int vi = tid + 256 * i;
    const int tok = vi / (D / 8);
    const int col = vi % (D / 8);
    koff[i] = static_cast<uint32_t>(((tok & 15) * tok_stride + static_cast<int64_t>(hkv) * D + col * 8) * EB);
    khi[i] = (64 * wave_u + 256 * i) / (D / 8) >= 16;
  }
  // global -> registers (cached loads: the other row tiles of this piece read the
  // same K/V from L2); past the last chunk the last one is read again (an L2 hit)
  auto load_ids = [&](int id0, int id1, Stage& st) {
    const int64_t b0 = static_cast<int64_t>(id0 < 0 ? 0 : id0) * blk_stride * EB;  // bytes
    const int64_t b1 = static_cast<int64_t>(id1 < 0 ? 0 : id1) * blk_stride * EB;
    const char* kbase = reinterpret_cast<const char*>(a.k_pages);
    const char* vbase = reinterpret_cast<const char*>(a.v_pages);
    // the block bases go to scalar registers as they are, so each load is one scalar base
    // plus the lane's 32-bit offset (no 64-bit address arithmetic per lane)
    typedef const char __attribute__((address_space(1))) gchar;
    auto sbase = [](const char* p) {
      const uint64_t u = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
      return (gchar*)((static_cast<uint64_t>(hi) << 32) | lo);  // global address space
    };
    typedef const KV __attribute__((address_space(1))) gKV;
#pragma unroll
    for (int i = 0; i < KVEC_PER_THREAD; ++i) {
      gchar* kb = sbase(kbase + (khi[i] ? b1 : b0));
      gchar* vb = sbase(vbase + (khi[i] ? b1 : b0));
      st.k[i] = *(gKV*)(kb + koff[i]);
      st.v[i] = *(gKV*)(vb + koff[i]);
    }
    if constexpr (Q8) {
      if (tid < 16) {  // (K | V) x (block 0 | 1) x rows 4 p .. 4 p + 3
        const int which = tid >> 2, part = tid & 3;
        const int id = (which & 1) ? id1 : id0;
        const float* sb = which < 2 ? a.k_scales : a.v_scales;
        st.sc = *reinterpret_cast<const f32x4*>(sb + (static_cast<int64_t>(id < 0 ? 0 : id) * Hkv + hkv) * 16 + 4 * part);
      }
    }
  };
  // The first two chunks' K/V loads go out as soon as the header is in (an idle item
  // reads block 0 and discards it), then the queries and the piece's block-id window;
  // nothing waits for them before the first chunk is staged.
  Stage s0, s1;
  {
    int fid[kItemFirstIds];  // the record's copy of the piece's first ids, checked as the window's are
#pragma unroll
    for (int j = 0; j < kItemFirstIds; ++j) {
      const int id = hrec[8 + j];
      fid[j] = id >= 0 && static_cast<int64_t>(id) < a.num_blocks ? id : -1;
    }
    const bool two = nchunks > 1;  // else chunk 1 is chunk 0 again, as load_chunk would read it
    load_ids(fid[0], fid[1], s0);
    load_ids(two ? fid[2] : fid[0], two ? fid[3] : fid[1], s1);
  }

  // queries of this lane's rows (one per row block), as B operands: loaded for every lane
  // (a lane past the node's rows reads its item's row 0 of q) and made final (zeroed past
  // the rows, sign-flipped for a negative scale) after the first chunk is staged
  u32x4 qb[RB][NKS];
  int my_h[RB];
  int my_limit[RB];  // last attended position, piece-local (rows past R attend to nothing)
  int wave_min_limit = INT_MAX;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bool in = my_b[rb] >= 0;  // the lane's row rb is one of the node's rows
    const int limit = my_limit_raw[rb];
    my_limit[rb] = !in ? -1 : limit == INT_MAX ? INT_MAX : limit - piece_tok0;
    my_h[rb] = hkv * G + (wave * 16 * RB + rb * 16 + lrow) % G;  // tile rows start at a multiple of G
    const uint16_t* qp = a.q + (static_cast<int64_t>(in ? my_b[rb] : 0) * a.num_q_heads + my_h[rb]) * D + lgrp * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qb[rb][ks] = ld16(qp + ks * 32);
    if (in) wave_min_limit = min(wave_min_limit, my_limit[rb]);
  }
  // the earliest last-attended position over the wave's rows (rows past R count as
  // unlimited: their results are never stored); chunks entirely at or before it
  // need no causal mask
  wave_min_limit = min(wave_min_limit, __shfl_xor(wave_min_limit, 1));
  wave_min_limit = min(wave_min_limit, __shfl_xor(wave_min_limit, 2));
  wave_min_limit = min(wave_min_limit, __shfl_xor(wave_min_limit, 4));
  wave_min_limit = min(wave_min_limit, __shfl_xor(wave_min_limit, 8));
  wave_min_limit = __builtin_amdgcn_readfirstlane(wave_min_limit);

  float m[RB], lsum[RB];
  f32x4 o[RB][NDT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    lsum[rb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the piece's block ids, lane j of register w holding block 64 w + j (a piece has
  // at most 64 NW blocks), -1 past the piece's end and for an id outside the pool; read
  // with readlane so the chunk loop issues no scalar memory loads, which would share a
  // wait counter with the LDS reads
  int blk_win[NW];
  int first_bad = nblk;  // the piece's first block with an id outside the pool (uniform)
#pragma unroll
  for (int w4 = 0; w4 < NW; ++w4) {
    const int j = 64 * w4 + lane;
    const int id = j < nblk ? a.node_blocks[blk_start + j] : -1;
    const bool bad = j < nblk && !(id >= 0 && static_cast<int64_t>(id) < a.num_blocks);
    blk_win[w4] = bad ? -1 : id;
    const uint64_t badm = __ballot(bad);
    if (badm != 0 && first_bad == nblk) first_bad = 64 * w4 + __builtin_ctzll(badm);
  }
  // an entry that names a block outside the pool is reported (its tokens get no weight)
  if (first_bad < nblk && a.status && tid == 0)
    __hip_atomic_fetch_or(a.status, PKV_STATUS_BAD_BLOCK, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto block_id = [&](int j) -> int {  // j: block within the piece (uniform, < 64 NW); -1: none
    int v = blk_win[0];
#pragma unroll
    for (int w4 = 1; w4 < NW; ++w4) v = (j >> 6) == w4 ? blk_win[w4] : v;
    return __builtin_amdgcn_readlane(v, j & 63);
  };
  // Chunks [0, clean_store) are whole, readable and inside the node's filled tokens: their
  // K/V go to LDS unmasked.  Chunks [0, clean_wave) also lie at or before every one of the
  // wave's rows' last attended positions: their scores need no mask.  Both uniform.
  const int clean_store = min(min(first_bad, nblk) / 2, piece_valid < 0 ? 0 : piece_valid / 32);
  const int clean_wave =
      wave_min_limit == INT_MAX ? clean_store : min(clean_store, wave_min_limit < 0 ? 0 : (wave_min_limit + 1) / 32);

  auto load_chunk = [&](int ch, Stage& st) {
    ch = min(ch, nchunks - 1);
    load_ids(block_id(2 * ch), block_id(2 * ch + 1), st);
  };
  // registers -> LDS buffer, K and V token-major as in the pages; K and V of tokens
  // without data (past the node's valid length, or in a block with a bad id) are
  // zeroed, so stale Inf / NaN bits meet neither a score's -inf bias nor a zero weight
  auto store_chunk = [&](const Stage& st_in, int ch, int buf) {
    Stage st = st_in;
    // block_id reads a lane of a register: its argument must be wave-uniform
    const bool ok0 = block_id(2 * ch) >= 0, ok1 = block_id(2 * ch + 1) >= 0;
    if (ch >= clean_store) {  // uniform
#pragma unroll
      for (int i = 0; i < KVEC_PER_THREAD; ++i) {
        const int tok = (tid + 256 * i) / (D / 8);
        const bool blk_ok = khi[i] ? ok1 : ok0;
        if (!(blk_ok && ch * 32 + tok < piece_valid)) st.k[i] = st.v[i] = KV{};
      }
    }
    if constexpr (Q8) {
      if (tid < 16) {
        const int which = tid >> 2, part = tid & 3;
        const bool blk_ok = (which & 1) ? ok1 : ok0;
        const int t0 = ch * 32 + (which & 1) * 16 + 4 * part;
        f32x4 v = st.sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (blk_ok && t0 + e < piece_valid) ? v[e] : 0.f;
        *reinterpret_cast<f32x4*>(&sc_lds[buf][(which >> 1) * 32 + (which & 1) * 16 + 4 * part]) = v;
      }
    }
#pragma unroll
    for (int i = 0; i < KVEC_PER_THREAD; ++i) {
      const int vi = tid + 256 * i;
      const int tok = vi / (D / 8);
      const int col = vi % (D / 8);
      u32x4 kw;
      if constexpr (Q8)
        kw = widen8<CT>(st.k[i]);
      else
        kw = st.k[i];
      *reinterpret_cast<u32x4*>(&k_lds[buf][tok * KPITCH + col * 8]) = kw;
    }
#pragma unroll
    for (int i = 0; i < KVEC_PER_THREAD; ++i) {
      const int vi = tid + 256 * i;
      const int tok = vi / (D / 8);
      const int col = vi % (D / 8);
      u32x4 vw;
      if constexpr (Q8)
        vw = widen8<CT>(st.v[i]);
      else
        vw = st.v[i];
      *reinterpret_cast<u32x4*>(&v_lds[buf][tok * VPITCH + col * 8]) = vw;
    }
  };
  // evaluate chunk ch from LDS buffer buf for this wave's RB x 16 rows
  auto compute_chunk = [&](int ch, int buf) {
    if (!wave_active) return;
    // Every LDS operand of the chunk is requested up front, K first, then V^T: the
    // reads' latencies overlap one another, the V^T reads complete under the QK
    // products and the softmax, and no matrix instruction waits on a read issued just
    // before it.
    // (With one row block per wave the registers this takes would cost a resident
    // wave per SIMD, so that instance reads each operand where it is used.)
    constexpr bool BATCH = RB >= 2;
    u32x4 kop[NKS][2], vop[NDT];
    const uint16_t* vsrc = &v_lds[buf][0];
    auto k_operand = [&](int ks, int tt) {
      return *reinterpret_cast<const u32x4*>(&k_lds[buf][(tt * 16 + lrow) * KPITCH + ks * 32 + lgrp * 8]);
    };
    const int trow = lrow >> 2, tcol = 4 * (lrow & 3);
    auto v_operand = [&](int dt) {
      const uint16_t* v0p = vsrc + (4 * lgrp + trow) * VPITCH + dt * 16 + tcol;
      const u32x2 t0 = tr_read16(v0p);                // tokens 4*lgrp .. +3
      const u32x2 t1 = tr_read16(v0p + 16 * VPITCH);  // tokens 16 + 4*lgrp .. +3
      return u32x4{t0.x, t0.y, t1.x, t1.y};
    };
    if constexpr (BATCH) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) kop[ks][tt] = k_operand(ks, tt);
    }
    // V^T operands by transpose reads of the token-major V: in each 16-lane group, the
    // lane 4 j + q supplies the address of token row tok_j, columns 4 q .. 4 q + 3 of
    // the d tile, and lane 4 q + e receives column 4 q + e of rows tok_0 .. tok_3, i.e.
    // its own d (the MFMA row) for four consecutive tokens.  Group g's k slots hold
    // tokens 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, the order the weights leave
    // the S^T accumulator in.
    if constexpr (BATCH) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vop[dt] = v_operand(dt);
    }
    // S^T tiles: st[rb][tt][j] = score of token 16*tt + 4*lgrp + j for this lane's row of
    // block rb; each K operand read from LDS feeds RB products
    f32x4 st[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st[rb][0] = st[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const u32x4 kv = BATCH ? kop[ks][tt] : k_operand(ks, tt);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) st[rb][tt] = mfma16x16x32<CT>(kv, qb[rb][ks], st[rb][tt]);
      }
    }
    float vsc[8];  // FP8: this lane's tokens' V scales; the K scales go onto the scores here
    if constexpr (Q8) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 kq = *reinterpret_cast<const f32x4*>(&sc_lds[buf][16 * tt + 4 * lgrp]);
        const f32x4 vq = *reinterpret_cast<const f32x4*>(&sc_lds[buf][32 + 16 * tt + 4 * lgrp]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) st[rb][tt][j] *= kq[j];
          vsc[4 * tt + j] = vq[j];
        }
      }
    }
    // Scores that must not count (a piece's odd end, bad ids, the node's partly filled
    // end, a row's last attended position) become -inf, in place (uniform branch; K is
    // zeroed where there is no data, so no stale bits are in play).
    if (ch >= clean_wave) {
      const bool valid0 = block_id(2 * ch) >= 0;
      const bool valid1 = block_id(2 * ch + 1) >= 0;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = ch * 32 + 16 * tt + 4 * lgrp + j;  // piece-local token
            const bool ok = (tt ? valid1 : valid0) && t <= my_limit[rb] && t < piece_valid;
            st[rb][tt][j] = ok ? st[rb][tt][j] : kNegInf;
          }
    }
    // c > 0, so a masked (-inf) score gives exp2(-inf) = 0 with no test per score
    const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
    u32x4 bh[RB], bl[RB];
    // max(x, y) as med3(x, y, +inf), with +inf opaque to the compiler so the median is
    // not turned back into a max that first quiets NaNs in both operands
    float pinf = __builtin_inff();
    asm volatile("" : "+v"(pinf));
    auto max2 = [pinf](float x, float y) { return __builtin_amdgcn_fmed3f(x, y, pinf); };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sv[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = st[rb][0][j];
        sv[4 + j] = st[rb][1][j];
      }
      // this lane's largest score of the chunk, in log2 units
      const float lmax =
          max2(max2(max2(sv[0], sv[1]), max2(sv[2], sv[3])), max2(max2(sv[4], sv[5]), max2(sv[6], sv[7]))) * c;
      // Rescale only when some score outgrows its row's running max by more than 2^8:
      // until then the weights 2^(s - m) stay <= 256, harmless in fp32 and in the 16-bit
      // terms.  The row's max over its four lane groups is needed only then, so the
      // cross-lane reduction stays on that (rare) path.
      if (__any(lmax > m[rb] + 8.f)) {
        float cm = xor_max<16>(lmax);
        cm = xor_max<32>(cm);  // the chunk max of the lane's row
        const float mn = fmaxf(m[rb], cm);
        const float alpha = exp2_diff(m[rb], mn);
        lsum[rb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[rb][dt] *= alpha;
        m[rb] = mn;
      }
      const float mref = fmaxf(m[rb], -3.0e38f);  // m = -inf only while every score is -inf
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        float p0 = fast_exp2(fmaf(sv[2 * j2], c, -mref));
        float p1 = fast_exp2(fmaf(sv[2 * j2 + 1], c, -mref));
        lsum[rb] += p0 + p1;
        if constexpr (Q8) {  // the V scale rides on the weight
          p0 = CT::finite_weight(p0 * vsc[2 * j2]);
          p1 = CT::finite_weight(p1 * vsc[2 * j2 + 1]);
        }
        if constexpr (P16) {  // one f16 term
          bh[rb][j2] = F16::pack2(p0, p1);
        } else {
          const uint32_t h = CT::pack2(p0, p1);  // the 16-bit terms, then what they leave
          bh[rb][j2] = h;
          bl[rb][j2] = CT::pack2(p0 - CT::lo(h), p1 - CT::hi(h));
        }
      }
    }
    // each V^T operand read from LDS feeds 2 x RB products
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 av = BATCH ? vop[dt] : v_operand(dt);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (P16) {
          o[rb][dt] = mfma16x16x32<F16>(av, bh[rb], o[rb][dt]);
        } else {
          o[rb][dt] = mfma16x16x32<CT>(av, bh[rb], o[rb][dt]);
          o[rb][dt] = mfma16x16x32<CT>(av, bl[rb], o[rb][dt]);
        }
      }
    }
  };

  if (nchunks > 0) {
    store_chunk(s0, 0, 0);
    load_chunk(2, s0);
    __syncthreads();
    // a negative scale is applied as |scale| on -q (flipping sign bits is exact), so the
    // running max can be taken on the unscaled scores; lanes past the node's rows get q = 0
    const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qb[rb][ks] = my_b[rb] >= 0 ? qb[rb][ks] ^ flip : u32x4{0, 0, 0, 0};
    for (int ch = 0; ch < nchunks; ch += 2) {
      compute_chunk(ch, 0);
      store_chunk(s1, ch + 1, 1);
      load_chunk(ch + 3, s1);
      __syncthreads();
      if (ch + 1 >= nchunks) break;
      compute_chunk(ch + 1, 1);
      store_chunk(s0, ch + 2, 0);
      load_chunk(ch + 4, s0);
      __syncthreads();
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // every lane group holds part of the row's weight sum
    float lo, hi;
    pair_values<16>(lsum[rb], lo, hi);
    float ls = lo + hi;
    pair_values<32>(ls, lo, hi);
    ls = lo + hi;
    if (my_b[rb] >= 0) {
      const int64_t rec = (static_cast<int64_t>(my_b[rb]) * a.slots + my_slot[rb]) * a.num_q_heads + my_h[rb];
      float* dst = a.acc + rec * D + lgrp * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<float4*>(dst + dt * 16) = make_float4(o[rb][dt][0], o[rb][dt][1], o[rb][dt][2], o[rb][dt][3]);
      if (lgrp == 0) a.ml[rec] = make_float2(m[rb], ls);
    }
  }
}

namespace {

template <class DT, int D, int G, int RB>
hipError_t launch_cascade_rb(const CascadeArgs& a, hipStream_t stream) {
  if (a.max_piece_blocks <= 64)
    hipLaunchKernelGGL((cascade_kernel<DT, D, G, 1, RB>), dim3(static_cast<unsigned>(a.num_items)), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((cascade_kernel<DT, D, G, kCascadeMaxPieceBlocks / 64, RB>),
                       dim3(static_cast<unsigned>(a.num_items)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class DT, int D, int G>
hipError_t launch_cascade_t(const CascadeArgs& a, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  if (a.max_piece_blocks > kCascadeMaxPieceBlocks) return hipErrorInvalidValue;
  if (a.rows_per_item == 64) return launch_cascade_rb<DT, D, G, 1>(a, stream);
  if (a.rows_per_item == 128) return launch_cascade_rb<DT, D, G, 2>(a, stream);
  if (a.rows_per_item == 256) return launch_cascade_rb<DT, D, G, 4>(a, stream);
  return hipErrorInvalidValue;
}

template <class DT, int D>
hipError_t launch_cascade_g(int group, const CascadeArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_cascade_t<DT, D, 1>(a, stream);
    case 2: return launch_cascade_t<DT, D, 2>(a, stream);
    case 4: return launch_cascade_t<DT, D, 4>(a, stream);
    case 8: return launch_cascade_t<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_cascade_d(int head_dim, int group, const CascadeArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_cascade_g<DT, 64>(group, a, stream);
    case 128: return launch_cascade_g<DT, 128>(group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_cascade(int dtype, int head_dim, int group, const CascadeArgs& a, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_cascade_d<F16>(head_dim, group, a, stream);
    case 1: return launch_cascade_d<BF16>(head_dim, group, a, stream);
    case 2: return launch_cascade_d<FP8<F16>>(head_dim, group, a, stream);
    case 3: return launch_cascade_d<FP8<BF16>>(head_dim, group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
