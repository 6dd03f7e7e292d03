// Device helpers for the gfx950 kernels: 16-bit float formats, wave64 lane
// exchanges, the partial-result layout shared by the decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// 16-bit storage formats.  A 32-bit word holds two consecutive elements, the
// lower-addressed one in the low half.

struct BF16 {
  typedef bf16x8 vec8;
  // low / high element of a packed pair as fp32 (bf16 is the top half of an fp32)
  static __device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
  // acc + a.lo*b.lo + a.hi*b.hi (products of two bf16 values are exact in fp32)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                           false);
  }
  // round-to-nearest-even fp32 -> 16-bit pattern
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  static __device__ __forceinline__ float to_float(uint16_t h) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
  }
  // two fp32 values -> one packed pair (a low), round-to-nearest-even
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  }
  // a non-negative weight that must stay finite when packed (bf16 has fp32's range)
  static __device__ __forceinline__ float finite_weight(float x) { return x; }
};

struct F16 {
  typedef f16x8 vec8;
  static __device__ __forceinline__ float lo(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(f16x2, w).x);
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(f16x2, w).y);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  static __device__ __forceinline__ float to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
  // a non-negative weight that must stay finite when packed: at most the largest
  // finite f16 (a weight <= 2^8 times an FP8 V scale <= 2^8 can reach 2^16)
  static __device__ __forceinline__ float finite_weight(float x) { return fminf(x, 65504.f); }
};

// FP8 pages: OCP E4M3 codes, one byte per element, with a power-of-two scale per
// (block, KV head, token row); q and the arithmetic use the 16-bit type CT.
// Every E4M3 value is exact in bf16 and in f16, so a code widens to CT exactly
// (through the hardware's E4M3 -> fp32 conversion).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class CT>
struct FP8 {
  typedef CT compute;
};

template <class T>
struct is_fp8 {
  static constexpr bool value = false;
  typedef T compute;
};
template <class CT>
struct is_fp8<FP8<CT>> {
  static constexpr bool value = true;
  typedef CT compute;
};

// Two E4M3 codes (byte pair 0,1 or 2,3 of a word) converted to fp32.  Consumers
// take the floats as returned: bit-casting one element of the pair was miscompiled
// (element 1 read as element 0) in both directions we tried.
template <bool HIGH>
__device__ __forceinline__ f32x2 fp8_pair_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HIGH);
}

// four E4M3 codes (one word) -> two words of CT pairs (codes 0,1 and 2,3)
template <class CT>
__device__ __forceinline__ void widen4(uint32_t w, uint32_t& lo, uint32_t& hi);

// gfx950 converts a pair of codes straight to a 16-bit pair (times a scale, here 1:
// every E4M3 value is exact in bf16 and in f16, so the conversion is exact)
template <>
__device__ __forceinline__ void widen4<BF16>(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

template <>
__device__ __forceinline__ void widen4<F16>(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// eight E4M3 codes -> eight CT values packed as in a 16-bit page vector
template <class CT>
__device__ __forceinline__ u32x4 widen8(u32x2 w) {
  uint32_t a, b, c, d;
  widen4<CT>(w.x, a, b);
  widen4<CT>(w.y, c, d);
  return u32x4{a, b, c, d};
}

// eight E4M3 codes -> eight fp32 values
__device__ __forceinline__ void fp8x8_to_f32(u32x2 w, float* out) {
  const f32x2 p0 = fp8_pair_f32<false>(w.x), p1 = fp8_pair_f32<true>(w.x);
  const f32x2 p2 = fp8_pair_f32<false>(w.y), p3 = fp8_pair_f32<true>(w.y);
  out[0] = p0.x;
  out[1] = p0.y;
  out[2] = p1.x;
  out[3] = p1.y;
  out[4] = p2.x;
  out[5] = p2.y;
  out[6] = p3.x;
  out[7] = p3.y;
}

// ---------------------------------------------------------------------------
// Lane exchanges inside a wave64.

// DPP move with the given control (row_mask/bank_mask all lanes, bound_ctrl on).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each 16
constexpr int kDppRowRor4 = 0x124;        // lane i <- lane (i - 4) mod 16 within each 16
constexpr int kDppRowRor8 = 0x128;        // lane i <- lane i ^ 8 within each 16
constexpr int kDppRowNewBcast = 0x150;    // + k: every lane of a 16-lane row <- lane k of that row

// Lane k of each 16-lane row, broadcast to the row (k must be a compile-time value
// after unrolling).
__device__ __forceinline__ float row_bcast_f32(float x, int k) {
  switch (k & 15) {
#define PKV_BCAST_CASE(n) \
  case n:                 \
    return dpp_f32<kDppRowNewBcast + n>(x);
    PKV_BCAST_CASE(0) PKV_BCAST_CASE(1) PKV_BCAST_CASE(2) PKV_BCAST_CASE(3)
    PKV_BCAST_CASE(4) PKV_BCAST_CASE(5) PKV_BCAST_CASE(6) PKV_BCAST_CASE(7)
    PKV_BCAST_CASE(8) PKV_BCAST_CASE(9) PKV_BCAST_CASE(10) PKV_BCAST_CASE(11)
    PKV_BCAST_CASE(12) PKV_BCAST_CASE(13) PKV_BCAST_CASE(14) PKV_BCAST_CASE(15)
#undef PKV_BCAST_CASE
  }
  return x;
}

// Sum over groups of N consecutive lanes (N in 1, 2, 4, 8, 16); every lane of a
// group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppRowMirror>(x);
  return x;
}

// The values of lane l and lane l ^ DIST (DIST = 8, 16 or 32) as (lower lane's,
// upper lane's), in both lanes, without LDS: DPP for 8 (within a 16-lane row),
// v_permlane16_swap / v_permlane32_swap for 16 / 32.
template <int DIST>
__device__ __forceinline__ void pair_values(float x, float& lo, float& hi) {
  static_assert(DIST == 8 || DIST == 16 || DIST == 32, "pair distance");
  if constexpr (DIST == 8) {
    const float other = dpp_f32<kDppRowRor8>(x);
    const bool upper = __lane_id() & 8;
    lo = upper ? other : x;
    hi = upper ? x : other;
  } else {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = DIST == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                              : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
    hi = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
  }
}

// max(x of lane l, x of lane l ^ DIST), in both lanes (DIST = 8, 16 or 32).
template <int DIST>
__device__ __forceinline__ float xor_max(float x) {
  float lo, hi;
  pair_values<DIST>(x, lo, hi);
  return fmaxf(lo, hi);
}

// Max over groups of N consecutive lanes (N in 1, 2, 4, 8, 16).
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(a - b) with exp2(-inf - anything) = 0 (an empty running state has m = -inf)
__device__ __forceinline__ float exp2_diff(float a, float b) { return a == kNegInf ? 0.f : fast_exp2(a - b); }

// Matrix-core product D = A B + C on a 16 x 16 tile with k = 32 (lane l, element j of
// 8: A row l % 16, k = 8 (l / 16) + j; B column l % 16, same k; accumulator element j
// of lane l is row 4 (l / 16) + j, column l % 16).
template <class DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 4 x 16-bit transpose read from LDS (gfx950 ds_read_b64_tr_b16).  In each 16-lane
// group, lane 4 j + q supplies the address of row j's 4 consecutive 16-bit values
// (columns 4 q .. 4 q + 3 of a 16-column tile), and lane 4 q + e receives column
// 4 q + e of rows 0 .. 3: a row-major 4 x 16 tile comes back column by column.
__device__ __forceinline__ u32x2 tr_read16(const uint16_t* p) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p)));
}

// 16-byte global load / store helpers
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Loads of K/V that are read once per call.
#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif
__device__ __forceinline__ u32x2 ld8_stream(const void* p) {
#if PKV_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#else
  return *reinterpret_cast<const u32x2*>(p);
#endif
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
#if PKV_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return ld16(p);
#endif
}

// ---------------------------------------------------------------------------
// Partial results.  Every (row b, partial slot p, query head h) owns
//   acc[((b * P + p) * Hq + h) * D + 0 .. D)   fp32, un-normalised sum_t 2^(s_t - m) v_t
//   ml [ (b * P + p) * Hq + h ]               (m, l): running max (log2 units) and sum_t 2^(s_t - m)
// Slots [0, depth_b) hold the shared-prefix nodes on row b's path, slots
// [depth_b, depth_b + n_splits_b) the split-K chunks of its own remainder.

struct PartialLayout {
  float* acc;
  float2* ml;
  int32_t slots;  // P
};

}  // namespace pkv
