// Device-side helpers shared by the libpagedkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pagedkv {

constexpr int kBlockTokens = 16;  // tokens per physical block
constexpr int kWave = 64;         // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;

// bf16 is the upper half of an fp32, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// 2^x on the hardware's transcendental unit (v_exp_f32).  Arguments here are
// always <= 0 or -inf, where it returns values in [0, 1] and exactly 1 at 0.
// Sliding window ("MLSys Engineer - Inference Systems Q&A", Q3 item 4 and
// Q4): a query at position pos sees positions pos - window + 1 .. pos, not
// below 0; window = 0 means the whole context.
__device__ __forceinline__ int window_first(int pos, int window) {
  return window > 0 && pos >= window ? pos - window + 1 : 0;
}
// First token of the range a decode query (position ctx - 1) walks: the start
// of the block holding its first visible position.  Split partitions are laid
// out from here, so none lies wholly before the window.
__device__ __forceinline__ int range_start(int ctx, int window) {
  return ctx > 0 ? window_first(ctx - 1, window) / kBlockTokens * kBlockTokens : 0;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_xor_max(float v, int lane_mask) {
  return fmaxf(v, __shfl_xor(v, lane_mask, kWave));
}
__device__ __forceinline__ float wave_xor_add(float v, int lane_mask) {
  return v + __shfl_xor(v, lane_mask, kWave);
}

// Data-parallel-primitive lane moves inside one 16-lane row (GCN/CDNA DPP
// control codes): quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror,
// row_mirror.  Applied in that order with a symmetric operation they leave the
// row's total in every lane of the row.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppRowMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppQuadXor1>(v);
  v += dpp_mov<kDppQuadXor2>(v);
  v += dpp_mov<kDppRowHalfMirror>(v);
  return v + dpp_mov<kDppRowMirror>(v);
}

// Combine the four 16-lane rows (lanes l, l^16, l^32, l^48) with gfx950's
// row-swap moves: permlane16_swap(x, x) yields rows {0,0,2,2} and {1,1,3,3};
// permlane32_swap(x, x) yields halves {lo,lo} and {hi,hi}.
__device__ __forceinline__ float cross_row_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float cross_row_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c on two packed bf16 pairs (v_dot2_f32_bf16): the
// bf16 products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 values to one packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Loads of pool tiles.  Every cached K/V byte is read exactly once per decode
// step and never again within it, so tile loads are non-temporal: they stream
// past the caches instead of evicting what is reused (tables, queries).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_tile16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_tile8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_tile4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Element-type traits.  storage: one cache element; act: one element of the
// query, the output and the rows handed to the cache write; kChunk: cache
// elements per 16-byte chunk of the K layout.
struct Bf16 {
  using storage = uint16_t;
  using act = uint16_t;
  static constexpr Kind kKind = Kind::kBf16;
  static constexpr int kChunk = 8;
  __device__ __forceinline__ static act from_f32(float f) { return f32_to_bf16_rne(f); }
};
struct F32 {
  using storage = float;
  using act = float;
  static constexpr Kind kKind = Kind::kF32;
  static constexpr int kChunk = 4;
  __device__ __forceinline__ static act from_f32(float f) { return f; }
};
// fp8 cache ("Forward Deployed Engineering Interview", Ch.2 section 9): OCP
// E4M3 codes with per-tensor scales; bf16 activations.
struct Fp8 {
  using storage = uint8_t;
  using act = uint16_t;
  static constexpr Kind kKind = Kind::kFp8;
  static constexpr int kChunk = 16;
  __device__ __forceinline__ static act from_f32(float f) { return f32_to_bf16_rne(f); }
};

// int8 cache ("MLSys Engineer - Inference Systems Q&A", Q3 item 1): codes with
// one float32 scale per (token, KV head) row, stored after the codes of each
// cache buffer; bf16 activations.
struct Int8 {
  using storage = uint8_t;
  using act = uint16_t;
  static constexpr Kind kKind = Kind::kInt8;
  static constexpr int kChunk = 16;
  __device__ __forceinline__ static act from_f32(float f) { return f32_to_bf16_rne(f); }
};

// int8 codes already rewritten as bf16 values (exact; see i8x2_to_bf16x2), in
// the bf16 tile layout, with the int8 cache's row scales still to apply.
struct Int8AsBf16 {
  using storage = uint16_t;
  using act = uint16_t;
  static constexpr Kind kKind = Kind::kInt8;
  static constexpr int kChunk = 8;
};

// Elements stored as one-byte codes (fp8 and int8 caches).
template <typename Tr>
constexpr bool kByteCodes = sizeof(typename Tr::storage) == 1;

// Two int8 codes (bytes 0, 1 of `w`, or bytes 2, 3 when `hi`) as a bf16 pair:
// exact, since |code| <= 127 needs 7 significant bits, so each float's upper
// half is its bf16 value.  The two halves are joined with one byte permute.
template <bool kHi>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w) {
  const float lo = float(int(w << (kHi ? 8 : 24)) >> 24);
  const float hi = float(int(w << (kHi ? 0 : 16)) >> 24);
  // bytes 2, 3 of lo, then bytes 2, 3 of hi
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// The row scales of an int8 cache buffer (after its codes).
__device__ __forceinline__ const float* row_scales(const void* cache, int64_t scales_offset) {
  return reinterpret_cast<const float*>(static_cast<const char*>(cache) + scales_offset);
}

// Two one-byte codes of a cache type as a bf16 pair.
template <Kind kK, bool kHi>
__device__ __forceinline__ uint32_t code2_to_bf16x2(uint32_t w);

// Two E4M3 codes (bytes 0, 1 of `w`, or bytes 2, 3 when `hi`) as a bf16 pair:
// exact, since every E4M3 value is a bf16 value.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

template <>
__device__ __forceinline__ uint32_t code2_to_bf16x2<Kind::kFp8, false>(uint32_t w) {
  return e4m3x2_to_bf16x2<false>(w);
}
template <>
__device__ __forceinline__ uint32_t code2_to_bf16x2<Kind::kFp8, true>(uint32_t w) {
  return e4m3x2_to_bf16x2<true>(w);
}
template <>
__device__ __forceinline__ uint32_t code2_to_bf16x2<Kind::kInt8, false>(uint32_t w) {
  return i8x2_to_bf16x2<false>(w);
}
template <>
__device__ __forceinline__ uint32_t code2_to_bf16x2<Kind::kInt8, true>(uint32_t w) {
  return i8x2_to_bf16x2<true>(w);
}

// int8 code of x under the row scale s (s = the row's largest finite
// magnitude / 127): round half to even of x / s, the division correctly
// rounded in fp32, clamped to +-127; 0 for a non-finite x or s = 0.
__device__ __forceinline__ uint32_t int8_code(float x, float s) {
  if (!(s > 0.f) || !__builtin_isfinite(x)) return 0u;
  const float q = fminf(fmaxf(__builtin_rintf(x / s), -127.f), 127.f);
  return uint32_t(int(q)) & 0xFFu;
}

// E4M3 code of x: the nearest value, ties to the even code (the hardware
// conversion), after clamping to +-448 so that an overflow stores the largest
// finite value rather than the NaN code; NaN stores sign | 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  if (x != x) return sign | 0x7Fu;
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xFFu;
}

template <typename Tr>
__device__ __forceinline__ float act_to_f32(typename Tr::act v) {
  if constexpr (Tr::kKind == Kind::kF32) return v; else return bf16_to_f32(v);
}

}  // namespace pagedkv
