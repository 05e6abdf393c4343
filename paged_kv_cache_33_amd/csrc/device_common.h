// Device-side helpers shared by the libpagedkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Element-type traits: storage type and elements per 16-byte chunk.
struct Bf16 {
  using storage = uint16_t;
  static constexpr int kChunk = 8;
  __device__ __forceinline__ static float to_f32(storage s) { return bf16_to_f32(s); }
  __device__ __forceinline__ static storage from_f32(float f) { return f32_to_bf16_rne(f); }
};
struct F32 {
  using storage = float;
  static constexpr int kChunk = 4;
  __device__ __forceinline__ static float to_f32(storage s) { return s; }
  __device__ __forceinline__ static storage from_f32(float f) { return f; }
};

// Unpack one 16-byte chunk (4 dwords) into kChunk floats.
__device__ __forceinline__ void unpack_chunk(const uint4& c, float (&f)[8], Bf16) {
  f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x);
  f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
  f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z);
  f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
}
__device__ __forceinline__ void unpack_chunk(const uint4& c, float (&f)[4], F32) {
  f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
  f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
}

}  // namespace pagedkv
