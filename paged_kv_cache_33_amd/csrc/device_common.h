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
