// Row writes into the pool, shared by the cache-write kernels and the fused
// decode step: a token's K and V rows (or chunks of them) stored into their
// slot in the pool layout, quantised for fp8 and int8 pools.
//
// Stores are non-temporal.  A decode step writes a few bytes into many cache
// lines (one token of each K chunk row and of each V dim row); left dirty in the
// caches, those lines would be evicted one by one in the middle of the next
// decode's read stream and cost it far more than their size.  Streamed out
// here, they are gone before the decode starts.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace pagedkv {

// Write chunk c (X elements) of one token's K and V rows, already in cache
// storage as kc and vc, into in-block slot t of tile `tile`: one 16-byte store
// for K ([d/X][16][X] tile), X element stores for V ([d][16] tile).
template <typename Tr>
__device__ __forceinline__ void write_token_chunk(void* k_cache, void* v_cache, int64_t tile, int C,
                                                  int head_dim, int c, int t, const uint4 kc,
                                                  const uint4 vc) {
  using S = typename Tr::storage;
  constexpr int X = Tr::kChunk;
  S* kdst = static_cast<S*>(k_cache) + ((tile * C + c) * kBlockTokens + t) * X;
  const u32x4_t ku = {kc.x, kc.y, kc.z, kc.w};
  __builtin_nontemporal_store(ku, reinterpret_cast<u32x4_t*>(kdst));
  S ve[X];
  __builtin_memcpy(ve, &vc, sizeof(vc));
  S* vdst = static_cast<S*>(v_cache) + (tile * head_dim + int64_t(c) * X) * kBlockTokens + t;
#pragma unroll
  for (int e = 0; e < X; ++e) __builtin_nontemporal_store(ve[e], vdst + e * kBlockTokens);
}

// Chunk c of a source row (key or value), whose first element is at element
// offset src, in cache storage.  bf16 / fp32: the row's own 16 bytes.  fp8: the
// row's 16 bf16 values (32 bytes), each stored as e4m3_code(x / scale), the
// division in fp32 (correctly rounded) - "Forward Deployed Engineering
// Interview", Ch.2 section 9: a per-tensor scale, 1.0 when uncalibrated.
template <typename Tr>
__device__ __forceinline__ uint4 source_chunk(const void* base, int64_t src, float scale) {
  if constexpr (Tr::kKind == Kind::kFp8) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + src);
    const uint4 lo = p[0], hi = p[1];
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      c[k] = e4m3_code(bf16_lo(w[2 * k]) / scale) | e4m3_code(bf16_hi(w[2 * k]) / scale) << 8 |
             e4m3_code(bf16_lo(w[2 * k + 1]) / scale) << 16 |
             e4m3_code(bf16_hi(w[2 * k + 1]) / scale) << 24;
    return make_uint4(c[0], c[1], c[2], c[3]);
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const typename Tr::storage*>(base) + src);
  }
}

// Chunk c (16 values) of a source row as int8 codes; s receives the row's
// scale, its largest finite magnitude / 127 ("MLSys Engineer - Inference
// Systems Q&A", Q3 item 1).  The C threads of one row are C consecutive lanes
// (C a power of two dividing 64) and all of them call this: the row maximum
// is combined across them with lane shuffles.
__device__ __forceinline__ uint4 int8_chunk(const void* base, int64_t src, int C, float& s) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + src);
  const uint4 lo = p[0], hi = p[1];
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = bf16_lo(w[k]);
    x[2 * k + 1] = bf16_hi(w[k]);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (__builtin_isfinite(x[k])) amax = fmaxf(amax, fabsf(x[k]));
  for (int off = 1; off < C; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  s = amax / 127.f;
  uint32_t c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    c[k] = int8_code(x[4 * k], s) | int8_code(x[4 * k + 1], s) << 8 |
           int8_code(x[4 * k + 2], s) << 16 | int8_code(x[4 * k + 3], s) << 24;
  return make_uint4(c[0], c[1], c[2], c[3]);
}

// Source chunks of one (token, head) row chunk for the cache: K and V codes
// or bits, and for an int8 cache the two row scales.
template <typename Tr>
__device__ __forceinline__ void row_chunks(const void* key, const void* value, int64_t src, int C,
                                           float k_scale, float v_scale, uint4& kc, uint4& vc,
                                           float& ks, float& vs) {
  if constexpr (Tr::kKind == Kind::kInt8) {
    kc = int8_chunk(key, src, C, ks);
    vc = int8_chunk(value, src, C, vs);
  } else {
    kc = source_chunk<Tr>(key, src, k_scale);
    vc = source_chunk<Tr>(value, src, v_scale);
  }
}

// An int8 row's two scales, stored by the thread of chunk 0 (tile = block *
// H_kv + head, t = in-block slot).
template <typename Tr>
__device__ __forceinline__ void write_row_scales(void* k_cache, void* v_cache,
                                                 int64_t scales_offset, int64_t tile, int t,
                                                 int c, float ks, float vs) {
  if constexpr (Tr::kKind == Kind::kInt8) {
    if (c != 0) return;
    const int64_t i = tile * kBlockTokens + t;
    __builtin_nontemporal_store(ks, reinterpret_cast<float*>(static_cast<char*>(k_cache) +
                                                             scales_offset) + i);
    __builtin_nontemporal_store(vs, reinterpret_cast<float*>(static_cast<char*>(v_cache) +
                                                             scales_offset) + i);
  }
}

// One new token per sequence: thread idx of B * H_kv * C (sequence, kv head,
// 16-byte chunk of the head's cached row) computes the slot of position
// ctx - 1 and writes its chunk there; -1 (nothing written) for ctx <= 0,
// ctx > max_nb*16 or a table entry outside the pool.  The C threads of one row
// must be C consecutive lanes of a wave (int8 rows reduce their maximum across
// them), all present or all absent.
template <typename Tr>
__device__ __forceinline__ void append_token_chunk(const AppendArgs& a, int64_t idx) {
  constexpr int X = Tr::kChunk;
  const int C = a.head_dim / X;
  const int c = int(idx % C);
  const int h = int((idx / C) % a.num_kv_heads);
  const int b = int(idx / (int64_t(C) * a.num_kv_heads));
  // Source chunk first: it overlaps the dependent length -> table loads.
  const int64_t src = (int64_t(b) * a.num_kv_heads + h) * a.head_dim + int64_t(c) * X;
  uint4 kc, vc;
  float ks = 0.f, vs = 0.f;
  row_chunks<Tr>(a.key, a.value, src, C, a.k_scale, a.v_scale, kc, vc, ks, vs);
  const int32_t n = a.context_lens[b];
  int64_t slot = -1;
  if (n > 0 && n <= a.max_nb * kBlockTokens) {
    const int32_t pos = n - 1;
    const int32_t blk = a.block_tables[int64_t(b) * a.max_nb + pos / kBlockTokens];
    if (blk >= 0 && blk < a.num_blocks) slot = int64_t(blk) * kBlockTokens + pos % kBlockTokens;
  }
  if (a.slot_mapping && h == 0 && c == 0) a.slot_mapping[b] = slot;
  if (slot < 0) return;
  const int64_t tile = (slot / kBlockTokens) * a.num_kv_heads + h;
  write_token_chunk<Tr>(a.k_cache, a.v_cache, tile, C, a.head_dim, c, int(slot % kBlockTokens), kc,
                        vc);
  write_row_scales<Tr>(a.k_cache, a.v_cache, a.scales_offset, tile, int(slot % kBlockTokens), c,
                       ks, vs);
}

// Work-group g of the cache write inside a fused decode step: its threads
// take append threads g * blockDim.x ..
template <typename Tr>
__device__ __forceinline__ void append_group(const AppendArgs& a, int64_t g);

// Threads of the one-token append: B * H_kv * (d / elements per chunk).
__host__ __device__ inline int64_t append_threads(const AppendArgs& a, Kind kind) {
  const int X = kind == Kind::kFp8 || kind == Kind::kInt8 ? 16 : kind == Kind::kBf16 ? 8 : 4;
  return int64_t(a.B) * a.num_kv_heads * (a.head_dim / X);
}

// Wave 0 of an item holding the newest position puts that position's K and V
// rows (sequence b, KV head kvh) into LDS as the cache will hold them once the
// step's write has run, and notes whether the table entry of its block lies
// outside the pool (the cache write skips such a row, so the step's result is
// NaN as when the decode meets such a block).  bf16 and fp32 caches store the
// rows' own bits, copied as they are.  One-byte caches store codes: the rows
// are quantised here with the write's own functions on the same inputs, so
// the codes are the ones the write stores, and each code goes to LDS as its
// bf16 value (exact), in dim order, where the decode reads its operands
// (an fp8 code without its scale, which the decode applies where it applies
// it to cached codes; an int8 code with its row scale in fresh_scale[0] (K)
// and [1] (V)).  LDS operations of one wave complete in order, so the same
// wave reads them back after its walk without a barrier; the other waves read
// them after the merge barrier.
template <typename Tr, int D>
__device__ __forceinline__ void fetch_fresh(const DecodeArgs& a, int b, int kvh, int lane,
                                            typename Tr::act (*sm_fresh)[D], int& sm_fresh_bad,
                                            float* sm_fresh_scale) {
  using A = typename Tr::act;
  constexpr int CH = D * int(sizeof(A)) / 16;  // 16-byte chunks per row (<= 32)
  const size_t row = (size_t(b) * a.num_kv_heads + kvh) * D;
  if constexpr (!kByteCodes<Tr>) {
    if (lane < 2 * CH) {
      const char* src = static_cast<const char*>(lane < CH ? a.fresh_key : a.fresh_value) +
                        row * sizeof(A) + (lane % CH) * 16;
      const uint4 r = *reinterpret_cast<const uint4*>(src);
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sm_fresh[lane / CH][0]) + (lane % CH) * 16) = r;
    }
  } else {
    // lanes r * CH + c: row r (0 = K, 1 = V), bf16 values 8c .. 8c + 7; the CH
    // lanes of a row are consecutive and CH divides 64 (row maxima by shuffles)
    static_assert(2 * CH <= kWave && (kWave % CH) == 0, "fresh rows in one wave");
    const int r = (lane / CH) & 1, c = lane % CH;
    const uint16_t* src = static_cast<const uint16_t*>(r ? a.fresh_value : a.fresh_key) + row + 8 * c;
    const uint4 raw = *reinterpret_cast<const uint4*>(src);  // every lane: in bounds, unused past 2 CH
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(w[k]);
      x[2 * k + 1] = bf16_hi(w[k]);
    }
    uint32_t o[4];
    if constexpr (Tr::kKind == Kind::kFp8) {
      // the code source_chunk<Fp8> stores, decoded as the block path decodes it
      const float scale = r ? a.append.v_scale : a.append.k_scale;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = code2_to_bf16x2<Kind::kFp8, false>(e4m3_code(x[2 * k] / scale) |
                                                  (e4m3_code(x[2 * k + 1] / scale) << 8));
    } else {
      // int8_chunk's scale: the row's largest finite magnitude / 127 (a max,
      // so the grouping of the lanes does not matter), then its codes
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (__builtin_isfinite(x[k])) amax = fmaxf(amax, fabsf(x[k]));
      for (int off = 1; off < CH; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
      const float s = amax / 127.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = code2_to_bf16x2<Kind::kInt8, false>(int8_code(x[2 * k], s) |
                                                   (int8_code(x[2 * k + 1], s) << 8));
      if (c == 0 && lane < 2 * CH) sm_fresh_scale[r] = s;
    }
    if (lane < 2 * CH)
      *reinterpret_cast<uint4*>(&sm_fresh[r][8 * c]) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) {
    const int pos = a.context_lens[b] - 1;
    const int p = a.block_tables[int64_t(b) * a.max_nb + pos / kBlockTokens];
    sm_fresh_bad = p < 0 || p >= a.num_blocks;
  }
}

template <typename Tr>
__device__ __forceinline__ void append_group(const AppendArgs& a, int64_t g) {
  const int64_t idx = g * blockDim.x + threadIdx.x;
  if (idx < append_threads(a, Tr::kKind)) append_token_chunk<Tr>(a, idx);
}

}  // namespace pagedkv
