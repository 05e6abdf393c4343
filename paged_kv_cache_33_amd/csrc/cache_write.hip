// Slot mapping and the cache write (reshape_and_cache, kv_cache_append,
// kv_cache_append_chunk).
//
// The block-table mapping is the one "MLSys Engineer - Inference Systems Q&A",
// Q1 gives: logical position i lives in block table[i / 16] at slot i % 16.  The
// write is the append step of the "LLM inference and serving" workbook's
// incremental decoder (K and V grow by one row per token), done for a whole
// batch in one launch.
//
// An fp8 pool stores each element as an E4M3 code of x / scale (see
// source_chunk); bf16 and fp32 pools store the bits unchanged.
// The row writes themselves (and why their stores are non-temporal) are in
// row_write.h.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "row_write.h"

namespace pagedkv {

// One thread per sequence: slot of the newest token (position ctx - 1).
__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotMappingArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int32_t n = a.context_lens[b];
  int64_t slot = -1;
  if (n > 0 && n <= a.max_nb * kBlockTokens) {
    const int32_t pos = n - 1;
    const int32_t blk = a.block_tables[int64_t(b) * a.max_nb + pos / kBlockTokens];
    if (blk >= 0) slot = int64_t(blk) * kBlockTokens + pos % kBlockTokens;
  }
  a.slot_mapping[b] = slot;
}

// One thread per (token, kv head, 16-byte chunk of the head's cached row).  K
// chunks land as one 16-byte store ([d/X][16][X] tile); V elements land one by
// one in the token-minor [d][16] tile.  bf16 / fp32: pure bit moves.
template <typename Tr>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int X = Tr::kChunk;
  const int C = a.head_dim / X;
  const int64_t total = int64_t(a.N) * a.num_kv_heads * C;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = int(idx % C);
  const int h = int((idx / C) % a.num_kv_heads);
  const int64_t i = idx / (int64_t(C) * a.num_kv_heads);
  // The source chunk does not depend on the slot: load it first, so its
  // latency overlaps that of the slot load.
  const int64_t src = (i * a.num_kv_heads + h) * a.head_dim + int64_t(c) * X;
  uint4 kc, vc;
  float ks = 0.f, vs = 0.f;
  row_chunks<Tr>(a.key, a.value, src, C, a.k_scale, a.v_scale, kc, vc, ks, vs);
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= int64_t(a.num_blocks) * kBlockTokens) return;
  const int64_t p = slot / kBlockTokens;
  const int t = int(slot % kBlockTokens);
  const int64_t tile = p * a.num_kv_heads + h;
  write_token_chunk<Tr>(a.k_cache, a.v_cache, tile, C, a.head_dim, c, t, kc, vc);
  write_row_scales<Tr>(a.k_cache, a.v_cache, a.scales_offset, tile, t, c, ks, vs);
}

// One new token per sequence, slot mapping and write in one launch: one thread
// per (sequence, kv head, 16-byte chunk).
template <typename Tr>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= append_threads(a, Tr::kKind)) return;
  append_token_chunk<Tr>(a, idx);
}

// Several new tokens per sequence (a prefill chunk, draft tokens).  Row
// query_start[b] + j sits at position ctx - n + j (n = query_start[b+1] -
// query_start[b], j < max_query_len); its slot follows the table as for one
// token.  One work-group per (block kb touched by the rows, KV head, sequence)
// writes that block's tile at once:
//   K: thread (chunk c, slot s) stores the 16-byte chunk; the 16 slots of one
//      chunk are contiguous in the [d/X][16][X] tile, so a wave's stores are;
//   V: the rows' values pass through LDS (slot-major, padded) and thread
//      (dim x, piece) stores the 16 bytes of the dim's [16]-slot row that the
//      piece covers.  A piece the rows cover only in part is read, merged and
//      written back: this work-group is the only writer of the tile in the call
//      (blocks are not shared between the sequences of one call), and the
//      slots it keeps are written back bit for bit.
// A sequence whose rows are not inside [0, num_rows) is skipped whole; a row
// whose position is negative or past the table, or whose block entry is
// outside the pool, gets slot -1 and no write.
constexpr int kChunkThreads = 256;

template <typename Tr>
__global__ __launch_bounds__(kChunkThreads) void append_chunk_kernel(AppendArgs a) {
  using S = typename Tr::storage;
  constexpr int X = Tr::kChunk;                 // elements per 16 bytes
  constexpr int kMaxRowU4 = 128 * 4 / 16 + 1;   // a padded LDS row of the widest case
  __shared__ uint4 sv[kBlockTokens][kMaxRowU4];

  const int b = blockIdx.z, h = blockIdx.y;
  const int32_t q0 = a.query_start[b], q1 = a.query_start[b + 1];
  if (q0 < 0 || q1 > a.num_rows || q1 <= q0) return;
  const int n = q1 - q0;
  const int nrows = min(n, a.max_query_len);
  const int64_t pos0 = int64_t(a.context_lens[b]) - n;  // position of row 0
  const int64_t cap = int64_t(a.max_nb) * kBlockTokens;
  const int64_t p_lo = max(pos0, int64_t(0));
  const int64_t p_hi = min(pos0 + nrows, cap);
  // rows with no position in the table: slot -1 (one work-group reports them)
  if (a.slot_mapping && blockIdx.x == 0 && h == 0) {
    for (int j = threadIdx.x; j < nrows; j += blockDim.x) {
      const int64_t pos = pos0 + j;
      if (pos < 0 || pos >= cap) a.slot_mapping[int64_t(q0) + j] = -1;
    }
  }
  if (p_lo >= p_hi) return;
  const int64_t kb = p_lo / kBlockTokens + blockIdx.x;
  if (kb * kBlockTokens >= p_hi) return;
  const int s_lo = int(max(p_lo, kb * kBlockTokens) - kb * kBlockTokens);  // slots [s_lo, s_hi)
  const int s_hi = int(min(p_hi, kb * kBlockTokens + kBlockTokens) - kb * kBlockTokens);
  const int32_t blk = a.block_tables[int64_t(b) * a.max_nb + kb];
  const bool ok = blk >= 0 && blk < a.num_blocks;
  // row of slot s: q0 + (kb*16 + s - pos0)
  const int64_t row0 = int64_t(q0) + kb * kBlockTokens - pos0;
  if (a.slot_mapping && h == 0) {
    for (int s = s_lo + int(threadIdx.x); s < s_hi; s += blockDim.x)
      a.slot_mapping[row0 + s] = ok ? int64_t(blk) * kBlockTokens + s : -1;
  }
  if (!ok) return;

  const int D = a.head_dim;
  const int C = D / X;                       // 16-byte chunks per row
  const int64_t tile = int64_t(blk) * a.num_kv_heads + h;
  S* kt = static_cast<S*>(a.k_cache) + tile * int64_t(kBlockTokens) * D;
  S* vt = static_cast<S*>(a.v_cache) + tile * int64_t(kBlockTokens) * D;

  // K straight to the tile; V chunks into LDS
  if constexpr (Tr::kKind == Kind::kInt8) {
    // A row's C chunks sit in C consecutive lanes (C divides 64), which
    // reduce its largest magnitude together; the lane of chunk 0 stores the
    // row's two scales.
    for (int idx = threadIdx.x; idx < C * kBlockTokens; idx += blockDim.x) {
      const int s = idx / C, c = idx % C;
      if (s < s_lo || s >= s_hi) continue;  // uniform over the row's lanes
      const int64_t src = ((row0 + s) * a.num_kv_heads + h) * D + int64_t(c) * X;
      float ks, vs;
      const uint4 kc = int8_chunk(a.key, src, C, ks);
      const u32x4_t ku = {kc.x, kc.y, kc.z, kc.w};
      __builtin_nontemporal_store(ku, reinterpret_cast<u32x4_t*>(kt + (int64_t(c) * kBlockTokens + s) * X));
      sv[s][c] = int8_chunk(a.value, src, C, vs);
      write_row_scales<Tr>(a.k_cache, a.v_cache, a.scales_offset, tile, s, c, ks, vs);
    }
  } else {
    for (int idx = threadIdx.x; idx < C * kBlockTokens; idx += blockDim.x) {
      const int c = idx / kBlockTokens, s = idx % kBlockTokens;
      if (s < s_lo || s >= s_hi) continue;
      const int64_t src = ((row0 + s) * a.num_kv_heads + h) * D + int64_t(c) * X;
      const uint4 kc = source_chunk<Tr>(a.key, src, a.k_scale);
      const u32x4_t ku = {kc.x, kc.y, kc.z, kc.w};
      __builtin_nontemporal_store(ku, reinterpret_cast<u32x4_t*>(kt + (int64_t(c) * kBlockTokens + s) * X));
      sv[s][c] = source_chunk<Tr>(a.value, src, a.v_scale);
    }
  }
  __syncthreads();

  // V rows: dim x, piece pc of X slots (16 bytes); elements move as integers
  using U = std::conditional_t<sizeof(S) == 4, uint32_t,
                               std::conditional_t<sizeof(S) == 2, uint16_t, uint8_t>>;
  constexpr int kPieces = kBlockTokens / X;
  const U* lds = reinterpret_cast<const U*>(&sv[0][0]);
  const int row_elems = kMaxRowU4 * X;       // LDS row stride in elements
  const bool full = s_lo == 0 && s_hi == kBlockTokens;
  for (int idx = threadIdx.x; idx < D * kPieces; idx += blockDim.x) {
    const int x = idx / kPieces, pc = idx % kPieces;
    const int f = pc * X;                    // first slot of the piece
    if (f + X <= s_lo || f >= s_hi) continue;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(vt + int64_t(x) * kBlockTokens + f);
    U e[X];
    if (!full && (f < s_lo || f + X > s_hi)) {
      const u32x4_t old = *dst;              // slots the rows do not cover stay as they are
      __builtin_memcpy(e, &old, sizeof(old));
    }
#pragma unroll
    for (int k = 0; k < X; ++k)
      if (f + k >= s_lo && f + k < s_hi) e[k] = lds[(f + k) * row_elems + x];
    u32x4_t v;
    __builtin_memcpy(&v, e, sizeof(v));
    __builtin_nontemporal_store(v, dst);
  }
}

hipError_t launch_slot_mapping(const SlotMappingArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (a.B + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// Copy-on-write data copy: work-group (i, c, z) copies slice z (kCopySlice
// bytes) of block src[i] of cache c (0 = K, 1 = V) to block dst[i], four
// 16-byte loads in flight per thread.  A lone copy thus still spreads over
// many work-groups.  Both sides stream (non-temporal): the source is not
// reread, and the destination's next reader is a later decode, which should
// not meet dirty lines in the caches.
constexpr int kCopyThreads = 256;
constexpr int64_t kCopySlice = int64_t(kCopyThreads) * 16 * 4;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int i = blockIdx.x;
  const int32_t s = a.src[i], d = a.dst[i];
  if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks || s == d) return;
  char* base = static_cast<char*>(blockIdx.y == 0 ? a.k_cache : a.v_cache);
  const int64_t lo = int64_t(blockIdx.z) * kCopySlice;
  const int64_t hi = min(lo + kCopySlice, a.block_bytes);
  if (a.scale_block_bytes > 0 && blockIdx.z == 0) {  // int8: the block's row scales
    const int n4 = a.scale_block_bytes / 4;
    const float* fs = reinterpret_cast<const float*>(base + a.scales_offset) + int64_t(s) * n4;
    float* fd = reinterpret_cast<float*>(base + a.scales_offset) + int64_t(d) * n4;
    for (int k = threadIdx.x; k < n4; k += kCopyThreads)
      __builtin_nontemporal_store(__builtin_nontemporal_load(fs + k), fd + k);
  }
  const u32x4_t* from = reinterpret_cast<const u32x4_t*>(base + int64_t(s) * a.block_bytes + lo);
  u32x4_t* to = reinterpret_cast<u32x4_t*>(base + int64_t(d) * a.block_bytes + lo);
  const int n16 = int((hi - lo) / 16);
  u32x4_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = threadIdx.x + u * kCopyThreads;
    if (k < n16) v[u] = __builtin_nontemporal_load(from + k);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = threadIdx.x + u * kCopyThreads;
    if (k < n16) __builtin_nontemporal_store(v[u], to + k);
  }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const unsigned slices = unsigned((a.block_bytes + kCopySlice - 1) / kCopySlice);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(a.n), 2, slices), dim3(kCopyThreads), 0, s,
                     a);
  return hipGetLastError();
}

static int chunk_elems(Kind kind) {
  return kind == Kind::kFp8 || kind == Kind::kInt8 ? 16 : kind == Kind::kBf16 ? Bf16::kChunk
                                                                             : F32::kChunk;
}

hipError_t launch_cache_write(const CacheWriteArgs& a, Kind kind, hipStream_t s) {
  const int64_t total = int64_t(a.N) * a.num_kv_heads * (a.head_dim / chunk_elems(kind));
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const unsigned blocks = unsigned((total + threads - 1) / threads);
  switch (kind) {
    case Kind::kBf16:
      hipLaunchKernelGGL(cache_write_kernel<Bf16>, dim3(blocks), dim3(threads), 0, s, a);
      break;
    case Kind::kF32:
      hipLaunchKernelGGL(cache_write_kernel<F32>, dim3(blocks), dim3(threads), 0, s, a);
      break;
    case Kind::kFp8:
      hipLaunchKernelGGL(cache_write_kernel<Fp8>, dim3(blocks), dim3(threads), 0, s, a);
      break;
    case Kind::kInt8:
      hipLaunchKernelGGL(cache_write_kernel<Int8>, dim3(blocks), dim3(threads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

template <typename Tr>
static void (*append_kernel_for(bool chunk))(AppendArgs) {
  return chunk ? append_chunk_kernel<Tr> : append_kernel<Tr>;
}

hipError_t launch_append(const AppendArgs& a, Kind kind, hipStream_t s) {
  const bool chunk = a.query_start != nullptr;
  void (*kern)(AppendArgs) = kind == Kind::kBf16   ? append_kernel_for<Bf16>(chunk)
                             : kind == Kind::kFp8  ? append_kernel_for<Fp8>(chunk)
                             : kind == Kind::kInt8 ? append_kernel_for<Int8>(chunk)
                                                   : append_kernel_for<F32>(chunk);
  if (!kern) return hipErrorInvalidValue;
  if (chunk) {
    // blocks the rows of one sequence may touch: ceil(max_query_len / 16) + 1
    if (a.B == 0 || a.max_query_len == 0) return hipSuccess;
    const int64_t nbk = (int64_t(a.max_query_len) + kBlockTokens - 1) / kBlockTokens + 1;
    hipLaunchKernelGGL(kern, dim3(unsigned(nbk), unsigned(a.num_kv_heads), unsigned(a.B)),
                       dim3(kChunkThreads), 0, s, a);
    return hipGetLastError();
  }
  const int64_t total = int64_t(a.B) * a.num_kv_heads * (a.head_dim / chunk_elems(kind));
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const unsigned blocks = unsigned((total + threads - 1) / threads);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
