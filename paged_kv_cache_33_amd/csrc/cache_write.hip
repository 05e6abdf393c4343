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
//
// Stores are non-temporal.  A decode step writes a few bytes into many cache
// lines (one token of each K chunk row and of each V dim row); left dirty in the
// caches, those lines would be evicted one by one in the middle of the next
// decode's read stream and cost it far more than their size.  Streamed out
// here, they are gone before the decode starts.
#include "device_common.h"
#include "launch.h"

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
  const uint4 kc = source_chunk<Tr>(a.key, src, a.k_scale);
  const uint4 vc = source_chunk<Tr>(a.value, src, a.v_scale);
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= int64_t(a.num_blocks) * kBlockTokens) return;
  const int64_t p = slot / kBlockTokens;
  const int t = int(slot % kBlockTokens);
  const int64_t tile = p * a.num_kv_heads + h;
  write_token_chunk<Tr>(a.k_cache, a.v_cache, tile, C, a.head_dim, c, t, kc, vc);
}

// One new token per sequence, slot mapping and write in one launch: one thread
// per (sequence, kv head, 16-byte chunk).  The slot is that of position
// ctx - 1; -1 (nothing written) for ctx <= 0, ctx > max_nb*16 or a table entry
// outside the pool.
template <typename Tr>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int X = Tr::kChunk;
  const int C = a.head_dim / X;
  const int64_t total = int64_t(a.B) * a.num_kv_heads * C;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = int(idx % C);
  const int h = int((idx / C) % a.num_kv_heads);
  const int b = int(idx / (int64_t(C) * a.num_kv_heads));
  // Source chunk first: it overlaps the dependent length -> table loads.
  const int64_t src = (int64_t(b) * a.num_kv_heads + h) * a.head_dim + int64_t(c) * X;
  const uint4 kc = source_chunk<Tr>(a.key, src, a.k_scale);
  const uint4 vc = source_chunk<Tr>(a.value, src, a.v_scale);
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
}

// Several new tokens per sequence (a prefill chunk, draft tokens): one thread
// per (row j of sequence b, kv head, 16-byte chunk), over j < max_query_len.
// Row query_start[b] + j sits at position ctx - n + j (n = query_start[b+1] -
// query_start[b]); its slot follows the table as for one token.  A sequence
// whose rows are not inside [0, num_rows) is skipped whole; a row whose
// position is negative or past the table, or whose entry is outside the pool,
// gets slot -1 and no write.
template <typename Tr>
__global__ __launch_bounds__(256) void append_chunk_kernel(AppendArgs a) {
  constexpr int X = Tr::kChunk;
  const int C = a.head_dim / X;
  const int64_t per_row = int64_t(a.num_kv_heads) * C;
  const int64_t total = int64_t(a.max_query_len) * a.B * per_row;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = int(idx % C);
  const int h = int((idx / C) % a.num_kv_heads);
  const int64_t rb = idx / per_row;  // j * B + b: neighbouring threads share j
  const int b = int(rb % a.B);
  const int j = int(rb / a.B);
  const int32_t q0 = a.query_start[b], q1 = a.query_start[b + 1];
  if (q0 < 0 || q1 > a.num_rows || j >= q1 - q0) return;
  const int64_t row = int64_t(q0) + j;
  const int64_t src = (row * a.num_kv_heads + h) * a.head_dim + int64_t(c) * X;
  const uint4 kc = source_chunk<Tr>(a.key, src, a.k_scale);
  const uint4 vc = source_chunk<Tr>(a.value, src, a.v_scale);
  const int64_t pos = int64_t(a.context_lens[b]) - (q1 - q0) + j;
  int64_t slot = -1;
  if (pos >= 0 && pos < int64_t(a.max_nb) * kBlockTokens) {
    const int32_t blk = a.block_tables[int64_t(b) * a.max_nb + pos / kBlockTokens];
    if (blk >= 0 && blk < a.num_blocks) slot = int64_t(blk) * kBlockTokens + pos % kBlockTokens;
  }
  if (a.slot_mapping && h == 0 && c == 0) a.slot_mapping[row] = slot;
  if (slot < 0) return;
  const int64_t tile = (slot / kBlockTokens) * a.num_kv_heads + h;
  write_token_chunk<Tr>(a.k_cache, a.v_cache, tile, C, a.head_dim, c, int(slot % kBlockTokens), kc,
                        vc);
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
  return kind == Kind::kFp8 ? Fp8::kChunk : kind == Kind::kBf16 ? Bf16::kChunk : F32::kChunk;
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
  }
  return hipGetLastError();
}

template <typename Tr>
static void (*append_kernel_for(bool chunk))(AppendArgs) {
  return chunk ? append_chunk_kernel<Tr> : append_kernel<Tr>;
}

hipError_t launch_append(const AppendArgs& a, Kind kind, hipStream_t s) {
  const bool chunk = a.query_start != nullptr;
  const int64_t rows = chunk ? int64_t(a.max_query_len) * a.B : a.B;
  const int64_t total = rows * a.num_kv_heads * (a.head_dim / chunk_elems(kind));
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const unsigned blocks = unsigned((total + threads - 1) / threads);
  void (*kern)(AppendArgs) = kind == Kind::kBf16  ? append_kernel_for<Bf16>(chunk)
                             : kind == Kind::kFp8 ? append_kernel_for<Fp8>(chunk)
                                                  : append_kernel_for<F32>(chunk);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
