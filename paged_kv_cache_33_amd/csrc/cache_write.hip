// Slot mapping and the cache write (reshape_and_cache).
//
// The block-table mapping is the one "MLSys Engineer - Inference Systems Q&A",
// Q1 gives: logical position i lives in block table[i / 16] at slot i % 16.  The
// write is the append step of the "LLM inference and serving" workbook's
// incremental decoder (K and V grow by one row per token), done for a whole
// batch in one launch.
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

// One thread per (token, kv head, 16-byte chunk of the head's row).  K chunks
// land as one 16-byte store ([d/X][16][X] tile); V elements land one by one in
// the token-minor [d][16] tile.  Pure bit moves: no value is converted.
template <typename Tr>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteArgs a) {
  using S = typename Tr::storage;
  constexpr int X = Tr::kChunk;
  const int C = a.head_dim / X;
  const int64_t total = int64_t(a.N) * a.num_kv_heads * C;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = int(idx % C);
  const int h = int((idx / C) % a.num_kv_heads);
  const int64_t i = idx / (int64_t(C) * a.num_kv_heads);
  const int64_t slot = a.slot_mapping[i];
  if (slot < 0 || slot >= int64_t(a.num_blocks) * kBlockTokens) return;
  const int64_t p = slot / kBlockTokens;
  const int t = int(slot % kBlockTokens);
  const int64_t src = (i * a.num_kv_heads + h) * a.head_dim + int64_t(c) * X;
  const int64_t tile = p * a.num_kv_heads + h;

  const uint4 kc = *reinterpret_cast<const uint4*>(static_cast<const S*>(a.key) + src);
  S* kdst = static_cast<S*>(a.k_cache) + ((tile * C + c) * kBlockTokens + t) * X;
  *reinterpret_cast<uint4*>(kdst) = kc;

  const uint4 vc = *reinterpret_cast<const uint4*>(static_cast<const S*>(a.value) + src);
  S ve[X];
  __builtin_memcpy(ve, &vc, sizeof(vc));
  S* vdst = static_cast<S*>(a.v_cache) + (tile * a.head_dim + int64_t(c) * X) * kBlockTokens + t;
#pragma unroll
  for (int e = 0; e < X; ++e) vdst[e * kBlockTokens] = ve[e];
}

hipError_t launch_slot_mapping(const SlotMappingArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (a.B + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, bool bf16, hipStream_t s) {
  const int X = bf16 ? Bf16::kChunk : F32::kChunk;
  const int64_t total = int64_t(a.N) * a.num_kv_heads * (a.head_dim / X);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const unsigned blocks = unsigned((total + threads - 1) / threads);
  if (bf16)
    hipLaunchKernelGGL(cache_write_kernel<Bf16>, dim3(blocks), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(cache_write_kernel<F32>, dim3(blocks), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
