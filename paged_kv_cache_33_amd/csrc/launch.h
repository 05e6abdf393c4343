// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pagedkv {

// Sequences one split-KV call may hold: the kernels keep one prefix-sum entry
// per sequence in LDS.
constexpr int kMaxSplitSeqs = 4096;

// Cache element type of a pool (see the traits in device_common.h).
enum class Kind { kF32, kBf16, kFp8, kInt8 };

// Work-groups of `kernel` (block size `threads`) the current GPU keeps
// resident at once, divided among `tiles` head tiles (at least 1 each).
int resident_workers(const void* kernel, int threads, int tiles);

// One new token per sequence: slot mapping and cache write in one launch.
struct AppendArgs {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  const void* key;              // [B][H_kv][d]
  const void* value;
  const int32_t* block_tables;  // [B][max_nb]
  int32_t max_nb;
  const int32_t* context_lens;  // [B]
  int32_t B;
  int64_t* slot_mapping;        // optional [B] out ([num_rows] with query_start)
  float k_scale;                // fp8: stored code = e4m3(x / scale)
  float v_scale;
  // Several rows per sequence: with query_start non-NULL, key/value are
  // [num_rows][H_kv][d] and sequence b's rows query_start[b] .. [b+1]-1 sit at
  // positions ctx_b - n_b .. ctx_b - 1 (n_b <= max_query_len).
  const int32_t* query_start;
  int32_t max_query_len;
  int32_t num_rows;
  int64_t scales_offset;        // int8: bytes from a cache buffer to its row scales
};

// Everything a decode kernel needs; passed by value as the kernel argument.
struct DecodeArgs {
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  const void* query;           // [B][H][d]
  void* out;                   // [B][H][d]
  const int32_t* block_tables; // [B][max_nb]
  int32_t max_nb;
  const int32_t* context_lens; // [B]
  int32_t B;
  int32_t H;
  int32_t max_context_len;
  float scale_log2;            // scale * log2(e) (* k_scale for fp8): scores in base 2
  float v_scale;               // output multiplier (fp8: the V scale; else 1)
  int32_t window;              // sliding window in tokens; 0 = whole context
  int32_t partition_size;      // tokens per partition; 0 = whole sequence
  int32_t num_partitions;      // partitions per sequence in the grid (1 if single pass)
  float* ws_o;                 // [B][H][P][d]   (split mode only)
  float* ws_m;                 // [B][H][P]
  float* ws_l;                 // [B][H][P]
  int64_t scales_offset;       // int8: bytes from a cache buffer to its row scales
  // Fused decode step (kv_decode_step): the K/V rows of each sequence's newest
  // position ctx - 1 ([B][H_kv][d] activations), which the decode takes from
  // here instead of the cache; NULL otherwise.  `append` is the cache write of
  // those rows, done by `append_groups` extra work-groups of the same launch.
  const void* fresh_key;
  const void* fresh_value;
  int32_t append_groups;
  AppendArgs append;
};

// Several new query tokens per sequence (a prefill chunk or draft tokens to
// verify), causal within them.  Sequence b's rows are query_start[b] ..
// query_start[b+1]-1, at positions ctx_b - n_b .. ctx_b - 1.
struct MultiArgs {
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  const void* query;            // [num_rows][H][d]
  void* out;                    // [num_rows][H][d]
  int32_t num_rows;
  const int32_t* query_start;   // [B+1]
  int32_t max_query_len;
  const int32_t* block_tables;  // [B][max_nb]
  int32_t max_nb;
  const int32_t* context_lens;  // [B]
  int32_t B;
  int32_t H;
  float scale_log2;             // as DecodeArgs
  float v_scale;
  int32_t window;               // sliding window per row; 0 = whole context
  int32_t tiles_per_set;        // 16-column tiles one wave carries (1 or 2)
  int32_t sets_per_group;       // column sets one work-group takes (1..4)
  int64_t scales_offset;        // int8: bytes from a cache buffer to its row scales
};

struct ReduceArgs {
  void* out;
  const float* ws_o;
  const float* ws_m;
  const float* ws_l;
  const int32_t* context_lens;
  int32_t B;
  int32_t H;
  int32_t head_dim;
  int32_t num_partitions;
  int32_t partition_size;
  int32_t window;               // as DecodeArgs: partitions start at range_start
};

struct CacheWriteArgs {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  const void* key;              // [N][H_kv][d]
  const void* value;
  const int64_t* slot_mapping;  // [N]
  int32_t N;
  float k_scale;                // fp8: stored code = e4m3(x / scale)
  float v_scale;
  int64_t scales_offset;        // int8: bytes from a cache buffer to its row scales
};

// Whole-block copies (copy-on-write): block src[i] -> dst[i] in both caches.
struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  int32_t num_blocks;
  int64_t block_bytes;          // bytes of one block in one cache (a multiple of 16)
  int64_t scales_offset;        // int8: bytes to the row scales (0: none)
  int32_t scale_block_bytes;    // int8: bytes of one block's row scales
  const int32_t* src;
  const int32_t* dst;
  int32_t n;
};

struct ReadTilesArgs {
  const void* k_cache;
  const void* v_cache;
  const int32_t* tiles;         // tile indices p * H_kv + h; others skipped
  int64_t n;
  int64_t tile_bytes;           // one tile of one cache (a multiple of 1 KiB)
  int64_t pool_tiles;           // num_blocks * H_kv
  uint32_t* sink;               // [groups]
};

struct SlotMappingArgs {
  const int32_t* block_tables;
  int32_t max_nb;
  const int32_t* context_lens;
  int32_t B;
  int64_t* slot_mapping;
};

// Launchers: return the hipError_t of the launch.
hipError_t launch_slot_mapping(const SlotMappingArgs& a, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteArgs& a, Kind kind, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, Kind kind, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
hipError_t launch_read_tiles(const ReadTilesArgs& a, int groups, hipStream_t s);
hipError_t launch_decode_valu(const DecodeArgs& a, Kind kind, int head_dim, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, Kind kind, int head_dim, hipStream_t s);
hipError_t launch_multi_mfma(const MultiArgs& a, Kind kind, int head_dim, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, bool bf16_out, hipStream_t s);

}  // namespace pagedkv
