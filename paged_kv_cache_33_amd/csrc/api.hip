// C ABI of libpagedkv: argument checks, kernel choice and launches.
// The operation and every convention are documented in include/pagedkv.h.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "errors.h"
#include "launch.h"
#include "pagedkv.h"

struct kv_pool {
  kv_pool_desc desc;
  void* k_cache;
  void* v_cache;
};

namespace pagedkv {

int resident_workers(const void* kernel, int threads, int tiles) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int total = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache[dev].find(kernel);
    if (it != cache[dev].end()) {
      total = it->second;
    } else {
      int cus = 0, per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
          per_cu < 1)
        per_cu = 1;
      total = cus * per_cu;
      cache[dev][kernel] = total;
    }
  }
  const int per_tile = total / (tiles > 0 ? tiles : 1);
  return per_tile > 0 ? per_tile : 1;
}

}  // namespace pagedkv

namespace {

using pagedkv::report;
constexpr auto fail = report;
kv_status ok() { return pagedkv::report_ok(); }

kv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_bytes(kv_dtype t) {
  return t == KV_FP8_E4M3 || t == KV_INT8 ? 1 : t == KV_BF16 ? 2 : 4;
}

// Bytes of the element (code) region of one cache buffer; an int8 buffer
// continues with one float32 scale per (block, head, slot) row.
int64_t codes_bytes(const kv_pool_desc& d) {
  return int64_t(d.num_blocks) * d.num_kv_heads * 16 * d.head_dim * int64_t(elem_bytes(d.dtype));
}
int64_t scales_offset(const kv_pool_desc& d) { return d.dtype == KV_INT8 ? codes_bytes(d) : 0; }

pagedkv::Kind kind_of(kv_dtype t) {
  return t == KV_FP8_E4M3 ? pagedkv::Kind::kFp8
         : t == KV_INT8   ? pagedkv::Kind::kInt8
         : t == KV_BF16   ? pagedkv::Kind::kBf16
                          : pagedkv::Kind::kF32;
}

bool positive_finite(float x) { return x > 0.f && x <= 3.4028234663852886e38f; }

// Longest split supported: the reduce keeps one weight per partition in LDS.
constexpr int64_t kMaxPartitions = 8192;

kv_status check_desc(const kv_pool_desc* d) {
  if (!d) return fail(KV_ERR_INVALID_ARG, "pool descriptor is NULL");
  if (d->dtype != KV_F32 && d->dtype != KV_BF16 && d->dtype != KV_FP8_E4M3 &&
      d->dtype != KV_INT8)
    return fail(KV_ERR_UNSUPPORTED,
                "dtype %d is not supported (f32=0, bf16=1, fp8_e4m3=2, int8=3)", int(d->dtype));
  if (d->dtype == KV_FP8_E4M3 && (!positive_finite(d->k_scale) || !positive_finite(d->v_scale)))
    return fail(KV_ERR_INVALID_ARG, "fp8 pool scales must be finite and > 0 (k %g, v %g)",
                double(d->k_scale), double(d->v_scale));
  if (d->block_size != 16)
    return fail(KV_ERR_UNSUPPORTED, "block_size %d is not supported (16 only)", d->block_size);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KV_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (d->num_blocks < 1) return fail(KV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (d->num_kv_heads < 1) return fail(KV_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  return KV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t num_partitions(int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0) return 1;
  const int64_t n = (int64_t(max_context_len) + partition_size - 1) / partition_size;
  return n < 1 ? 1 : n;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WorkspaceView {
  float* o;
  float* m;
  float* l;
  size_t bytes;
};

WorkspaceView workspace_view(void* ws, int32_t B, int32_t H, int32_t d, int64_t P) {
  const size_t n = size_t(B) * size_t(H) * size_t(P);
  const size_t o_bytes = align256(n * size_t(d) * sizeof(float));
  const size_t ml_bytes = align256(n * sizeof(float));
  char* base = static_cast<char*>(ws);
  WorkspaceView v;
  v.o = reinterpret_cast<float*>(base);
  v.m = reinterpret_cast<float*>(base + o_bytes);
  v.l = reinterpret_cast<float*>(base + o_bytes + ml_bytes);
  v.bytes = o_bytes + 2 * ml_bytes;
  return v;
}

kv_status check_partition(int32_t max_context_len, int32_t partition_size) {
  if (max_context_len < 0) return fail(KV_ERR_INVALID_ARG, "max_context_len must be >= 0");
  if (partition_size < 0 || partition_size % 16 != 0)
    return fail(KV_ERR_INVALID_ARG,
                "partition_size %d must be 0 (single pass) or a positive multiple of 16",
                partition_size);
  if (num_partitions(max_context_len, partition_size) > kMaxPartitions)
    return fail(KV_ERR_INVALID_ARG, "more than %lld partitions per sequence",
                static_cast<long long>(kMaxPartitions));
  return KV_OK;
}

}  // namespace

extern "C" {

size_t kv_pool_bytes(const kv_pool_desc* desc) {
  if (check_desc(desc) != KV_OK) return 0;
  const size_t rows = size_t(desc->num_blocks) * size_t(desc->num_kv_heads) * 16u;
  return rows * size_t(desc->head_dim) * elem_bytes(desc->dtype) +
         (desc->dtype == KV_INT8 ? rows * sizeof(float) : 0);
}

kv_status kv_pool_create(const kv_pool_desc* desc, void* k_cache, void* v_cache, kv_pool** out) {
  if (!out) return fail(KV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (kv_status s = check_desc(desc); s != KV_OK) return s;
  if (!k_cache || !v_cache) return fail(KV_ERR_INVALID_ARG, "k_cache and v_cache must be non-NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(KV_ERR_INVALID_ARG, "k_cache and v_cache must be 16-byte aligned");
  kv_pool* p = new (std::nothrow) kv_pool;
  if (!p) return fail(KV_ERR_INVALID_ARG, "out of host memory");
  p->desc = *desc;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  *out = p;
  return ok();
}

void kv_pool_destroy(kv_pool* pool) { delete pool; }

kv_status kv_slot_mapping(const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                          int32_t B, int64_t* slot_mapping, void* stream) {
  if (B < 0) return fail(KV_ERR_INVALID_ARG, "B must be >= 0");
  if (max_nb < 1) return fail(KV_ERR_INVALID_ARG, "max_nb must be >= 1");
  if (B > 0 && (!block_tables || !context_lens || !slot_mapping))
    return fail(KV_ERR_INVALID_ARG, "block_tables, context_lens and slot_mapping must be non-NULL");
  pagedkv::SlotMappingArgs a{block_tables, max_nb, context_lens, B, slot_mapping};
  return hip_status(pagedkv::launch_slot_mapping(a, static_cast<hipStream_t>(stream)),
                    "slot mapping launch");
}

kv_status reshape_and_cache(const kv_pool* pool, const void* key, const void* value,
                            const int64_t* slot_mapping, int32_t N, void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (N < 0) return fail(KV_ERR_INVALID_ARG, "N must be >= 0");
  if (N == 0) return ok();
  if (!key || !value || !slot_mapping)
    return fail(KV_ERR_INVALID_ARG, "key, value and slot_mapping must be non-NULL");
  if (!aligned16(key) || !aligned16(value))
    return fail(KV_ERR_INVALID_ARG, "key and value must be 16-byte aligned");
  const kv_pool_desc& d = pool->desc;
  pagedkv::CacheWriteArgs a{pool->k_cache, pool->v_cache, d.num_blocks, d.num_kv_heads,
                            d.head_dim, key,           value,           slot_mapping,
                            N,           d.k_scale,     d.v_scale,       scales_offset(d)};
  return hip_status(pagedkv::launch_cache_write(a, kind_of(d.dtype),
                                                static_cast<hipStream_t>(stream)),
                    "cache write launch");
}

size_t paged_attention_workspace_bytes(int32_t B, int32_t H, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size) {
  if (partition_size <= 0 || B <= 0 || H <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  const int64_t P = num_partitions(max_context_len, partition_size);
  return workspace_view(nullptr, B, H, head_dim, P).bytes;
}

int32_t kv_decode_kernel_kind(const kv_pool* pool, int32_t H) {
  if (!pool || H < 1 || H % pool->desc.num_kv_heads != 0) return -1;
  const bool packed = pool->desc.dtype == KV_BF16 || pool->desc.dtype == KV_FP8_E4M3 ||
                      pool->desc.dtype == KV_INT8;
  return (packed && H > pool->desc.num_kv_heads) ? 1 : 0;
}

}  // extern "C"

namespace {

// key / value non-NULL: the fused step (kv_decode_step), which also writes
// those rows and takes the newest position from them.
kv_status decode_impl(const kv_pool* pool, void* out, const void* query,
                      const int32_t* block_tables, int32_t max_nb, const int32_t* context_lens,
                      int32_t B, int32_t H, int32_t max_context_len, float scale, int32_t window,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      void* stream, const void* key = nullptr, const void* value = nullptr,
                      int64_t* slot_mapping = nullptr) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  const bool fused = key != nullptr || value != nullptr;
  if (window < 0) return fail(KV_ERR_INVALID_ARG, "window must be >= 0 (0 = whole context)");
  const kv_pool_desc& d = pool->desc;
  if (B < 0) return fail(KV_ERR_INVALID_ARG, "B must be >= 0");
  if (H < 1 || H % d.num_kv_heads != 0)
    return fail(KV_ERR_INVALID_ARG, "H (%d) must be a positive multiple of num_kv_heads (%d)", H,
                d.num_kv_heads);
  if (max_nb < 1) return fail(KV_ERR_INVALID_ARG, "max_nb must be >= 1");
  if (kv_status s = check_partition(max_context_len, partition_size); s != KV_OK) return s;
  if (!(scale > 0.f && scale <= FLT_MAX))
    return fail(KV_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", double(scale));
  if (B == 0) return ok();
  if (partition_size > 0 && B > pagedkv::kMaxSplitSeqs)
    return fail(KV_ERR_UNSUPPORTED, "split mode holds at most %d sequences per call (got %d)",
                pagedkv::kMaxSplitSeqs, B);
  if (!out || !query || !block_tables || !context_lens)
    return fail(KV_ERR_INVALID_ARG, "out, query, block_tables and context_lens must be non-NULL");
  if (!aligned16(query) || !aligned16(out))
    return fail(KV_ERR_INVALID_ARG, "query and out must be 16-byte aligned");
  if (fused && (!key || !value || !aligned16(key) || !aligned16(value)))
    return fail(KV_ERR_INVALID_ARG, "key and value must both be non-NULL and 16-byte aligned");
  const int64_t P = num_partitions(max_context_len, partition_size);
  WorkspaceView ws{nullptr, nullptr, nullptr, 0};
  if (partition_size > 0) {
    ws = workspace_view(workspace, B, H, d.head_dim, P);
    if (!workspace || workspace_bytes < ws.bytes)
      return fail(KV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.bytes,
                  workspace ? workspace_bytes : size_t(0));
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(KV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  pagedkv::DecodeArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.num_blocks = d.num_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.query = query;
  a.out = out;
  a.block_tables = block_tables;
  a.max_nb = max_nb;
  a.context_lens = context_lens;
  a.B = B;
  a.H = H;
  a.max_context_len = max_context_len;
  const bool fp8 = d.dtype == KV_FP8_E4M3;
  // an fp8 key is code * k_scale, so its score is (q . code) * k_scale: the
  // factor joins the softmax scale; V's factor multiplies the output
  a.scale_log2 = scale * 1.4426950408889634f * (fp8 ? d.k_scale : 1.f);
  a.v_scale = fp8 ? d.v_scale : 1.f;
  a.window = window;
  a.scales_offset = scales_offset(d);
  a.partition_size = partition_size;
  a.num_partitions = static_cast<int32_t>(P);
  a.ws_o = ws.o;
  a.ws_m = ws.m;
  a.ws_l = ws.l;
  if (fused) {
    a.fresh_key = key;
    a.fresh_value = value;
    a.append = pagedkv::AppendArgs{pool->k_cache, pool->v_cache, d.num_blocks, d.num_kv_heads,
                                   d.head_dim,    key,           value,        block_tables,
                                   max_nb,        context_lens,  B,            slot_mapping,
                                   d.k_scale,     d.v_scale};
    a.append.scales_offset = scales_offset(d);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (kv_decode_kernel_kind(pool, H) == 1)
    e = pagedkv::launch_decode_mfma(a, kind_of(d.dtype), d.head_dim, s);
  else
    e = pagedkv::launch_decode_valu(a, kind_of(d.dtype), d.head_dim, s);
  return hip_status(e, "decode launch");
}

}  // namespace

extern "C" {

kv_status paged_attention_decode(const kv_pool* pool, void* out, const void* query,
                                 const int32_t* block_tables, int32_t max_nb,
                                 const int32_t* context_lens, int32_t B, int32_t H,
                                 int32_t max_context_len, float scale, int32_t partition_size,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(pool, out, query, block_tables, max_nb, context_lens, B, H, max_context_len,
                     scale, 0, partition_size, workspace, workspace_bytes, stream);
}

kv_status paged_attention_decode_window(const kv_pool* pool, void* out, const void* query,
                                        const int32_t* block_tables, int32_t max_nb,
                                        const int32_t* context_lens, int32_t B, int32_t H,
                                        int32_t max_context_len, float scale, int32_t window,
                                        int32_t partition_size, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return decode_impl(pool, out, query, block_tables, max_nb, context_lens, B, H, max_context_len,
                     scale, window, partition_size, workspace, workspace_bytes, stream);
}

kv_status kv_decode_step(const kv_pool* pool, void* out, const void* query, const void* key,
                         const void* value, const int32_t* block_tables, int32_t max_nb,
                         const int32_t* context_lens, int32_t B, int32_t H,
                         int32_t max_context_len, float scale, int32_t window,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         int64_t* slot_mapping, void* stream) {
  if (B > 0 && (!key || !value))
    return fail(KV_ERR_INVALID_ARG, "key and value must be non-NULL");
  return decode_impl(pool, out, query, block_tables, max_nb, context_lens, B, H, max_context_len,
                     scale, window, partition_size, workspace, workspace_bytes, stream, key, value,
                     slot_mapping);
}

kv_status kv_cache_append(const kv_pool* pool, const void* key, const void* value,
                          const int32_t* block_tables, int32_t max_nb,
                          const int32_t* context_lens, int32_t B, int64_t* slot_mapping,
                          void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (B < 0) return fail(KV_ERR_INVALID_ARG, "B must be >= 0");
  if (max_nb < 1) return fail(KV_ERR_INVALID_ARG, "max_nb must be >= 1");
  if (B == 0) return ok();
  if (!key || !value || !block_tables || !context_lens)
    return fail(KV_ERR_INVALID_ARG, "key, value, block_tables and context_lens must be non-NULL");
  if (!aligned16(key) || !aligned16(value))
    return fail(KV_ERR_INVALID_ARG, "key and value must be 16-byte aligned");
  const kv_pool_desc& d = pool->desc;
  pagedkv::AppendArgs a{pool->k_cache, pool->v_cache, d.num_blocks, d.num_kv_heads, d.head_dim,
                        key,           value,          block_tables, max_nb,     context_lens,
                        B,             slot_mapping,   d.k_scale,    d.v_scale};
  a.scales_offset = scales_offset(d);
  return hip_status(pagedkv::launch_append(a, kind_of(d.dtype), static_cast<hipStream_t>(stream)),
                    "append launch");
}

kv_status kv_cache_append_chunk(const kv_pool* pool, const void* key, const void* value,
                                int32_t num_rows, const int32_t* query_start,
                                int32_t max_query_len, const int32_t* block_tables,
                                int32_t max_nb, const int32_t* context_lens, int32_t B,
                                int64_t* slot_mapping, void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (B < 0 || num_rows < 0 || max_query_len < 0)
    return fail(KV_ERR_INVALID_ARG, "B, num_rows and max_query_len must be >= 0");
  if (max_nb < 1) return fail(KV_ERR_INVALID_ARG, "max_nb must be >= 1");
  if (B == 0 || num_rows == 0 || max_query_len == 0) return ok();
  if (!key || !value || !query_start || !block_tables || !context_lens)
    return fail(KV_ERR_INVALID_ARG,
                "key, value, query_start, block_tables and context_lens must be non-NULL");
  if (!aligned16(key) || !aligned16(value))
    return fail(KV_ERR_INVALID_ARG, "key and value must be 16-byte aligned");
  const kv_pool_desc& d = pool->desc;
  pagedkv::AppendArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.num_blocks = d.num_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.head_dim = d.head_dim;
  a.key = key;
  a.value = value;
  a.block_tables = block_tables;
  a.max_nb = max_nb;
  a.context_lens = context_lens;
  a.B = B;
  a.slot_mapping = slot_mapping;
  a.k_scale = d.k_scale;
  a.v_scale = d.v_scale;
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  a.num_rows = num_rows;
  a.scales_offset = scales_offset(d);
  return hip_status(pagedkv::launch_append(a, kind_of(d.dtype), static_cast<hipStream_t>(stream)),
                    "chunk append launch");
}

kv_status paged_attention_multi(const kv_pool* pool, void* out, const void* query,
                                int32_t num_rows, const int32_t* query_start,
                                int32_t max_query_len, const int32_t* block_tables,
                                int32_t max_nb, const int32_t* context_lens, int32_t B, int32_t H,
                                float scale, int32_t window, void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (window < 0) return fail(KV_ERR_INVALID_ARG, "window must be >= 0 (0 = whole context)");
  const kv_pool_desc& d = pool->desc;
  if (d.dtype == KV_F32)
    return fail(KV_ERR_UNSUPPORTED, "multi-token attention needs a bf16, fp8 or int8 pool");
  if (B < 0 || num_rows < 0 || max_query_len < 0)
    return fail(KV_ERR_INVALID_ARG, "B, num_rows and max_query_len must be >= 0");
  if (H < 1 || H % d.num_kv_heads != 0)
    return fail(KV_ERR_INVALID_ARG, "H (%d) must be a positive multiple of num_kv_heads (%d)", H,
                d.num_kv_heads);
  if (max_nb < 1) return fail(KV_ERR_INVALID_ARG, "max_nb must be >= 1");
  if (!(scale > 0.f && scale <= FLT_MAX))
    return fail(KV_ERR_INVALID_ARG, "scale must be finite and > 0 (got %g)", double(scale));
  if (B > 65535) return fail(KV_ERR_UNSUPPORTED, "at most 65535 sequences per call (got %d)", B);
  const int64_t tiles = (int64_t(max_query_len) * (H / d.num_kv_heads) + 15) / 16;
  if (tiles > (int64_t(1) << 30))
    return fail(KV_ERR_INVALID_ARG, "max_query_len * H / H_kv is too large");
  if (B == 0 || num_rows == 0 || max_query_len == 0) return ok();
  if (!out || !query || !query_start || !block_tables || !context_lens)
    return fail(KV_ERR_INVALID_ARG,
                "out, query, query_start, block_tables and context_lens must be non-NULL");
  if (!aligned16(query) || !aligned16(out))
    return fail(KV_ERR_INVALID_ARG, "query and out must be 16-byte aligned");
  pagedkv::MultiArgs a{};
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.num_blocks = d.num_blocks;
  a.num_kv_heads = d.num_kv_heads;
  a.query = query;
  a.out = out;
  a.num_rows = num_rows;
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  a.block_tables = block_tables;
  a.max_nb = max_nb;
  a.context_lens = context_lens;
  a.B = B;
  a.H = H;
  const bool fp8 = d.dtype == KV_FP8_E4M3;
  a.scale_log2 = scale * 1.4426950408889634f * (fp8 ? d.k_scale : 1.f);
  a.v_scale = fp8 ? d.v_scale : 1.f;
  a.window = window;
  a.scales_offset = scales_offset(d);
  // one tile per wave when one tile holds every column; else two per wave,
  // and up to four such sets per work-group
  a.tiles_per_set = tiles > 1 ? 2 : 1;
  const int64_t sets = (tiles + a.tiles_per_set - 1) / a.tiles_per_set;
  a.sets_per_group = static_cast<int32_t>(sets < 4 ? sets : 4);
  return hip_status(pagedkv::launch_multi_mfma(a, kind_of(d.dtype), d.head_dim,
                                               static_cast<hipStream_t>(stream)),
                    "multi-token attention launch");
}

kv_status kv_copy_blocks(const kv_pool* pool, const int32_t* src, const int32_t* dst, int32_t n,
                         void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(KV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  if (!src || !dst) return fail(KV_ERR_INVALID_ARG, "src and dst must be non-NULL");
  const kv_pool_desc& d = pool->desc;
  pagedkv::CopyBlocksArgs a{pool->k_cache,
                            pool->v_cache,
                            d.num_blocks,
                            int64_t(d.num_kv_heads) * 16 * d.head_dim * int64_t(elem_bytes(d.dtype)),
                            scales_offset(d),
                            d.dtype == KV_INT8 ? d.num_kv_heads * 16 * int32_t(sizeof(float)) : 0,
                            src,
                            dst,
                            n};
  return hip_status(pagedkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream)),
                    "copy_blocks launch");
}

kv_status kv_read_tiles(const kv_pool* pool, const int32_t* tiles, int64_t n, uint32_t* sink,
                        int32_t groups, void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(KV_ERR_INVALID_ARG, "n must be >= 0");
  if (groups < 1 || groups > (1 << 20))
    return fail(KV_ERR_INVALID_ARG, "groups must be in 1 .. 2^20 (got %d)", int(groups));
  if (!sink) return fail(KV_ERR_INVALID_ARG, "sink must be non-NULL");
  if (n > 0 && !tiles) return fail(KV_ERR_INVALID_ARG, "tiles must be non-NULL");
  const kv_pool_desc& d = pool->desc;
  pagedkv::ReadTilesArgs a{pool->k_cache,
                           pool->v_cache,
                           tiles,
                           n,
                           int64_t(16) * d.head_dim * int64_t(elem_bytes(d.dtype)),
                           int64_t(d.num_blocks) * d.num_kv_heads,
                           sink};
  return hip_status(pagedkv::launch_read_tiles(a, groups, static_cast<hipStream_t>(stream)),
                    "read_tiles launch");
}

static kv_status reduce_impl(void* out, const void* workspace, const int32_t* context_lens,
                             int32_t B, int32_t H, int32_t head_dim, int32_t max_context_len,
                             int32_t window, int32_t partition_size, kv_dtype out_dtype,
                             void* stream) {
  if (B < 0 || H < 1) return fail(KV_ERR_INVALID_ARG, "B must be >= 0 and H >= 1");
  if (window < 0) return fail(KV_ERR_INVALID_ARG, "window must be >= 0 (0 = whole context)");
  if (head_dim != 64 && head_dim != 128)
    return fail(KV_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  if (out_dtype != KV_F32 && out_dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "dtype %d is not supported", int(out_dtype));
  if (partition_size <= 0)
    return fail(KV_ERR_INVALID_ARG, "reduce needs the split partition_size (> 0)");
  if (kv_status s = check_partition(max_context_len, partition_size); s != KV_OK) return s;
  if (B == 0) return ok();
  if (!out || !workspace || !context_lens)
    return fail(KV_ERR_INVALID_ARG, "out, workspace and context_lens must be non-NULL");
  const int64_t P = num_partitions(max_context_len, partition_size);
  WorkspaceView ws = workspace_view(const_cast<void*>(workspace), B, H, head_dim, P);
  pagedkv::ReduceArgs a{out, ws.o, ws.m, ws.l, context_lens, B, H, head_dim,
                        static_cast<int32_t>(P), partition_size, window};
  return hip_status(
      pagedkv::launch_reduce(a, out_dtype == KV_BF16, static_cast<hipStream_t>(stream)),
      "reduce launch");
}

kv_status paged_attention_reduce(void* out, const void* workspace, const int32_t* context_lens,
                                 int32_t B, int32_t H, int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size, kv_dtype out_dtype, void* stream) {
  return reduce_impl(out, workspace, context_lens, B, H, head_dim, max_context_len, 0,
                     partition_size, out_dtype, stream);
}

kv_status paged_attention_reduce_window(void* out, const void* workspace,
                                        const int32_t* context_lens, int32_t B, int32_t H,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t window, int32_t partition_size,
                                        kv_dtype out_dtype, void* stream) {
  return reduce_impl(out, workspace, context_lens, B, H, head_dim, max_context_len, window,
                     partition_size, out_dtype, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free split decode.  The split partials live in `scratch`, a
// file-scope device array, instead of a caller workspace; each GPU holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is looked up once per device (with that
// device current) and only that address is handed to the kernels.
namespace {

static_assert(KV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[KV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

kv_status scratch_address(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KV_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess || !p)
      return e != hipSuccess ? hip_status(e, "hipGetSymbolAddress(scratch)")
                             : fail(KV_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return KV_OK;
}

}  // namespace

extern "C" {

kv_status paged_attention_decode_noalloc(const kv_pool* pool, void* out, const void* query,
                                         const int32_t* block_tables, int32_t max_nb,
                                         const int32_t* context_lens, int32_t B, int32_t H,
                                         int32_t max_context_len, float scale,
                                         int32_t partition_size, void* stream) {
  if (!pool) return fail(KV_ERR_INVALID_ARG, "pool is NULL");
  if (partition_size == 0)  // single pass: nothing to keep between kernels
    return decode_impl(pool, out, query, block_tables, max_nb, context_lens, B, H,
                       max_context_len, scale, 0, 0, nullptr, 0, stream);
  if (kv_status s = check_partition(max_context_len, partition_size); s != KV_OK) return s;
  const kv_pool_desc& d = pool->desc;
  const size_t need = paged_attention_workspace_bytes(B, H, d.head_dim, max_context_len,
                                                      partition_size);
  if (need > size_t(KV_NOALLOC_SCRATCH_BYTES))
    return fail(KV_ERR_WORKSPACE,
                "split partials need %zu bytes; the allocation-free call holds at most %zu "
                "(use paged_attention_decode with a workspace)",
                need, size_t(KV_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (kv_status s = scratch_address(&ws); s != KV_OK) return s;
  if (kv_status s = decode_impl(pool, out, query, block_tables, max_nb, context_lens, B, H,
                                max_context_len, scale, 0, partition_size, ws,
                                size_t(KV_NOALLOC_SCRATCH_BYTES), stream);
      s != KV_OK)
    return s;
  if (B == 0) return ok();
  return reduce_impl(out, ws, context_lens, B, H, d.head_dim, max_context_len, 0, partition_size,
                     d.dtype == KV_F32 ? KV_F32 : KV_BF16, stream);
}

}  // extern "C"
