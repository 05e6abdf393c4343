/*
 * pagedkv.h - C ABI of libpagedkv: decode attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   - "MLSys Engineer - Inference Systems Q&A", Q1 (How does PagedAttention
 *     work?): the cache is split into fixed blocks of 16 tokens; each sequence
 *     has a block table mapping logical token position i to physical block
 *     block_table[i / 16], slot i % 16; the attention kernel reads K and V
 *     through that table instead of a contiguous buffer.
 *   - "LLM inference and serving" workbook, Code from memory (naive
 *     incremental decoding): each decode step appends the new token's K and V
 *     rows, then attends with softmax(K q / sqrt(d)) V over every cached row,
 *     the new one included.
 *   - same Q&A page, Q4 (fused attention kernel): scores never leave the chip;
 *     a running max m and denominator l are rescaled by exp(m_old - m_new)
 *     whenever the max rises (online softmax); accumulation is in fp32.
 *   - "Anthropic Interview: Design an LLM Inference API with GPU Batching",
 *     4.1/4.2 Data model: a sequence owns a block_table of block ids; blocks
 *     come from a free stack kept by the host.
 *   - "Forward Deployed Engineering Interview", Ch.2 section 9 (shrinking the
 *     cache) and its annotated serving configuration: an fp8_e4m3 cache, with
 *     per-tensor scales (1.0 when uncalibrated), halves the bytes per token.
 *
 * Conventions shared by every call:
 *   - Ownership: the caller allocates and owns every buffer (pool, query,
 *     output, tables, lengths, slots, workspace).  The library never allocates
 *     or frees device memory and never synchronises a stream.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Every
 *     call enqueues its kernels there and returns at once; ordering between
 *     calls is stream order.
 *   - Errors: every argument the host can check (null pointers, sizes,
 *     dtypes, head counts, workspace size) is checked before anything is
 *     enqueued; a failed check returns a negative kv_status and leaves a
 *     message for kv_last_error().  Device-resident values (table entries,
 *     lengths, slots) are checked by the kernels themselves: a bad value never
 *     makes a kernel read or write outside the buffers; it is reported as NaN
 *     in the affected output rows (decode) or as a skipped write (cache write).
 *   - Threading: all calls are re-entrant; a kv_pool is immutable after
 *     creation and may be shared by threads.
 *
 * Pool layout in HBM (one K cache and one V cache, each num_blocks *
 * num_kv_heads * 16 * head_dim elements).  Every (block p, kv head h) tile is
 * 16 * head_dim contiguous elements starting at element (p*H_kv + h)*16*d.
 * Inside a tile, with X = 16 / sizeof(element) (8 for bf16, 4 for fp32, 16 for
 * fp8):
 *   K[p][h][t][x] at (((p*H_kv + h)*(d/X) + x/X)*16 + t)*X + x%X
 *       i.e. the tile is [d/X][16 tokens][X]: the 16 bytes holding dims
 *       x..x+X-1 of one token are contiguous, and the 16 tokens' copies of one
 *       such chunk follow one another;
 *   V[p][h][t][x] at ((p*H_kv + h)*d + x)*16 + t
 *       i.e. the tile is [d][16 tokens]: one dim's 16 tokens are contiguous.
 * These are the operand layouts of the gfx950 matrix-core instructions the
 * grouped-query kernel feeds straight from memory (K as the row operand of
 * S = K Q^T, V^T as the row operand of O^T = V^T P^T); the same layout keeps
 * every load of the VALU kernel a coalesced 16-byte access.
 *
 * Query and output: [B][H][d], contiguous, of the pool's activation type: the
 * pool dtype for KV_F32 / KV_BF16, bf16 for KV_FP8_E4M3.  Query head h reads
 * KV head h / (H / H_kv) (contiguous groups).
 *
 * fp8 pools (KV_FP8_E4M3).  Each cached element is an OCP E4M3 code (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent 15 with mantissa 7 is
 * NaN; largest finite value 448); the value it stands for is code value * the
 * pool's k_scale (K) or v_scale (V).  The cache write stores, for a bf16 input
 * x, the nearest E4M3 value of x / scale (the division in fp32), ties to the
 * code with an even mantissa; magnitudes beyond 448 store +-448 and NaN stores
 * sign | 0x7F.  The decode converts codes to bf16 exactly and applies the
 * scales in fp32.
 *
 * int8 pools (KV_INT8; "MLSys Engineer - Inference Systems Q&A", Q3 item 1:
 * INT8 with per-token scaling).  Each cached (token, KV head) row of K and of
 * V has its own float32 scale s = a / 127, a the row's largest finite
 * magnitude; element x is stored as the integer nearest x / s (the division
 * in fp32), ties to even, clamped to +-127 (code 0 for a non-finite x or
 * s = 0), and stands for code * s.  Codes use the fp8 layout (X = 16); each
 * cache buffer continues, after its num_blocks*H_kv*16*d code bytes, with the
 * scales: the scale of (block p, head h, slot t) is float number
 * (p*H_kv + h)*16 + t of that region.  The desc's k_scale / v_scale are
 * ignored.  Every write (reshape_and_cache, kv_cache_append,
 * kv_cache_append_chunk) quantises this way and every attention call reads
 * code * s.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID_ARG = -1,  /* null pointer, negative or inconsistent size   */
  KV_ERR_UNSUPPORTED = -2,  /* a dtype / head_dim / block size not built      */
  KV_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required     */
  KV_ERR_HIP = -4,          /* a HIP runtime call failed (message has detail) */
  KV_ERR_NO_BLOCKS = -5     /* block manager: not enough free blocks; nothing changed */
} kv_status;

typedef enum {
  KV_F32 = 0,      /* fp32 cache, fp32 activations                          */
  KV_BF16 = 1,     /* bf16 cache, bf16 activations                          */
  KV_FP8_E4M3 = 2, /* E4M3 cache codes with per-tensor scales, bf16 activations */
  KV_INT8 = 3      /* int8 cache codes with per-token row scales, bf16 activations */
} kv_dtype;

typedef struct {
  int32_t num_blocks;    /* physical blocks in the pool, >= 1              */
  int32_t block_size;    /* tokens per block; only 16 is supported          */
  int32_t num_kv_heads;  /* H_kv, >= 1                                      */
  int32_t head_dim;      /* d: 64 or 128                                    */
  kv_dtype dtype;        /* cache element type (activations: see above)     */
  float k_scale;         /* KV_FP8_E4M3: scale of K codes, finite and > 0;  */
  float v_scale;         /*   of V codes.  Ignored for the other dtypes.    */
} kv_pool_desc;

typedef struct kv_pool kv_pool; /* opaque host object; borrows the two caches */

/* Bytes of ONE cache (K or V) for this geometry; 0 if the descriptor is
 * invalid.  The pool is num_blocks*H_kv*16*d elements (the KV-cache size
 * formula of the workbook's "The equations" with L = 1, per cache) of 4, 2 or
 * 1 byte, plus 4 bytes per (block, head, slot) row for an int8 pool's row
 * scales. */
size_t kv_pool_bytes(const kv_pool_desc* desc);

/* Wrap two caller-owned device buffers (each kv_pool_bytes(desc) bytes, 16-byte
 * aligned) as a pool: the fixed pool of 16-token blocks that every sequence's
 * block table points into ("MLSys Engineer - Inference Systems Q&A", Q1: the
 * cache is one pool of fixed blocks; "Anthropic Interview: Design an LLM
 * Inference API with GPU Batching", Key concepts (Paged KV memory) and 4.1:
 * the physical blocks are a preallocated pool, handed out by the host).  Host
 * metadata only; nothing is copied or cleared.  Returns KV_OK and *out on
 * success; a NULL pointer, an invalid descriptor (see kv_pool_desc) or a cache
 * pointer not 16-byte aligned gives KV_ERR_INVALID_ARG or KV_ERR_UNSUPPORTED
 * and leaves *out unchanged. */
kv_status kv_pool_create(const kv_pool_desc* desc, void* k_cache, void* v_cache,
                         kv_pool** out);

/* Free the host object (never the caller's buffers).  NULL is ignored. */
void kv_pool_destroy(kv_pool* pool);

/* Slot of each sequence's newest token: for b < B with n = context_lens[b],
 *   slot_mapping[b] = block_tables[b*max_nb + (n-1)/16] * 16 + (n-1) % 16,
 * the block-table mapping of the Q&A page's Q1 applied to position n - 1
 * (context_lens count the token being written).  n <= 0, n > max_nb*16 or a
 * negative table entry give -1 (the cache write skips it).
 * block_tables: device int32 [B][max_nb]; context_lens: device int32 [B];
 * slot_mapping: device int64 [B] (written). */
kv_status kv_slot_mapping(const int32_t* block_tables, int32_t max_nb,
                          const int32_t* context_lens, int32_t B,
                          int64_t* slot_mapping, void* stream);

/* Cache write: store token i's K and V rows (key/value: device [N][H_kv][d]
 * of the activation type) into slot s = slot_mapping[i] (device int64 [N]):
 * block s / 16, in-block token s % 16, using the pool layout above.  The
 * workbook's decode step appends the new row before attending; the Q&A page's
 * Q7 stores all K/V of a batch in one pass.  KV_F32 / KV_BF16: a bit copy,
 * every bit pattern, NaN payloads and -0.0 included, lands unchanged.
 * KV_FP8_E4M3: each element is stored as its E4M3 code (see above).  s < 0 and
 * s >= num_blocks*16 are skipped.  Two tokens naming one slot in one call race
 * (undefined result). */
kv_status reshape_and_cache(const kv_pool* pool, const void* key, const void* value,
                            const int64_t* slot_mapping, int32_t N, void* stream);

/* Append one new token per sequence: the slot mapping and the cache write in
 * one launch.  For b < B with n = context_lens[b], the new token sits at
 * position n - 1 (context_lens count it, as the workbook's decoder appends the
 * row before attending); its K and V rows (key/value: device [B][H_kv][d] of
 * the activation type) are stored, as reshape_and_cache stores them, into block
 * block_tables[b*max_nb + (n-1)/16], in-block slot (n-1) % 16.  The same result
 * as kv_slot_mapping followed by reshape_and_cache.  slot_mapping: optional device int64 [B]
 * (NULL = not wanted) receiving each slot, or -1 where nothing was written:
 * n <= 0, n > max_nb*16, or a table entry outside the pool.  The block must not
 * be shared with another sequence of the same call (the host block manager
 * copies a shared last block before appending). */
kv_status kv_cache_append(const kv_pool* pool, const void* key, const void* value,
                          const int32_t* block_tables, int32_t max_nb,
                          const int32_t* context_lens, int32_t B, int64_t* slot_mapping,
                          void* stream);

/* Append several new tokens per sequence (a prefill chunk, or draft tokens to
 * verify) in one launch: sequence b's n_b = query_start[b+1] - query_start[b]
 * rows, key/value rows query_start[b] .. query_start[b+1]-1 (device
 * [num_rows][H_kv][d] of the activation type), are the tokens at positions
 * ctx_b - n_b .. ctx_b - 1 (context_lens count them, as for kv_cache_append);
 * row j is stored, as reshape_and_cache stores it, into block
 * block_tables[b*max_nb + p/16], slot p % 16, p = ctx_b - n_b + j.  This is
 * the workbook's append step for the n_b rows of one pass, as chunked prefill
 * ("Anthropic Interview: Design an LLM Inference API with GPU Batching",
 * scheduling) and speculative verification (the Q&A page) feed them.
 * query_start: device int32 [B+1]; max_query_len: a host bound on every n_b
 * (rows j >= max_query_len are not written).  slot_mapping: optional device
 * int64 [num_rows] receiving each row's slot, or -1 where nothing was written:
 * p < 0, p >= max_nb*16 or a table entry outside the pool.  A sequence whose
 * rows do not lie inside [0, num_rows) is skipped whole. */
kv_status kv_cache_append_chunk(const kv_pool* pool, const void* key, const void* value,
                                int32_t num_rows, const int32_t* query_start,
                                int32_t max_query_len, const int32_t* block_tables,
                                int32_t max_nb, const int32_t* context_lens, int32_t B,
                                int64_t* slot_mapping, void* stream);

/* Workspace bytes paged_attention_decode needs in split mode, i.e. room for
 * one partial result (o, m, l) per partition and query head: the running
 * output, max and denominator that the Q&A page's Q4 keeps per query while it
 * walks K/V tiles, here kept per partition so that partitions can run in
 * parallel and be merged afterwards by the same rescale rule.  With
 * P = ceil(max_context_len / partition_size) partitions per sequence,
 *   o: float [B][H][P][d], then m: float [B][H][P], then l: float [B][H][P]
 * (each region 256-byte aligned).  0 when partition_size == 0. */
size_t paged_attention_workspace_bytes(int32_t B, int32_t H, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

/* Decode attention for one new query token per sequence: the attention half
 * of the workbook's decode step ("LLM inference and serving", Code from
 * memory: softmax(K q / sqrt(d)) V over every cached row, the new one
 * included), with the rows read through the block table as the Q&A page's Q1
 * describes, and computed as Q4's fused kernel computes it (online softmax,
 * fp32 accumulation; scores never leave the chip):
 *   out[b][h][:] = softmax_t(scale * q[b][h] . K_b[t]) V_b[t], t < ctx_b,
 * where K_b[t], V_b[t] are read from block block_tables[b*max_nb + t/16],
 * slot t % 16 (ctx_b = context_lens[b], which includes the token written this
 * step; for an fp8 pool K_b[t] and V_b[t] are code values times the pool's
 * scales).  fp32 accumulation; bf16 outputs are rounded to nearest-even.
 * query, out: device [B][H][d] of the activation type; block_tables: device int32
 * [B][max_nb] (entries past ceil(ctx_b/16) are never read); context_lens:
 * device int32 [B]; max_context_len: a host upper bound on every ctx_b.
 * ctx_b <= 0 gives zeros.  ctx_b > max_nb*16, ctx_b > max_context_len (split
 * mode) or a table entry outside the pool gives NaN for that sequence.
 * partition_size == 0: single pass, writes out.  partition_size = 16*k > 0:
 * split-KV; each partition of partition_size tokens writes (o, m, l) into the
 * workspace (base-2 units: with s = scale*log2(e)*q.k over the partition, m is
 * a reference value with max(s) - 8 <= m <= max(s), l = sum of 2^(s - m), o =
 * normalised partial output); sequences with a single partition write out
 * directly.  Follow with paged_attention_reduce.
 * scale: finite and > 0 (a softmax temperature; the pages use 1/sqrt(d)),
 * else KV_ERR_INVALID_ARG.
 * H must be a multiple of H_kv.  Kernel choice: H_kv < H with a bf16, fp8 or
 * int8 pool uses the matrix-core kernel; otherwise the vector-ALU kernel. */
kv_status paged_attention_decode(const kv_pool* pool, void* out, const void* query,
                                 const int32_t* block_tables, int32_t max_nb,
                                 const int32_t* context_lens, int32_t B, int32_t H,
                                 int32_t max_context_len, float scale,
                                 int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* paged_attention_decode with a sliding window ("MLSys Engineer - Inference
 * Systems Q&A", Q3 item 4: a local-attention layer needs only the last W
 * tokens; Q4: tiles wholly before the window are never loaded): the query of
 * sequence b (position ctx_b - 1) attends to positions
 * max(0, ctx_b - window) .. ctx_b - 1 only, the last `window` tokens; window
 * = 0 is paged_attention_decode.  Blocks wholly before the window are not
 * read (their table entries may be anything).  Split mode lays the partitions
 * out from the start of the block holding the first visible position:
 * partition k covers [r + k*partition_size, r + (k+1)*partition_size), r =
 * 16 * floor(max(0, ctx_b - window) / 16), so a sequence has
 * ceil((ctx_b - r) / partition_size) partitions; merge them with
 * paged_attention_reduce_window and the same window.  window < 0 is
 * KV_ERR_INVALID_ARG. */
kv_status paged_attention_decode_window(const kv_pool* pool, void* out, const void* query,
                                        const int32_t* block_tables, int32_t max_nb,
                                        const int32_t* context_lens, int32_t B, int32_t H,
                                        int32_t max_context_len, float scale, int32_t window,
                                        int32_t partition_size, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* One whole decode step in one launch: the cache write of kv_cache_append
 * and the attention of paged_attention_decode_window, i.e. the workbook's
 * decode step ("LLM inference and serving", Code from memory: append the new
 * token's K and V rows, then attend over every cached row, the new one
 * included).  key, value: device [B][H_kv][d] (the pool's activation type),
 * the rows of each sequence's newest position ctx_b - 1; they are stored as
 * kv_cache_append stores them (slot_mapping, optional device int64 [B],
 * receives the slots as there), and out gets what paged_attention_decode_window
 * gives after that write.  The attention takes position ctx_b - 1 from key and
 * value themselves, so it does not wait for the write: both run in the same
 * launch, the write on a few extra work-groups.  The arithmetic order differs
 * from the two calls in a row (the newest position joins the softmax last),
 * so results agree within rounding, not bit for bit.  Every other argument is
 * as for paged_attention_decode_window (window = 0: the whole context); in
 * split mode follow with paged_attention_reduce(_window) as usual.  A table
 * entry outside the pool for the newest position's block gives NaN for that
 * sequence (and no write).  Every pool type: for fp8 and int8 pools the
 * newest position enters the attention as the codes (and, int8, the row
 * scales) the write stores, computed from key and value by the write's own
 * rules, so it is the value the cache holds after the step. */
kv_status kv_decode_step(const kv_pool* pool, void* out, const void* query, const void* key,
                         const void* value, const int32_t* block_tables, int32_t max_nb,
                         const int32_t* context_lens, int32_t B, int32_t H,
                         int32_t max_context_len, float scale, int32_t window,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         int64_t* slot_mapping, void* stream);

/* Merge split partials (the workspace paged_attention_decode wrote with the
 * same B, H, head_dim, max_context_len and partition_size) by log-sum-exp:
 * with M = max_k m_k and w_k = l_k * 2^(m_k - M),
 *   out[b][h] = sum_k w_k o_k / sum_k w_k   over the ceil(ctx_b/partition_size)
 * partitions of sequence b; this is Q4's rescale rule applied to whole
 * partitions.  Sequences with one partition are left as the decode wrote
 * them; ctx_b <= 0 gives zeros; ctx_b > max_context_len gives NaN.
 * out: device [B][H][head_dim] of out_dtype, the pool's activation type
 * (KV_BF16 for an fp8 pool; KV_FP8_E4M3 is refused). */
kv_status paged_attention_reduce(void* out, const void* workspace,
                                 const int32_t* context_lens, int32_t B, int32_t H,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size, kv_dtype out_dtype,
                                 void* stream);

/* paged_attention_reduce for partials paged_attention_decode_window wrote
 * (the partition layout above); window = 0 is paged_attention_reduce. */
kv_status paged_attention_reduce_window(void* out, const void* workspace,
                                        const int32_t* context_lens, int32_t B, int32_t H,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t window, int32_t partition_size,
                                        kv_dtype out_dtype, void* stream);

/* Attention of several new query tokens per sequence, causal within them: the
 * workbook's incremental decoder with the rows appended one at a time,
 * evaluated for all of them in one pass (a prefill chunk; the K draft tokens
 * speculative decoding verifies, the Q&A page and the workbook).  Sequence b
 * has n_b = query_start[b+1] - query_start[b] query rows, rows query_start[b]
 * .. query_start[b+1]-1 of query (device [num_rows][H][d], bf16), the tokens
 * at positions ctx_b - n_b .. ctx_b - 1 whose K/V rows are already cached
 * (context_lens count them; write them first with kv_cache_append_chunk).
 * The row at position p gets
 *   out[row][h][:] = softmax_t(scale * q[row][h] . K_b[t]) V_b[t], t <= p,
 * with K_b, V_b read through the block table as in paged_attention_decode;
 * out: device [num_rows][H][d], bf16 (rounded to nearest-even).  n_b = 1 is
 * the decode step.  Matrix-core kernel for every H / H_kv, bf16, fp8 or int8
 * pools (KV_F32 is refused).  scale: finite and > 0, as for the decode.
 * max_query_len: a host bound on every n_b.  Rows of a sequence with
 * n_b > ctx_b, n_b > max_query_len or ctx_b > max_nb*16 are NaN
 * (those below max_query_len; nothing is written past it).  A table entry
 * outside the pool that a row's range reaches makes that row NaN (and may make
 * other rows of its sequence NaN).  n_b <= 0 writes nothing, and a sequence
 * whose rows do not lie inside [0, num_rows) is skipped whole.  window > 0: a
 * sliding window as in paged_attention_decode_window, per row (the row at
 * position p sees max(0, p - window + 1) .. p); 0 = the whole context. */
kv_status paged_attention_multi(const kv_pool* pool, void* out, const void* query,
                                int32_t num_rows, const int32_t* query_start,
                                int32_t max_query_len, const int32_t* block_tables,
                                int32_t max_nb, const int32_t* context_lens, int32_t B, int32_t H,
                                float scale, int32_t window, void* stream);

/* Copy whole blocks on the GPU: for i < n, block src[i] of both caches (all KV
 * heads, all 16 slots, K and V) is copied to block dst[i].  This is the data
 * half of copy-on-write: the block manager below names the pair when a token
 * is appended to a shared last block, and the copy must run (stream order)
 * before that token is written.  src, dst: device int32 [n]; a pair with an
 * index outside the pool, or src == dst, is skipped.  No block may be a
 * destination twice, or both a source and a destination, in one call. */
kv_status kv_copy_blocks(const kv_pool* pool, const int32_t* src, const int32_t* dst, int32_t n,
                         void* stream);

/* Measurement helper, not a step of the decode: read tiles[i] (a tile index
 * p * H_kv + h, naming the 16-slot tile of block p and KV head h) of both
 * caches once, as the decode kernels read a tile (non-temporal 16-byte loads),
 * with no arithmetic.  Timed over the tiles a decode step visits, it gives the
 * bandwidth that access pattern can reach on the device (the decode's own
 * ceiling, below the published peak).  Entries outside [0, num_blocks*H_kv)
 * are skipped.  An int8 pool's row scales are not read.  groups work-groups
 * (1 .. 2^20) share the entries; work-group i stores into sink[i] (device
 * uint32 [groups]) the XOR of every 32-bit word it read, so the XOR over sink
 * is the XOR of all listed tiles' words (a checksum the caller can verify). */
kv_status kv_read_tiles(const kv_pool* pool, const int32_t* tiles, int64_t n, uint32_t* sink,
                        int32_t groups, void* stream);

/* ---------------------------------------------------------------------------
 * Host block manager ("Forward Deployed Engineering Interview", Ch.2 section 8,
 * the block-manager teaching model; "Anthropic Interview: Design an LLM
 * Inference API with GPU Batching", 4.1/4.2 data model): block tables,
 * reference counts, a free queue and a prefix cache for a pool of num_blocks
 * blocks of 16 token slots.  Host memory only; it never touches the GPU.
 *   - The key of a full block covers its parent's key (the block before it in
 *     the table; the sequence's salt for a first block) and its 16 token ids.
 *   - admit reuses the cached blocks of the unbroken run of full blocks at the
 *     start of a prompt (a released block still holding its prefix is taken
 *     back from the free queue) and takes fresh blocks for the rest.
 *   - A fresh block is the front of the free queue (least recently freed); it
 *     loses the cache entry it still carried.
 *   - append opens a fresh block when the last one is full, and copies the
 *     last block first when it is shared (copy-on-write).
 *   - fork gives a child the parent's table, every block shared.
 *   - release drops one reference per block, last block first; unreferenced
 *     blocks join the back of the free queue and stay cached until reused.
 * An operation that needs more free blocks than exist returns KV_ERR_NO_BLOCKS
 * and changes nothing (the caller preempts a sequence and retries).  Sequence
 * ids are the caller's.  Calls on one manager are serialised by a lock. */
typedef struct kv_block_manager kv_block_manager;

kv_status kv_bm_create(int32_t num_blocks, kv_block_manager** out);
void kv_bm_destroy(kv_block_manager* bm);

/* Build sequence seq's table for a prompt of n token ids (host int32), salt
 * (salt_len bytes, may be 0).  *hits = prompt tokens found in cached blocks (a
 * multiple of 16): their K/V rows are already in the pool; the caller writes
 * the rest at slots table[i/16]*16 + i%16, i >= *hits. */
kv_status kv_bm_admit(kv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n,
                      const char* salt, int32_t salt_len, int32_t* hits);

/* Append one token to seq.  *slot = its slot (block*16 + offset).  When the
 * last block was shared, *copy_src / *copy_dst name the block to copy first
 * (kv_copy_blocks); otherwise both are -1. */
kv_status kv_bm_append(kv_block_manager* bm, int64_t seq, int32_t token, int64_t* slot,
                       int32_t* copy_src, int32_t* copy_dst);

/* kv_bm_append for seqs[0..B) in order (one token each, host arrays):
 * slots[b] receives each slot; the copies to make first are written to
 * copy_src / copy_dst (host int32, room for B) and counted in *n_copies.  On a
 * failure the sequences before the failing one stay appended: *done (may be
 * NULL) counts them, and the status is returned. */
kv_status kv_bm_append_batch(kv_block_manager* bm, const int64_t* seqs, const int32_t* tokens,
                             int32_t B, int64_t* slots, int32_t* copy_src, int32_t* copy_dst,
                             int32_t* n_copies, int32_t* done);

/* Child shares every block of seq (parallel sampling, beam search). */
kv_status kv_bm_fork(kv_block_manager* bm, int64_t seq, int64_t child);

/* Drop seq and its references. */
kv_status kv_bm_release(kv_block_manager* bm, int64_t seq);

/* Free blocks (-1 for a NULL manager). */
int32_t kv_bm_num_free(kv_block_manager* bm);

/* seq's block ids (host int32, capacity entries; NULL to ask only for the
 * counts), number of blocks and of tokens. */
kv_status kv_bm_table(kv_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                      int32_t* num_blocks, int32_t* num_tokens);

/* Decode inputs for a batch: row b of tables (host int32 [B][max_nb]) gets
 * seqs[b]'s block ids, then -1; context_lens[b] (host int32 [B]) its token
 * count.  Fails, writing nothing, if a sequence is unknown or has more than
 * max_nb blocks. */
kv_status kv_bm_batch_tables(kv_block_manager* bm, const int64_t* seqs, int32_t B, int32_t max_nb,
                             int32_t* tables, int32_t* context_lens);

/* Bytes of device scratch the allocation-free decode below holds per GPU. */
#define KV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* paged_attention_decode followed by paged_attention_reduce, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the split partials go to a
 * library-held scratch array of KV_NOALLOC_SCRATCH_BYTES bytes per GPU (held
 * from the first call on that GPU until the process ends) instead of a
 * caller workspace.  The caller still passes inputs and outputs; the
 * arguments mean what they mean for paged_attention_decode, and out receives
 * the merged result.  partition_size == 0 is the single pass (no scratch
 * used).  Split sizes whose partials exceed the scratch
 * (paged_attention_workspace_bytes(B, H, head_dim, max_context_len,
 * partition_size) > KV_NOALLOC_SCRATCH_BYTES) return KV_ERR_WORKSPACE before
 * anything is enqueued.  No device memory is allocated or freed; nothing in
 * the scratch needs to start cleared (every partial is written before it is
 * read).  Every call on one GPU shares that GPU's scratch and leaves its
 * partials there: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls in stream order do not. */
kv_status paged_attention_decode_noalloc(const kv_pool* pool, void* out, const void* query,
                                         const int32_t* block_tables, int32_t max_nb,
                                         const int32_t* context_lens, int32_t B, int32_t H,
                                         int32_t max_context_len, float scale,
                                         int32_t partition_size, void* stream);

/* Which decode kernel paged_attention_decode launches for this pool and H:
 * 0 = vector-ALU kernel, 1 = matrix-core (MFMA) kernel, < 0 = unsupported. */
int32_t kv_decode_kernel_kind(const kv_pool* pool, int32_t H);

/* Message of the last failed call on this thread ("" if none).  Argument
 * errors are refused before anything is enqueued, rather than left to fail in
 * the middle of a step ("Ch.29 Building a Production LLM Serving Stack",
 * 29.1.2: admission refuses what the pool cannot hold instead of running out
 * mid-step); this call says which check failed.  The string belongs to the
 * library and stays valid until the thread's next failing call. */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
