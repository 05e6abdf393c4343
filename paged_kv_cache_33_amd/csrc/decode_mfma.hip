// Paged decode attention for grouped-query heads on the gfx950 matrix cores.
//
// With g = H / H_kv query heads sharing one KV head, each K/V tile read from
// HBM serves g queries ("MLSys Engineer - Inference Systems Q&A", Q4: the win
// is queries per loaded K/V tile; Q7 of the "LLM inference and serving"
// workbook: GQA heads share one KV head).  Per 16-token block the work is two
// small dense products, done as MFMA tiles with fp32 accumulation:
//   S  [16 tokens x 16 heads] = K [16 x d] . Q^T [d x 16]      (d/32 x 16x16x32)
//   O^T [d x 16 heads]       += V^T [d x 16 tokens] . P^T [16 x 16] (d/16 x 16x16x16)
// Query heads beyond g in the 16-wide tile are zero columns and are never
// written out.  Softmax is online per head column, as in the VALU kernel.
// The tile code (operands, online softmax per block) is in mfma_tile.h.
#include "device_common.h"
#include "launch.h"
#include "mfma_tile.h"
#include "row_write.h"
#include "work_list.h"

namespace pagedkv {
namespace {

// Waves per work-group and work-groups per CU.  Single pass: 4 waves, three
// work-groups per CU (168 VGPRs leave room for 3 waves per SIMD), so a
// finishing work-group's successor fetches its first blocks while two others
// stream.  Split, bf16: 8 waves, one work-group per CU (its work-list loop
// does not fit 3 waves per SIMD without spilling).  Split, one-byte codes (fp8,
// int8): 4 waves, two per CU; a 512-token item is half the bytes there, so
// the start of each item (length, table and first tile loads in a row) weighs
// twice as much, and a second work-group streaming meanwhile hides it
// (measured on the long-context mix with fp8: 104 -> 86 us; bf16 is 1% slower
// that way).
template <typename E, bool kSplit>
constexpr int kWavesOf = kSplit && !kByteCodes<E> ? 8 : 4;
template <typename E, bool kSplit>
constexpr int kGroupsPerCu = !kSplit ? 3 : kByteCodes<E> ? 2 : 1;
// LDS where a work-group's waves merge their (m, l, O): one padded row of O
// per wave and head of the tile.  Fused step: the newest position's K and V
// rows (bf16), its score per head of the tile, and whether its block's table
// entry lies outside the pool.
template <int kWaves, int D>
struct MergeLds {
  __attribute__((aligned(16))) float o[kWaves][kHeadsPerTile][D + 4];
  float m[kWaves][kHeadsPerTile];
  float l[kWaves][kHeadsPerTile];
  int bad[kWaves];
  __attribute__((aligned(16))) uint16_t fresh[2][D];
  float fresh_scale[2];  // int8: the newest rows' scales (K, V)
  float fresh_s[kHeadsPerTile];
  int fresh_bad;
};

// q_n . k of the newest position's key (operand order: lane quarter q holds
// the dims that pair with K operand i), the four quarters combined: head n's
// raw score in every lane of column n.
template <typename E, int D>
__device__ __forceinline__ float fresh_score(const uint4 (&krow)[MfmaShape<D>::KI],
                                             const bf16x8_t (&qop)[MfmaShape<D>::KI]) {
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < MfmaShape<D>::KI; ++i) {
    const uint4 qq = __builtin_bit_cast(uint4, qop[i]);
    dot = dot2_bf16(krow[i].x, qq.x, dot);
    dot = dot2_bf16(krow[i].y, qq.y, dot);
    dot = dot2_bf16(krow[i].z, qq.z, dot);
    dot = dot2_bf16(krow[i].w, qq.w, dot);
  }
  return cross_row_sum(dot);
}

// Split mode with several work-groups per CU (one-byte caches): the work-groups
// sharing a CU are not served alike (the instruction arbiter of each SIMD
// prefers the oldest wave, so the oldest work-group's loads go first), and
// with items dealt round-robin the starved worker finishes last: on the
// long-context mix with an fp8 cache, first items took 9 to 31 us and workers
// ended between 45 and 78 us.  Each worker therefore raises its waves'
// priority with the number of items it still has, so one that has fallen
// behind is served first (fp8 84.7 -> 80.5 us, int8 92.7 -> 90.8 us; with
// one work-group per CU there is nothing to balance).  p: 0..3, wave-uniform.
__device__ __forceinline__ void set_priority(int p) {
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// One work item: partition `part` of sequence b, head tile `tile_y` (a KV
// head and a group of up to 16 of its query heads).
template <typename E, int D, int kWaves>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, const int part, const int tile_y,
                                          const int b, MergeLds<kWaves, D>& sm) {
  using S = typename E::storage;
  constexpr int KI = MfmaShape<D>::KI;
  constexpr int MC = MfmaShape<D>::MC;
  auto& sm_o = sm.o;
  auto& sm_m = sm.m;
  auto& sm_l = sm.l;
  auto& sm_bad = sm.bad;

  const int g = a.H / a.num_kv_heads;
  const int ngroups = (g + kHeadsPerTile - 1) / kHeadsPerTile;
  const int kvh = tile_y / ngroups;
  const int hg = tile_y % ngroups;
  const int head0 = kvh * g + hg * kHeadsPerTile;
  const int nh = min(kHeadsPerTile, g - hg * kHeadsPerTile);
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, q = lane >> 4;

  const int ctx = a.context_lens[b];
  const bool split = a.partition_size > 0;
  const int first = ctx > 0 ? window_first(ctx - 1, a.window) : 0;  // first visible token
  const int rs = range_start(ctx, a.window);
  const int nparts = split ? (ctx > 0 ? (ctx - rs + a.partition_size - 1) / a.partition_size : 0) : 1;
  const bool bad_len = ctx > a.max_nb * kBlockTokens || (split && nparts > a.num_partitions);
  uint16_t* out = static_cast<uint16_t*>(a.out);
  auto out_at = [&](int hh, int x) -> uint16_t& {
    return out[(size_t(b) * a.H + head0 + hh) * D + x];
  };
  auto prow = [&](int hh) -> size_t {
    return (size_t(b) * a.H + head0 + hh) * a.num_partitions + part;
  };

  if (!split && (ctx <= 0 || bad_len)) {
    const uint16_t fill = ctx <= 0 ? uint16_t(0) : uint16_t(0x7fc0);
    for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) out_at(idx / D, idx % D) = fill;
    return;
  }
  if (split && bad_len) {
    if (part >= nparts) return;
    for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
      const int hh = idx / D, x = idx % D;
      if (nparts == 1) {
        out_at(hh, x) = 0x7fc0;
      } else {
        a.ws_o[prow(hh) * D + x] = __int_as_float(0x7fc00000);
        if (x == 0) { a.ws_m[prow(hh)] = 0.f; a.ws_l[prow(hh)] = 1.f; }
      }
    }
    return;
  }
  if (split && part >= nparts) return;

  const int tb = rs + (split ? part * a.partition_size : 0);
  int te = split ? min(tb + a.partition_size, ctx) : ctx;
  // Fused step: the item holding position ctx - 1 takes it from the fresh rows
  // (folded in at the merge) and walks the cache up to ctx - 2 only.
  const bool fold = a.fresh_key != nullptr && (!split || part == nparts - 1);
  if (fold) te = ctx - 1 > max(tb, first) ? ctx - 1 : tb;
  const int jb = tb / kBlockTokens;
  const int je = (te + kBlockTokens - 1) / kBlockTokens;

  // The wave's blocks are j = jb + w + 8n, n = 0, 1, ...  Their table
  // entries are read 64 at a time into one register (lane i holds entry n0 + i)
  // so that a tile's address never waits on a dependent load.  The first window
  // is requested before anything else: the first tile loads wait only for it.
  const int32_t* table = a.block_tables + int64_t(b) * a.max_nb;
  int win;
  {
    const int jj = jb + w + kWaves * lane;
    win = jj < je ? table[jj] : -1;
  }

  // Q^T operand: head n of this tile, dims of chunk 4i + q; zero past the group.
  bf16x8_t qop[KI];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.query) + (size_t(b) * a.H + head0 + min(n, nh - 1)) * D;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + query_dim0<E>(i, q));
      if (n >= nh) raw = make_uint4(0u, 0u, 0u, 0u);
      qop[i] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  if (fold && w == 0) fetch_fresh<E, D>(a, b, kvh, lane, sm.fresh, sm.fresh_bad, sm.fresh_scale);

  const S* kc = static_cast<const S*>(a.k_cache);
  const S* vc = static_cast<const S*>(a.v_cache);
  const int64_t tile_elems = int64_t(kBlockTokens) * D;

  MfmaState<D> st;
#pragma unroll
  for (int mc = 0; mc < MC; ++mc) st.o[mc] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  int bad_blk = 0;

  // Block n of this wave's walk, from the current window of table entries
  // (lane i of `win` holds entry n0 + i).  No branch around the loads: an entry
  // outside the pool loads tile 0 instead (always valid memory) and is
  // reported as -1, so every load in the loop below is unconditional and the
  // compiler can keep the next block's loads in flight while one computes.
  int n0 = 0;
  auto fetch = [&](int n, MfmaFrag<E, D>& f) -> int64_t {
    const int p = __builtin_amdgcn_readlane(win, n - n0);
    const bool ok = p >= 0 && p < a.num_blocks;
    const int64_t tile = (int64_t(ok ? p : 0) * a.num_kv_heads + kvh) * tile_elems;
    if constexpr (E::kKind == Kind::kInt8) {
      const int64_t row0 = tile / D;  // the tile's first (block, head, slot) row
      load_block<E, D>(f, kc + tile, vc + tile, lane, row_scales(a.k_cache, a.scales_offset) + row0,
                        row_scales(a.v_cache, a.scales_offset) + row0);
    } else {
      load_block<E, D>(f, kc + tile, vc + tile, lane);
    }
    return ok ? tile : -1;
  };
  auto consume = [&](int j, int64_t tile, const MfmaFrag<E, D>& f) {
    if (tile < 0) { bad_blk = 1; return; }
    const int nvalid = te - j * kBlockTokens;
    const int nfirst = first - j * kBlockTokens;  // > 0 only where a window starts
    if (nvalid >= kBlockTokens && nfirst <= 0)
      compute_block<E, D, false>(f, qop, st, 0, nvalid, a.scale_log2, lane);
    else
      compute_block<E, D, true>(f, qop, st, nfirst, nvalid, a.scale_log2, lane);
  };
  // Ping-pong over two register buffers: block n+1 is in flight while n
  // computes.  Windows of 64 blocks; inside one, every iteration has a next
  // block to fetch (the last one or two are peeled off).
  const int nblk = je - jb - w > 0 ? (je - jb - w + kWaves - 1) / kWaves : 0;
  MfmaFrag<E, D> fa, fb;
  for (; n0 < nblk; n0 += kWave) {
    const int cnt = min(kWave, nblk - n0);
    if (n0 > 0) {
      const int jj = jb + w + kWaves * (n0 + lane);
      win = lane < cnt ? table[jj] : -1;
    }
    int64_t tile_a = fetch(n0, fa), tile_b;
    int n = 0;
    for (; n + 2 < cnt; n += 2) {
      tile_b = fetch(n0 + n + 1, fb);
      consume(jb + w + kWaves * (n0 + n), tile_a, fa);
      tile_a = fetch(n0 + n + 2, fa);
      consume(jb + w + kWaves * (n0 + n + 1), tile_b, fb);
    }
    if (n + 1 < cnt) {
      tile_b = fetch(n0 + n + 1, fb);
      consume(jb + w + kWaves * (n0 + n), tile_a, fa);
      consume(jb + w + kWaves * (n0 + n + 1), tile_b, fb);
    } else {
      consume(jb + w + kWaves * (n0 + n), tile_a, fa);
    }
  }

  if (fold && w == 0) {
    uint4 krow[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i)
      krow[i] = *reinterpret_cast<const uint4*>(&sm.fresh[0][query_dim0<E>(i, q)]);
    float sf = fresh_score<E, D>(krow, qop) * a.scale_log2;
    if constexpr (E::kKind == Kind::kInt8) sf *= sm.fresh_scale[0];  // as the blocks' ks
    if (q == 0) sm.fresh_s[n] = sf;
  }
  const float lsum = cross_row_sum(st.l);
  if (q == 0) {
    sm_m[w][n] = st.m;
    sm_l[w][n] = lsum;
  }
  if (lane == 0) sm_bad[w] = bad_blk;
#pragma unroll
  for (int mc = 0; mc < MC; ++mc)
    *reinterpret_cast<floatx4_t*>(&sm_o[w][n][16 * mc + 4 * q]) = st.o[mc];
  __syncthreads();

  int bad = fold ? sm.fresh_bad : 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) bad |= sm_bad[ww];
  for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
    const int hh = idx / D, x = idx % D;
    float M = fold ? sm.fresh_s[hh] : -INFINITY;  // the newest position: m = its score, l = 1
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if (sm_m[ww][hh] == -INFINITY) continue;
      const float sc = fast_exp2(sm_m[ww][hh] - M);
      L = fmaf(sm_l[ww][hh], sc, L);
      acc = fmaf(sm_o[ww][hh][x], sc, acc);
    }
    if (fold) {
      const float sc = fast_exp2(sm.fresh_s[hh] - M);
      L += sc;
      float v = bf16_to_f32(sm.fresh[1][x]);
      if constexpr (E::kKind == Kind::kInt8) v *= sm.fresh_scale[1];  // as the blocks' vs
      acc = fmaf(v, sc, acc);
    }
    float res = acc / L * a.v_scale;
    if (bad) res = __int_as_float(0x7fc00000);
    if (!split || nparts == 1) {
      out_at(hh, x) = f32_to_bf16_rne(res);
    } else {
      a.ws_o[prow(hh) * D + x] = res;
      if (x == 0) {
        a.ws_m[prow(hh)] = bad ? 0.f : M;
        a.ws_l[prow(hh)] = bad ? 1.f : L;
      }
    }
  }
}

// Split mode: a worker (work-group) takes items i = i0, i0 + G, ... of the
// work list (G workers per head tile) and streams them back to back.  Each
// wave's blocks of one 512-token item are few (4 at 8 waves), so an item that
// only started loading once the previous one had merged its waves' results
// would spend part of its time filling the pipeline.  Here the next item's
// table window is requested when an item starts, and its first block and
// query operand as soon as the item's last block is computed, so the LDS
// merge and the partial's write-out overlap those loads.  Three things keep
// them in flight: the merge's barriers wait for LDS only, none of those loads
// sits behind a branch (the compiler waits for every load in flight where a
// branch holding one rejoins), and the merge loop's stride is a constant
// (blockDim.x is itself a load from the dispatch packet, and waiting for it
// would wait for all the others).  Partitions of more than 64 blocks per wave,
// and fp8 pools, take mfma_item item by item instead.
template <typename E, int D, int kWaves>
__device__ __forceinline__ void mfma_split_worker(const DecodeArgs& a, const int tile_y,
                                                  const int* starts, const int n_items,
                                                  MergeLds<kWaves, D>& sm) {
  constexpr int KI = MfmaShape<D>::KI;
  constexpr int MC = MfmaShape<D>::MC;
  using S = typename E::storage;
  auto& sm_o = sm.o;
  auto& sm_m = sm.m;
  auto& sm_l = sm.l;
  auto& sm_bad = sm.bad;

  const int g = a.H / a.num_kv_heads;
  const int ngroups = (g + kHeadsPerTile - 1) / kHeadsPerTile;
  const int kvh = tile_y / ngroups;
  const int hg = tile_y % ngroups;
  const int head0 = kvh * g + hg * kHeadsPerTile;
  const int nh = min(kHeadsPerTile, g - hg * kHeadsPerTile);
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, q = lane >> 4;
  const S* kc = static_cast<const S*>(a.k_cache);
  const S* vc = static_cast<const S*>(a.v_cache);
  const int64_t tile_elems = int64_t(kBlockTokens) * D;
  const int stride = gridDim.x;

  // An item's uniform description: its sequence, token range and this wave's
  // block count; valid = false past the end of the list.
  struct Item {
    int b, part, ctx, first, nparts, te, jb, nblk;
    bool valid, bad_len, fold;
  };
  auto describe = [&](int i) -> Item {
    Item it{};
    it.valid = i < n_items;
    if (!it.valid) return it;
    locate_item(starts, a.B, i, it.b, it.part);
    it.b = __builtin_amdgcn_readfirstlane(it.b);
    it.part = __builtin_amdgcn_readfirstlane(it.part);
    it.ctx = a.context_lens[it.b];
    it.first = it.ctx > 0 ? window_first(it.ctx - 1, a.window) : 0;
    const int rs = range_start(it.ctx, a.window);
    it.nparts = it.ctx > 0 ? (it.ctx - rs + a.partition_size - 1) / a.partition_size : 0;
    it.bad_len = it.ctx > a.max_nb * kBlockTokens || it.nparts > a.num_partitions;
    const int tb = rs + it.part * a.partition_size;
    it.te = min(tb + a.partition_size, it.ctx);
    // fused step: the last partition takes position ctx - 1 from the fresh rows
    it.fold = a.fresh_key != nullptr && it.part == it.nparts - 1;
    if (it.fold) it.te = it.ctx - 1 > max(tb, it.first) ? it.ctx - 1 : tb;
    it.jb = tb / kBlockTokens;
    const int je = (it.te + kBlockTokens - 1) / kBlockTokens;
    it.nblk = !it.bad_len && je - it.jb - w > 0 ? (je - it.jb - w + kWaves - 1) / kWaves : 0;
    return it;
  };
  // lane i of the window: the table entry of this wave's block i of the item
  // (always loaded, from a clamped index: a load behind a branch makes the
  // compiler wait for every load in flight where the branch rejoins)
  auto load_window = [&](const Item& it) -> int {
    const int jj = min(max(it.jb + w + kWaves * lane, 0), a.max_nb - 1);
    const int e = a.block_tables[int64_t(it.valid ? it.b : 0) * a.max_nb + jj];
    return it.valid && !it.bad_len && lane < it.nblk ? e : -1;
  };
  auto load_query = [&](const Item& it, bf16x8_t (&qop)[KI]) {
    const int bb = it.valid ? it.b : 0;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.query) + (size_t(bb) * a.H + head0 + min(n, nh - 1)) * D;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + query_dim0<E>(i, q));
      if (n >= nh) raw = make_uint4(0u, 0u, 0u, 0u);
      qop[i] = __builtin_bit_cast(bf16x8_t, raw);
    }
  };
  // Block i of the wave's walk through `win`; an entry outside the pool loads
  // tile 0 (valid memory) and is reported as -1.
  auto fetch = [&](int win, int i, MfmaFrag<E, D>& f) -> int64_t {
    const int p = __builtin_amdgcn_readlane(win, i);
    const bool ok = p >= 0 && p < a.num_blocks;
    const int64_t tile = (int64_t(ok ? p : 0) * a.num_kv_heads + kvh) * tile_elems;
    if constexpr (E::kKind == Kind::kInt8) {
      const int64_t row0 = tile / D;
      load_block<E, D>(f, kc + tile, vc + tile, lane, row_scales(a.k_cache, a.scales_offset) + row0,
                        row_scales(a.v_cache, a.scales_offset) + row0);
    } else {
      load_block<E, D>(f, kc + tile, vc + tile, lane);
    }
    return ok ? tile : -1;
  };

  Item cur = describe(blockIdx.x);
  int win = load_window(cur);
  bf16x8_t qop[KI];
  load_query(cur, qop);
  MfmaFrag<E, D> fa, fb;
  int64_t tile_a = fetch(win, 0, fa), tile_b;
  if (cur.nblk == 0) tile_a = -1;

  for (int i = blockIdx.x; i < n_items; i += stride) {
    if constexpr (kGroupsPerCu<E, true> > 1) set_priority((n_items - i + stride - 1) / stride - 1);
    // the next item's table window, in flight while this item streams
    const Item nxt = describe(i + stride);
    const int win_next = load_window(nxt);
    MfmaState<D> st;
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) st.o[mc] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    int bad_blk = 0;
    auto consume = [&](int k, int64_t tile, const MfmaFrag<E, D>& f) {
      bad_blk |= tile < 0;
      const int j = cur.jb + w + kWaves * k;
      const int nvalid = cur.te - j * kBlockTokens;
      const int nfirst = cur.first - j * kBlockTokens;
      if (nvalid >= kBlockTokens && nfirst <= 0)
        compute_block<E, D, false>(f, qop, st, 0, nvalid, a.scale_log2, lane);
      else
        compute_block<E, D, true>(f, qop, st, nfirst, nvalid, a.scale_log2, lane);
    };
    // Ping-pong; block 0 is already in flight in fa.  Once the last block is
    // computed the next item's block 0 and query are requested (requesting
    // them one block earlier needed more registers than the 256 a wave has
    // here and spilled).
    const int cnt = cur.nblk;
    if (cnt > 0) {
      int k = 0;
      for (; k + 2 < cnt; k += 2) {
        tile_b = fetch(win, k + 1, fb);
        consume(k, tile_a, fa);
        tile_a = fetch(win, k + 2, fa);
        consume(k + 1, tile_b, fb);
      }
      if (k + 1 < cnt) {
        tile_b = fetch(win, k + 1, fb);
        consume(k, tile_a, fa);
        consume(k + 1, tile_b, fb);
      } else {
        consume(k, tile_a, fa);
      }
    }
    // Fused step, last partition: wave 0 puts the newest position's K and V
    // rows into LDS as the cache will hold them (fetch_fresh), scores the K row
    // against the current query (qop moves on to the next item below) and
    // leaves score, V row and the table check for the merge.  Nothing else is
    // in flight here (this item's blocks are consumed, the next item's come
    // after), so the loads' wait costs one latency, on the last partitions
    // only.
    if (cur.fold && w == 0) {
      fetch_fresh<E, D>(a, cur.b, kvh, lane, sm.fresh, sm.fresh_bad, sm.fresh_scale);
      uint4 krow[KI];
#pragma unroll
      for (int k = 0; k < KI; ++k)
        krow[k] = *reinterpret_cast<const uint4*>(&sm.fresh[0][query_dim0<E>(k, q)]);
      float sf = fresh_score<E, D>(krow, qop) * a.scale_log2;
      if constexpr (E::kKind == Kind::kInt8) sf *= sm.fresh_scale[0];  // as the blocks' ks
      if (q == 0) sm.fresh_s[n] = sf;
    }
    // unconditional (an entry outside the pool loads tile 0); see load_window
    tile_a = fetch(win_next, 0, fa);
    if (nxt.nblk == 0) tile_a = -1;
    load_query(nxt, qop);

    // merge the waves' (m, l, O) through LDS; the barriers leave the next
    // item's loads in flight
    const float lsum = cross_row_sum(st.l);
    if (q == 0) {
      sm_m[w][n] = st.m;
      sm_l[w][n] = lsum;
    }
    if (lane == 0) sm_bad[w] = bad_blk;
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
      *reinterpret_cast<floatx4_t*>(&sm_o[w][n][16 * mc + 4 * q]) = st.o[mc];
    lds_barrier();
    int bad = cur.bad_len ? 1 : 0;
    if (cur.fold) bad |= sm.fresh_bad;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) bad |= sm_bad[ww];
    uint16_t* out = static_cast<uint16_t*>(a.out);
    for (int idx = threadIdx.x; idx < nh * D; idx += kWaves * kWave) {
      const int hh = idx / D, x = idx % D;
      float M = cur.fold ? sm.fresh_s[hh] : -INFINITY;  // newest position: m = its score, l = 1
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][hh]);
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if (sm_m[ww][hh] == -INFINITY) continue;
        const float sc = fast_exp2(sm_m[ww][hh] - M);
        L = fmaf(sm_l[ww][hh], sc, L);
        acc = fmaf(sm_o[ww][hh][x], sc, acc);
      }
      if (cur.fold) {
        const float sc = fast_exp2(sm.fresh_s[hh] - M);
        L += sc;
        float v = bf16_to_f32(sm.fresh[1][x]);
        if constexpr (E::kKind == Kind::kInt8) v *= sm.fresh_scale[1];  // as the blocks' vs
        acc = fmaf(v, sc, acc);
      }
      float res = acc / L * a.v_scale;
      if (bad) res = __int_as_float(0x7fc00000);
      if (cur.nparts == 1) {
        out[(size_t(cur.b) * a.H + head0 + hh) * D + x] = f32_to_bf16_rne(res);
      } else {
        const size_t row = (size_t(cur.b) * a.H + head0 + hh) * a.num_partitions + cur.part;
        a.ws_o[row * D + x] = res;
        if (x == 0) {
          a.ws_m[row] = bad ? 0.f : M;
          a.ws_l[row] = bad ? 1.f : L;
        }
      }
    }
    lds_barrier();  // the next item reuses the merge buffers

    cur = nxt;
    win = win_next;
  }
}

// Single pass (kSplit = false): grid (1, head tiles, B), one work-group per
// sequence and head tile, sequences taken longest first.  Split (kSplit =
// true): grid (resident workers, head tiles, 1) walking the work list.  Two instantiations keep each one's
// register allocation that of a single inlined item.
//
// Fused step: append_groups more work-groups write the new rows, placed as in
// the vector-ALU kernel (after every decode work-group: z-slabs past the
// sequences of a single pass, y-slabs past the head tiles of a split launch);
// the decode takes the newest position from the fresh rows and never waits
// for them.
template <typename E, int D, bool kSplit>
__global__ __launch_bounds__((kWavesOf<E, kSplit> * kWave),
                             (kGroupsPerCu<E, kSplit>)) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int kWaves = kWavesOf<E, kSplit>;
  __shared__ MergeLds<kWaves, D> sm_merge;
  if constexpr (!kSplit) {
    const int z = blockIdx.z;
    if (a.append_groups > 0 && z >= a.B) {
      append_group<E>(a.append, int64_t(z - a.B) * gridDim.y + blockIdx.y);
      return;
    }
    __shared__ int sm_order[kOrderBuckets + kWaves + 1];
    const int b = a.B <= kMaxOrderedSeqs
        ? sequence_of_rank<kWaves * kWave>(a.context_lens, a.B, a.max_nb, z, sm_order)
        : z;
    mfma_item<E, D, kWaves>(a, 0, blockIdx.y, b, sm_merge);
  } else {
    const int g = a.H / a.num_kv_heads;
    const int tiles = a.num_kv_heads * ((g + kHeadsPerTile - 1) / kHeadsPerTile);
    if (int(blockIdx.y) >= tiles) {
      append_group<E>(a.append, int64_t(blockIdx.y - tiles) * gridDim.x + blockIdx.x);
      return;
    }
    __shared__ int sm_starts[kMaxSplitSeqs + 1];
    const int n_items = build_work_list(a, sm_starts);
    // fp8: the streamed worker measured 2.5% slower on the long-context mix
    // (its items are half the bytes); bf16 2.8% and int8 1.5% faster
    if (E::kKind != Kind::kFp8 && a.partition_size <= kWaves * kWave * kBlockTokens) {
      mfma_split_worker<E, D, kWaves>(a, blockIdx.y, sm_starts, n_items, sm_merge);
      return;
    }
    for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
      if constexpr (kGroupsPerCu<E, kSplit> > 1)
        set_priority((n_items - i + int(gridDim.x) - 1) / int(gridDim.x) - 1);
      int b, part;
      locate_item(sm_starts, a.B, i, b, part);
      mfma_item<E, D, kWaves>(a, part, blockIdx.y, b, sm_merge);
      __syncthreads();  // the next item reuses the merge buffers
    }
  }
}

}  // namespace

template <typename E>
void (*mfma_kernel(int head_dim, bool split))(DecodeArgs) {
  if (head_dim == 128)
    return split ? decode_mfma_kernel<E, 128, true> : decode_mfma_kernel<E, 128, false>;
  if (head_dim == 64)
    return split ? decode_mfma_kernel<E, 64, true> : decode_mfma_kernel<E, 64, false>;
  return nullptr;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, Kind kind, int head_dim, hipStream_t s) {
  const bool split = a.partition_size > 0;
  void (*kern)(DecodeArgs) = kind == Kind::kBf16   ? mfma_kernel<Bf16>(head_dim, split)
                             : kind == Kind::kFp8  ? mfma_kernel<Fp8>(head_dim, split)
                             : kind == Kind::kInt8 ? mfma_kernel<Int8>(head_dim, split)
                                                   : nullptr;
  if (!kern) return hipErrorInvalidValue;
  const int g = a.H / a.num_kv_heads;
  const int tiles = a.num_kv_heads * ((g + kHeadsPerTile - 1) / kHeadsPerTile);
  const bool bytes = kind == Kind::kFp8 || kind == Kind::kInt8;
  const int waves = bytes ? (split ? kWavesOf<Fp8, true> : kWavesOf<Fp8, false>)
                          : (split ? kWavesOf<Bf16, true> : kWavesOf<Bf16, false>);
  const dim3 block(waves * kWave);
  dim3 grid(1, tiles, a.B);
  if (a.partition_size > 0) {
    const int64_t most = int64_t(a.B) * a.num_partitions;
    const int workers = resident_workers(reinterpret_cast<const void*>(kern), block.x, tiles);
    grid = dim3(unsigned(most < workers ? most : workers), tiles, 1);
  }
  DecodeArgs args = a;
  args.append_groups = 0;
  if (a.fresh_key) {  // fused step: add the work-groups of the cache write
    const int64_t need = append_threads(a.append, kind);
    if (a.partition_size > 0) {
      const int64_t slab = int64_t(grid.x) * block.x;
      const int64_t slabs = (need + slab - 1) / slab;
      grid.y += unsigned(slabs);
      args.append_groups = int32_t(slabs * grid.x);
    } else {
      const int64_t slab = int64_t(grid.y) * block.x;
      const int64_t slabs = (need + slab - 1) / slab;
      grid.z += unsigned(slabs);
      args.append_groups = int32_t(slabs * grid.y);
    }
  }
  hipLaunchKernelGGL(kern, grid, block, 0, s, args);
  return hipGetLastError();
}

}  // namespace pagedkv
