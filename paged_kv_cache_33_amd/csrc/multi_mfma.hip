// Attention of several new query tokens per sequence over a paged KV cache,
// causal within them, on the gfx950 matrix cores.
//
// A sequence's n new tokens sit at positions ctx - n .. ctx - 1 and their K/V
// rows are already cached; the token at position p attends to positions 0..p.
// That is the incremental decoder of the "LLM inference and serving" workbook
// (Code from memory) with the rows appended one at a time, evaluated for all n
// rows in one pass: a prompt chunk of chunked prefill ("Anthropic Interview:
// Design an LLM Inference API with GPU Batching", scheduling: a long prompt
// enters in chunks alongside decode steps), or the K draft tokens the target
// model verifies in one pass under speculative decoding ("MLSys Engineer -
// Inference Systems Q&A" and the workbook's speculative-decoding questions).
//
// The 16 columns of an MFMA tile are (token, query head) pairs of one KV head:
// column c is token c / g, head c % g (g = H / H_kv), so each K/V tile read
// from HBM serves every head of the group for up to 16/g tokens at once (or 16
// heads of one token when g > 16).  The per-block arithmetic is the decode
// kernel's (mfma_tile.h) with one more mask: lane column c may see keys up to
// its own position (and, with a sliding window, none before its position
// minus window - 1).  Blocks wholly visible to every column of the tile take
// the unmasked path; blocks wholly before every column's window are skipped.
//
// A wave carries one or two column tiles (a column set): the tiles' query
// operands and running states sit side by side in its registers and every
// K/V block it loads feeds all of them, so K/V bytes are loaded once per 16 or
// 32 columns.  A work-group (4 waves) takes up to 4 consecutive column sets of
// one sequence and KV head.  With s sets in hand (rounded up to 1, 2 or 4),
// 4 / s waves share each set and split its blocks round-robin; their partial
// (m, l, O) merge in LDS as in the decode kernel.  One set (a decode step, or
// draft verification with g * n <= 32) keeps all four waves streaming the
// sequence once; four sets (a long prefill chunk) give each wave its own
// columns, and the four waves read the same K/V blocks at nearly the same
// time, so most of those reads hit in the CU's cache.
#include "device_common.h"
#include "launch.h"
#include "mfma_tile.h"
#include "work_list.h"

namespace pagedkv {
namespace {

constexpr int kMultiWaves = 4;
constexpr int kMaxSetsPerGroup = 4;

// kTiles (1 or 2): 16-column tiles one wave carries.  A wave holds the query
// operands and running state of each of its tiles and feeds them all from
// the same K/V registers, so a block is loaded once for 16 * kTiles columns.
// Both variants run 2 waves per SIMD: the second state costs 48 VGPRs at
// d = 128, and even one tile with its per-column causal and window bounds
// spills at 3 (measured: 3 per SIMD with spills was 8% slower).
template <typename E, int D, int kTiles>
__global__ __launch_bounds__(kMultiWaves* kWave, 2) void multi_mfma_kernel(
    MultiArgs a) {
  using S = typename E::storage;
  constexpr int KI = MfmaShape<D>::KI;
  constexpr int MC = MfmaShape<D>::MC;
  constexpr int kRow = D + 4;  // padded LDS row (floats)
  constexpr int kSetCols = kHeadsPerTile * kTiles;

  __shared__ __attribute__((aligned(16))) float sm_o[kMultiWaves][kSetCols][kRow];
  __shared__ float sm_m[kMultiWaves][kSetCols];
  __shared__ float sm_l[kMultiWaves][kSetCols];
  __shared__ int sm_bad[kMultiWaves];

  // sequences longest first, as in the decode kernel: work-group z takes the
  // z-th longest context
  __shared__ int sm_order[kOrderBuckets + kMultiWaves + 1];
  const int b = a.B <= kMaxOrderedSeqs ? sequence_of_rank<kMultiWaves * kWave>(
                                             a.context_lens, a.B, a.max_nb, blockIdx.z, sm_order)
                                       : int(blockIdx.z);
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, q = lane >> 4;
  const int g = a.H / a.num_kv_heads;

  const int32_t q0 = a.query_start[b], q1 = a.query_start[b + 1];
  // rows outside the buffers: nothing can be read or written for b
  if (q0 < 0 || q1 > a.num_rows || q1 <= q0) return;
  const int nq = q1 - q0;
  const int ctx = a.context_lens[b];
  const int ncols = min(nq, a.max_query_len) * g;  // columns the grid covers
  const int nsets = (ncols + kSetCols - 1) / kSetCols;
  const int s0 = blockIdx.x * a.sets_per_group;
  if (s0 >= nsets) return;
  const int cs = min(a.sets_per_group, nsets - s0);  // 1..4 column sets in hand
  const int wps = cs == 1 ? kMultiWaves : cs == 2 ? kMultiWaves / 2 : 1;  // waves per set
  const int my = w / wps;  // this wave's set in the group
  const int phase = w % wps;

  uint16_t* out = static_cast<uint16_t*>(a.out);
  // Output element (column c, dim x) of this sequence and KV head.
  auto out_at = [&](int c, int x) -> uint16_t& {
    return out[((int64_t(q0) + c / g) * a.H + kvh * g + c % g) * D + x];
  };
  const int cbeg = s0 * kSetCols;
  const int cend = min(cbeg + cs * kSetCols, ncols);

  if (nq > ctx || nq > a.max_query_len || ctx > a.max_nb * kBlockTokens) {
    for (int idx = threadIdx.x; idx < (cend - cbeg) * D; idx += blockDim.x)
      out_at(cbeg + idx / D, idx % D) = 0x7fc0;
    return;
  }

  // This wave's columns: [scb, sce) of set s0 + my (none past the group).
  const bool active = my < cs;
  const int scb = (s0 + my) * kSetCols;
  const int sce = active ? min(scb + kSetCols, ncols) : scb;
  const int pos0 = ctx - nq;  // position of the sequence's first new token
  // Keys every column of the set may see (klo_max .. kmin) and that some
  // column may see (klo .. kend - 1): the first column has the lowest position,
  // the last the highest (with a sliding window both bounds move with it).
  const int kmin = pos0 + scb / g;
  const int kend = active ? pos0 + (sce - 1) / g + 1 : 0;
  const int klo = window_first(kmin, a.window);
  const int klo_max = active ? window_first(kend - 1, a.window) : 0;
  const int jb = klo / kBlockTokens;
  const int je = (kend + kBlockTokens - 1) / kBlockTokens;
  // Tiles of the set that hold columns (uniform): the second may be empty.
  const int ntiles = active ? (sce - scb + kHeadsPerTile - 1) / kHeadsPerTile : 0;

  // Lane column c = scb + 16 tt + n of tile tt: token c / g (it sees lo ..
  // limit, limit its own position), head c % g.  Columns past the set's end
  // take zero queries and see what the last column sees.
  int limit[kTiles], lo[kTiles];
  bf16x8_t qop[kTiles][KI];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const int c = scb + tt * kHeadsPerTile + n;
    const bool col_ok = c < sce;
    limit[tt] = col_ok ? pos0 + c / g : kend - 1;
    lo[tt] = window_first(limit[tt], a.window);
    const int cc = col_ok ? c : scb;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.query) +
                           ((int64_t(q0) + cc / g) * a.H + kvh * g + cc % g) * D;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok) raw = *reinterpret_cast<const uint4*>(qrow + query_dim0<E>(i, q));
      qop[tt][i] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  const int32_t* table = a.block_tables + int64_t(b) * a.max_nb;
  const S* kc = static_cast<const S*>(a.k_cache);
  const S* vc = static_cast<const S*>(a.v_cache);
  const int64_t tile_elems = int64_t(kBlockTokens) * D;

  MfmaState<D> st[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) st[tt].o[mc] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    st[tt].m = -INFINITY;
    st[tt].l = 0.f;
  }
  int bad_blk = 0;

  auto fetch = [&](int p, MfmaFrag<E, D>& f) -> int64_t {
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
    const int key0 = j * kBlockTokens;
    const int nvalid = kend - key0;
    const int nfirst = klo - key0;  // tokens below klo: masked for every column
    const bool open =
        nvalid >= kBlockTokens && key0 + kBlockTokens - 1 <= kmin && key0 >= klo_max;
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
      if (tt > 0 && tt >= ntiles) break;  // uniform: an empty second tile
      if (open)
        compute_block<E, D, false>(f, qop[tt], st[tt], 0, nvalid, a.scale_log2, lane);
      else
        compute_block<E, D, true, true>(f, qop[tt], st[tt], nfirst, nvalid, a.scale_log2, lane,
                                        key0, lo[tt], limit[tt]);
    }
  };
  walk_blocks<MfmaFrag<E, D>>(jb + phase, wps, je, lane, table, fetch, consume);

#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const float lsum = cross_row_sum(st[tt].l);
    const int col = tt * kHeadsPerTile + n;
    if (q == 0) {
      sm_m[w][col] = st[tt].m;
      sm_l[w][col] = lsum;
    }
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
      *reinterpret_cast<floatx4_t*>(&sm_o[w][col][16 * mc + 4 * q]) = st[tt].o[mc];
  }
  if (lane == 0) sm_bad[w] = bad_blk;
  __syncthreads();

  // Merge the waves of each set: column cbeg + idx / D, dim idx % D.
  for (int idx = threadIdx.x; idx < (cend - cbeg) * D; idx += blockDim.x) {
    const int cl = idx / D, x = idx % D;
    const int w0 = (cl / kSetCols) * wps, col = cl % kSetCols;
    float M = -INFINITY;
    int bad = 0;
    for (int ww = w0; ww < w0 + wps; ++ww) {
      M = fmaxf(M, sm_m[ww][col]);
      bad |= sm_bad[ww];
    }
    float L = 0.f, acc = 0.f;
    for (int ww = w0; ww < w0 + wps; ++ww) {
      if (sm_m[ww][col] == -INFINITY) continue;
      const float sc = fast_exp2(sm_m[ww][col] - M);
      L = fmaf(sm_l[ww][col], sc, L);
      acc = fmaf(sm_o[ww][col][x], sc, acc);
    }
    float res = acc / L * a.v_scale;
    if (bad) res = __int_as_float(0x7fc00000);
    out_at(cbeg + cl, x) = f32_to_bf16_rne(res);
  }
}

// s_waitcnt immediate for "at most n vector-memory operations of this wave
// outstanding" (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt at their maxima, i.e. not waited for).
constexpr int vm_wait_imm(int n) {
  return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8);
}

// Wait until at most min(later, L) blocks of kPer loads each are still in
// flight (later is uniform; s_waitcnt takes only an immediate count).
template <int L, int kPer>
__device__ __forceinline__ void wait_vm_later(int later) {
  if constexpr (L == 0) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  } else {
    static_assert(L * kPer < 64, "vmcnt holds 6 bits");
    if (later >= L) __builtin_amdgcn_s_waitcnt(vm_wait_imm(L * kPer));
    else wait_vm_later<L - 1, kPer>(later);
  }
}

// Fourth word of a raw buffer resource (stride 0, byte-addressed range): the
// 32-bit data format, without which the gfx9 family treats every access as
// out of range.
constexpr int kRawBufferWord3 = 0x00020000;

// Byte offset of an LDS object (the low 32 bits of its generic address).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// An int8 block's row scales from its LDS stage, where they follow the two
// tiles (K's 16, then V's); lane (n, q) takes those of token 4q + n % 4 (see
// MfmaScales).
template <typename E, int D, typename F>
__device__ __forceinline__ void load_scales_lds_asm(F& f, uint32_t base, int lane) {
  constexpr int kTileBytes = kBlockTokens * D;
  const uint32_t sa = base + 2 * kTileBytes + uint32_t(4 * (lane >> 4) + (lane & 3)) * 4;
  float ks, vs;
  __asm__ volatile("ds_read_b32 %0, %1" : "=v"(ks) : "v"(sa));
  __asm__ volatile("ds_read_b32 %0, %1 offset:64" : "=v"(vs) : "v"(sa));
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __asm__ volatile("" : "+v"(ks));
  __asm__ volatile("" : "+v"(vs));
  f.ks = ks;
  f.vs = vs;
}

// The K half and the V half of load_block_lds_asm, each with its own wait.
template <typename E, int D>
__device__ __forceinline__ void load_k_lds_asm(MfmaFrag<E, D>& f, uint32_t base, int lane) {
  constexpr int KL = MfmaFrag<E, D>::KL;
  static_assert(E::kChunk * int(sizeof(typename E::storage)) == 16, "16-byte K chunks");
  const uint32_t ka = base + uint32_t(lane) * 16;
  u32x4_t k[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i)
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(k[i]) : "v"(ka), "i"(i * kWave * 16));
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    __asm__ volatile("" : "+v"(k[i]));
    f.k[i] = make_uint4(k[i].x, k[i].y, k[i].z, k[i].w);
  }
}
// V operands mc0 .. mc0 + MC - 1 (all of them by default).
template <typename E, int D, int MC = MfmaShape<D>::MC, int mc0 = 0>
__device__ __forceinline__ void load_v_lds_asm(MfmaFrag<E, D>& f, uint32_t base, int lane) {
  using S = typename E::storage;
  constexpr int kTileBytes = kBlockTokens * D * int(sizeof(S));
  constexpr int kRowStep = 16 * kBlockTokens * int(sizeof(S));  // 16 dims of V
  const int n = lane & 15, q = lane >> 4;
  const uint32_t va = base + kTileBytes + uint32_t(n * kBlockTokens + 4 * q) * uint32_t(sizeof(S));
  if constexpr (MfmaFrag<E, D>::kFp8) {
    uint32_t v[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
      __asm__ volatile("ds_read_b32 %0, %1 offset:%2"
                       : "=v"(v[mc]) : "v"(va), "i"((mc0 + mc) * kRowStep));
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      __asm__ volatile("" : "+v"(v[mc]));
      f.v[mc0 + mc] = v[mc];
    }
  } else {
    u32x2_t v[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
      __asm__ volatile("ds_read_b64 %0, %1 offset:%2"
                       : "=v"(v[mc]) : "v"(va), "i"((mc0 + mc) * kRowStep));
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) {
      __asm__ volatile("" : "+v"(v[mc]));
      f.v[mc0 + mc] = make_uint2(v[mc].x, v[mc].y);
    }
  }
}

// load_block_lds with the LDS reads written out, then a wait for them.  The
// compiler does not see these reads as LDS accesses, so it does not order
// them after the in-flight global-to-LDS loads of later blocks (it cannot tell
// the ring's buffers apart); the explicit block waits and the barrier provide
// that order.  It also takes an asm result as ready at once, so after the wait
// every loaded register passes through an empty volatile statement: volatile
// statements keep their order, so no use can move above the wait.
template <typename E, int D>
__device__ __forceinline__ void load_block_lds_asm(MfmaFrag<E, D>& f, uint32_t base, int lane) {
  load_k_lds_asm<E, D>(f, base, lane);
  load_v_lds_asm<E, D>(f, base, lane);
}

// One 16-byte unit of an int8 block's LDS stage (K units first: chunk u / 16
// of token u % 16, 16 dims; then V rows, 16 tokens each) rewritten as bf16
// into the bf16 tile layouts of the same block, K [d/8][16][8] at cvk and V
// [d][16] at cvv: two 16-byte units.  int8 codes are bf16 values, so the
// operands the products see are exactly those of converting in registers.
// The LDS accesses are written out: the compiler would otherwise order them
// after the stage ring's global-to-LDS loads in flight (see
// load_block_lds_asm).
// (write_int8_unit_lds: the second half, for codes c already read.)
template <int D>
__device__ __forceinline__ void write_int8_unit_lds(u32x4_t c, uint32_t cvk, uint32_t cvv,
                                                    int u) {
  constexpr int kKUnits = kBlockTokens * D / 16;  // int8 K units; bf16 has twice as many
  const u32x4_t lo = {i8x2_to_bf16x2<false>(c.x), i8x2_to_bf16x2<true>(c.x),
                      i8x2_to_bf16x2<false>(c.y), i8x2_to_bf16x2<true>(c.y)};
  const u32x4_t hi = {i8x2_to_bf16x2<false>(c.z), i8x2_to_bf16x2<true>(c.z),
                      i8x2_to_bf16x2<false>(c.w), i8x2_to_bf16x2<true>(c.w)};
  uint32_t a0, a1;  // destination addresses
  if (u < kKUnits) {
    const int c16 = u / kBlockTokens, t = u % kBlockTokens;
    a0 = cvk + uint32_t((2 * c16) * kBlockTokens + t) * 16;
    a1 = a0 + kBlockTokens * 16;
  } else {
    a0 = cvv + uint32_t(2 * (u - kKUnits)) * 16;
    a1 = a0 + 16;
  }
  __asm__ volatile("ds_write_b128 %0, %1" ::"v"(a0), "v"(lo) : "memory");
  __asm__ volatile("ds_write_b128 %0, %1" ::"v"(a1), "v"(hi) : "memory");
}
template <int D>
__device__ __forceinline__ void convert_int8_unit_lds(uint32_t stage, uint32_t cvk, uint32_t cvv,
                                                      int u) {
  u32x4_t c;
  __asm__ volatile("ds_read_b128 %0, %1" : "=v"(c) : "v"(stage + uint32_t(u) * 16));
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __asm__ volatile("" : "+v"(c));
  write_int8_unit_lds<D>(c, cvk, cvv, u);
}

// The four row scales of tokens 4q .. 4q + 3 (lane quarter q) of two blocks'
// K rows, at ka and ka + 64 (16 floats each), and of their V rows, at va and
// va + 64; one wait for the four reads.
__device__ __forceinline__ void read_pair_scales_lds(uint32_t ka, uint32_t va, int lane,
                                                     float (*ks)[4], float (*vs)[4]) {
  const uint32_t off = uint32_t(lane >> 4) * 16;
  u32x4_t r[4];
  __asm__ volatile("ds_read_b128 %0, %1" : "=v"(r[0]) : "v"(ka + off));
  __asm__ volatile("ds_read_b128 %0, %1 offset:64" : "=v"(r[1]) : "v"(ka + off));
  __asm__ volatile("ds_read_b128 %0, %1" : "=v"(r[2]) : "v"(va + off));
  __asm__ volatile("ds_read_b128 %0, %1 offset:64" : "=v"(r[3]) : "v"(va + off));
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __asm__ volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ks[h][0] = __uint_as_float(r[h].x);
    ks[h][1] = __uint_as_float(r[h].y);
    ks[h][2] = __uint_as_float(r[h].z);
    ks[h][3] = __uint_as_float(r[h].w);
    vs[h][0] = __uint_as_float(r[2 + h].x);
    vs[h][1] = __uint_as_float(r[2 + h].y);
    vs[h][2] = __uint_as_float(r[2 + h].z);
    vs[h][3] = __uint_as_float(r[2 + h].w);
  }
}

// Two consecutive 16-token blocks a, b (keys key0 .. key0 + 31), read from
// their LDS stages sa, sb, for kT column tiles, with one 32-deep product per
// output tile for P V.  The contraction runs over the 32 keys in the order
// lane quarter q holds them: tokens 4q..4q+3 of a, then tokens 4q..4q+3 of b.
// That is where the score accumulators of S_a = K_a Q^T and S_b = K_b Q^T
// already put them (register j: token 4q + j), and where the V^T operand
// takes them from the two token-minor V tiles (8 bytes of each for bf16), so
// a pair needs no lane exchange and half the P V instructions of two 16-deep
// products.  The softmax runs once over both blocks (one reference max for
// the pair).  bf16 and fp8 pools, and int8 pools converted to bf16.  The
// work comes in three parts, so a caller can compute the next pair's scores
// while this pair's weights and products run: pair_scores, pair_rescale,
// pair_pv.
//
// pair_scores: the raw scores s[h][tt] (h = 0: block a, 1: block b).  To
// stay within 256 VGPRs at two waves per SIMD the operands are read in
// stages: K of a, its products; K of b, its products.
template <typename E, int D, int kT>
__device__ __forceinline__ void pair_scores(uint32_t sa, uint32_t sb,
                                            const bf16x8_t (*qop)[MfmaShape<D>::KI],
                                            floatx4_t (*s)[kT], int lane) {
  static_assert(!(E::kKind == Kind::kInt8 && kByteCodes<E>), "int8 codes are converted first");
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    MfmaFrag<E, D> f;
    load_k_lds_asm<E, D>(f, h ? sb : sa, lane);
#pragma unroll
    for (int tt = 0; tt < kT; ++tt) s[h][tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MfmaShape<D>::KI; ++i) {
      const bf16x8_t kop = k_operand<E, D>(f, i);
#pragma unroll
      for (int tt = 0; tt < kT; ++tt)
        s[h][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[tt][i], s[h][tt], 0, 0, 0);
    }
  }
}

// pair_rescale: with kScaled (int8 pools) each score times its key row's
// scale ks[h][j] (token 4q + j of block h); masks (as in compute_block_tiles,
// with nfirst / nvalid relative to the pair's first token: -inf by select, the
// slot may hold NaN), then the reference max: when some score exceeds it by
// more than the slack, the state is rescaled (wave-uniform branch, as in
// compute_block_tiles).
//
// thr (optional): per column tile, (m + slack) / scale_log2, the reference in
// raw score units, kept up to date here; the test then compares raw maxima
// (two fewer instructions per tile, as m changes only in the rare rescale).
template <int D, bool kTail, bool kCausal, int kT, bool kScaled = false>
__device__ __forceinline__ void pair_rescale(floatx4_t (*s)[kT], MfmaState<D>* st, int nfirst,
                                             int nvalid, float scale_log2, int lane, int key0,
                                             const int* lo, const int* limit,
                                             const float (*ks)[4] = nullptr,
                                             float* thr = nullptr) {
  constexpr int MC = MfmaShape<D>::MC;
  const int q = lane >> 4;
  float lmax[kT];
  bool exceeds = false;
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 16 * h + 4 * q + j;  // token within the pair
        if constexpr (kScaled) s[h][tt][j] *= ks[h][j];
        const bool masked = (kTail && (t >= nvalid || t < nfirst)) ||
                            (kCausal && (key0 + t > limit[tt] || key0 + t < lo[tt]));
        if (masked) s[h][tt][j] = -INFINITY;
      }
    lmax[tt] = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(
            __builtin_elementwise_maximum(s[0][tt][0], s[0][tt][1]),
            __builtin_elementwise_maximum(s[0][tt][2], s[0][tt][3])),
        __builtin_elementwise_maximum(
            __builtin_elementwise_maximum(s[1][tt][0], s[1][tt][1]),
            __builtin_elementwise_maximum(s[1][tt][2], s[1][tt][3])));
    if (thr) {
      exceeds = exceeds || lmax[tt] > thr[tt];
    } else {
      lmax[tt] *= scale_log2;
      exceeds = exceeds || lmax[tt] > st[tt].m + kRescaleSlack;
    }
  }
  if (__builtin_amdgcn_ballot_w64(exceeds) != 0) {
#pragma unroll
    for (int tt = 0; tt < kT; ++tt) {
      const float mx = cross_row_max(lmax[tt]) * (thr ? scale_log2 : 1.f);
      const bool grow = mx > st[tt].m + kRescaleSlack;
      const float alpha = grow ? fast_exp2(st[tt].m - mx) : 1.f;
      st[tt].l *= alpha;
#pragma unroll
      for (int mc = 0; mc < MC; ++mc) st[tt].o[mc] *= alpha;
      st[tt].m = grow ? mx : st[tt].m;
      if (thr) thr[tt] = (st[tt].m + kRescaleSlack) / scale_log2;
    }
  }
}

// pair_pv: the weights 2^(s scale - m) as bf16, their row sums, and
// O^T += V^T P^T, the V operands read in two halves of the dims, each
// followed by its products.  With kTail the V of tokens outside the range
// is zeroed (weight 0 times NaN would be NaN).  kScaled (int8 pools): the
// products take each weight times its token's V row scale vs[h][j] (0 where
// masked, as the scale may be NaN there); the row sums take the weights alone.
template <typename E, int D, bool kTail, bool kCausal, int kT, bool kScaled = false>
__device__ __forceinline__ void pair_pv(uint32_t sa, uint32_t sb, const floatx4_t (*s)[kT],
                                        MfmaState<D>* st, int nfirst, int nvalid,
                                        float scale_log2, int lane,
                                        const float (*vs)[4] = nullptr) {
  constexpr int MC = MfmaShape<D>::MC;
  const int q = lane >> 4;
  bf16x8_t pop[kT];
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
    const float mref = (kCausal && st[tt].m == -INFINITY) ? 0.f : st[tt].m;
    uint32_t pk[4], pkv[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pw[j] = fast_exp2(__builtin_fmaf(s[h][tt][j], scale_log2, -mref));
      pk[2 * h] = pack_bf16x2(pw[0], pw[1]);
      pk[2 * h + 1] = pack_bf16x2(pw[2], pw[3]);
      if constexpr (kScaled) {
        float pv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pv[j] = ((kTail || kCausal) && s[h][tt][j] == -INFINITY) ? 0.f : pw[j] * vs[h][j];
        pkv[2 * h] = pack_bf16x2(pv[0], pv[1]);
        pkv[2 * h + 1] = pack_bf16x2(pv[2], pv[3]);
      }
    }
    constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
    float l = st[tt].l;
#pragma unroll
    for (int k = 0; k < 4; ++k) l = dot2_bf16(pk[k], kOnes, l);
    st[tt].l = l;
    if constexpr (kScaled)
      pop[tt] = __builtin_bit_cast(bf16x8_t, make_uint4(pkv[0], pkv[1], pkv[2], pkv[3]));
    else
      pop[tt] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  }
  auto pv = [&](const MfmaFrag<E, D>& fa, const MfmaFrag<E, D>& fb, int mc) {
    uint2 va = v_operand<E, D>(fa, mc), vb = v_operand<E, D>(fb, mc);
    if (kTail) {
      const int t = 4 * q;
      va.x = zero_masked_pair(va.x, t >= nfirst && t < nvalid, t + 1 >= nfirst && t + 1 < nvalid);
      va.y = zero_masked_pair(va.y, t + 2 >= nfirst && t + 2 < nvalid,
                              t + 3 >= nfirst && t + 3 < nvalid);
      const int u = 16 + 4 * q;
      vb.x = zero_masked_pair(vb.x, u >= nfirst && u < nvalid, u + 1 >= nfirst && u + 1 < nvalid);
      vb.y = zero_masked_pair(vb.y, u + 2 >= nfirst && u + 2 < nvalid,
                              u + 3 >= nfirst && u + 3 < nvalid);
    }
    const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
#pragma unroll
    for (int tt = 0; tt < kT; ++tt)
      st[tt].o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[tt], st[tt].o[mc], 0, 0, 0);
  };
  {
    MfmaFrag<E, D> fa, fb;
    load_v_lds_asm<E, D, MC / 2, 0>(fa, sa, lane);
    load_v_lds_asm<E, D, MC / 2, 0>(fb, sb, lane);
#pragma unroll
    for (int mc = 0; mc < MC / 2; ++mc) pv(fa, fb, mc);
  }
  {
    MfmaFrag<E, D> fa, fb;
    load_v_lds_asm<E, D, MC / 2, MC / 2>(fa, sa, lane);
    load_v_lds_asm<E, D, MC / 2, MC / 2>(fb, sb, lane);
#pragma unroll
    for (int mc = MC / 2; mc < MC; ++mc) pv(fa, fb, mc);
  }
}

// LDS reads written out without their wait: the K pieces of a block's stage
// (as load_k_lds_asm), and V pieces mc0 .. mc0 + H - 1 (as load_v_lds_asm).
// kl / vl: the lane's K / V address in stage 0, kOff the stage's byte offset
// (an immediate of the read).  wait_lds<N> then waits until at most N of this
// wave's LDS operations are outstanding (they complete in order); the
// registers a wait covers pass through an empty volatile statement after it,
// so no use moves above it.
template <typename E, int D>
using VRaw = std::conditional_t<MfmaFrag<E, D>::kFp8, uint32_t, u32x2_t>;
template <int KL, uint32_t kOff>
__device__ __forceinline__ void issue_k_lds(u32x4_t (&k)[KL], uint32_t kl) {
#pragma unroll
  for (int i = 0; i < KL; ++i)
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2"
                     : "=v"(k[i]) : "v"(kl), "i"(kOff + i * kWave * 16));
}
template <typename E, int D, int H, int mc0, uint32_t kOff>
__device__ __forceinline__ void issue_v_lds(VRaw<E, D> (&v)[H], uint32_t vl) {
  constexpr int kRowStep = 16 * kBlockTokens * int(sizeof(typename E::storage));  // 16 dims
#pragma unroll
  for (int mc = 0; mc < H; ++mc) {
    if constexpr (MfmaFrag<E, D>::kFp8)
      __asm__ volatile("ds_read_b32 %0, %1 offset:%2"
                       : "=v"(v[mc]) : "v"(vl), "i"(kOff + (mc0 + mc) * kRowStep));
    else
      __asm__ volatile("ds_read_b64 %0, %1 offset:%2"
                       : "=v"(v[mc]) : "v"(vl), "i"(kOff + (mc0 + mc) * kRowStep));
  }
}
template <int N>
__device__ __forceinline__ void wait_lds() {
  static_assert(N >= 0 && N < 16, "lgkmcnt holds 4 bits");
  __asm__ volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T, int N>
__device__ __forceinline__ void pin(T (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) __asm__ volatile("" : "+v"(r[i]));
}

// One step of the software-pipelined pair loop, for pairs every column sees
// whole (no masks): the scores of the next pair (stages at byte offsets kNa,
// kNb) into sn, and the weights and P V products of the current pair (scores
// sc, already rescaled for; stages kCa, kCb).  All LDS reads of the step are
// issued at its start (K of the next pair, then the first half of the
// current pair's V; the second half once the first K has landed), so the
// waits find them mostly done, and the exponentials of the current weights
// have no dependence on any of them.  kScaled (int8 pools, the blocks
// converted to bf16): the products take each weight times its token's V row
// scale vs[h][j], the row sums the weights alone (as pair_pv).
template <typename E, int D, int kT, uint32_t kNa, uint32_t kNb, uint32_t kCa, uint32_t kCb,
          bool kScaled = false>
__device__ __forceinline__ void pair_pipelined(uint32_t kl, uint32_t vl,
                                               const bf16x8_t (*qop)[MfmaShape<D>::KI],
                                               const floatx4_t (*sc)[kT], floatx4_t (*sn)[kT],
                                               MfmaState<D>* st, float scale_log2,
                                               const float (*vs)[4] = nullptr) {
  constexpr int KL = MfmaFrag<E, D>::KL;
  constexpr int MC = MfmaShape<D>::MC;
  constexpr int H = MC / 2;
  static_assert(KL + 2 * H < 16, "outstanding LDS reads fit lgkmcnt");
  u32x4_t kr[2][KL];
  VRaw<E, D> v1[2][H], v2[2][H];
  issue_k_lds<KL, kNa>(kr[0], kl);
  issue_k_lds<KL, kNb>(kr[1], kl);
  issue_v_lds<E, D, H, 0, kCa>(v1[0], vl);
  issue_v_lds<E, D, H, 0, kCb>(v1[1], vl);
  // the current pair's weights and their row sums
  bf16x8_t pop[kT];
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
    const float mref = st[tt].m;
    uint32_t pk[4], pkv[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pw[j] = fast_exp2(__builtin_fmaf(sc[h][tt][j], scale_log2, -mref));
      pk[2 * h] = pack_bf16x2(pw[0], pw[1]);
      pk[2 * h + 1] = pack_bf16x2(pw[2], pw[3]);
      if constexpr (kScaled) {
        pkv[2 * h] = pack_bf16x2(pw[0] * vs[h][0], pw[1] * vs[h][1]);
        pkv[2 * h + 1] = pack_bf16x2(pw[2] * vs[h][2], pw[3] * vs[h][3]);
      }
    }
    constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
    float l = st[tt].l;
#pragma unroll
    for (int k = 0; k < 4; ++k) l = dot2_bf16(pk[k], kOnes, l);
    st[tt].l = l;
    if constexpr (kScaled)
      pop[tt] = __builtin_bit_cast(bf16x8_t, make_uint4(pkv[0], pkv[1], pkv[2], pkv[3]));
    else
      pop[tt] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  }
  // the next pair's scores, block by block as its K lands
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 0) wait_lds<KL + 2 * H>();
    else wait_lds<2 * H>();
    pin(kr[h]);
    MfmaFrag<E, D> f;
#pragma unroll
    for (int i = 0; i < KL; ++i) f.k[i] = make_uint4(kr[h][i].x, kr[h][i].y, kr[h][i].z, kr[h][i].w);
#pragma unroll
    for (int tt = 0; tt < kT; ++tt) sn[h][tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MfmaShape<D>::KI; ++i) {
      const bf16x8_t kop = k_operand<E, D>(f, i);
#pragma unroll
      for (int tt = 0; tt < kT; ++tt)
        sn[h][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[tt][i], sn[h][tt], 0, 0, 0);
    }
  }
  // the current pair's products, the V halves in turn
  auto pv = [&](const VRaw<E, D>& ra, const VRaw<E, D>& rb, int mc) {
    MfmaFrag<E, D> fa, fb;
    if constexpr (MfmaFrag<E, D>::kFp8) {
      fa.v[mc] = ra;
      fb.v[mc] = rb;
    } else {
      fa.v[mc] = make_uint2(ra.x, ra.y);
      fb.v[mc] = make_uint2(rb.x, rb.y);
    }
    const uint2 va = v_operand<E, D>(fa, mc), vb = v_operand<E, D>(fb, mc);
    const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
#pragma unroll
    for (int tt = 0; tt < kT; ++tt)
      st[tt].o[mc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[tt], st[tt].o[mc], 0, 0, 0);
  };
  // The compiler checks no hazard against registers an asm statement writes,
  // and the score products above may still be reading their accumulator
  // operands from registers these reads reuse: 16 wait states first.
  __asm__ volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  issue_v_lds<E, D, H, H, kCa>(v2[0], vl);
  issue_v_lds<E, D, H, H, kCb>(v2[1], vl);
  wait_lds<2 * H>();
  pin(v1[0]);
  pin(v1[1]);
#pragma unroll
  for (int mc = 0; mc < H; ++mc) pv(v1[0][mc], v1[1][mc], mc);
  wait_lds<0>();
  pin(v2[0]);
  pin(v2[1]);
#pragma unroll
  for (int mc = 0; mc < H; ++mc) pv(v2[0][mc], v2[1][mc], H + mc);
}

// The whole pair: scores, masks and rescale, weights and products.  int8
// pools (E = Int8AsBf16: the blocks converted to bf16 at sa, sb): the row
// scales come from the blocks' ring stages ra, rb, where they follow the two
// code tiles (K's 16, then V's); lane quarter q reads tokens 4q..4q+3 of each.
template <typename E, int D, bool kTail, bool kCausal, int kT>
__device__ __forceinline__ void compute_pair_lds(uint32_t sa, uint32_t sb,
                                                 const bf16x8_t (*qop)[MfmaShape<D>::KI],
                                                 MfmaState<D>* st, int nfirst, int nvalid,
                                                 float scale_log2, int lane, int key0,
                                                 const int* lo, const int* limit,
                                                 uint32_t ra = 0, uint32_t rb = 0) {
  constexpr bool kScaled = E::kKind == Kind::kInt8;
  floatx4_t s[2][kT];
  pair_scores<E, D, kT>(sa, sb, qop, s, lane);
  if constexpr (kScaled) {
    constexpr uint32_t kCodes = 2 * kBlockTokens * D;  // both int8 code tiles
    const uint32_t off = kCodes + uint32_t(lane >> 4) * 16;
    // four scales of each block, K's before the rescale, V's before the
    // products (so they are not held at once)
    auto read4 = [&](uint32_t addr, float (*x)[4]) {
      u32x4_t r[2];
      __asm__ volatile("ds_read_b128 %0, %1" : "=v"(r[0]) : "v"(ra + addr));
      __asm__ volatile("ds_read_b128 %0, %1" : "=v"(r[1]) : "v"(rb + addr));
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      pin(r);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x[h][0] = __uint_as_float(r[h].x);
        x[h][1] = __uint_as_float(r[h].y);
        x[h][2] = __uint_as_float(r[h].z);
        x[h][3] = __uint_as_float(r[h].w);
      }
    };
    float ks[2][4], vs[2][4];
    read4(off, ks);
    pair_rescale<D, kTail, kCausal, kT, true>(s, st, nfirst, nvalid, scale_log2, lane, key0, lo,
                                              limit, ks);
    read4(off + 64, vs);
    pair_pv<E, D, kTail, kCausal, kT, true>(sa, sb, s, st, nfirst, nvalid, scale_log2, lane, vs);
  } else {
    pair_rescale<D, kTail, kCausal, kT>(s, st, nfirst, nvalid, scale_log2, lane, key0, lo, limit);
    pair_pv<E, D, kTail, kCausal, kT>(sa, sb, s, st, nfirst, nvalid, scale_log2, lane);
  }
}

// Several column sets per sequence and KV head (a prefill chunk, or draft
// verification with 33..64 columns).  Each wave owns one set of 16 * kTiles
// columns (kTiles = 2 for prefill chunks, 1 for verification: three
// work-groups per CU) and walks every block its columns see, two blocks at a
// time; the waves of a work-group need nearly the same blocks (their
// positions differ by at most 128 / g tokens), so the work-group loads each
// block once, cooperatively, into an LDS ring of six or eight stages (direct
// global-to-LDS loads, two pairs ahead), and every wave reads its operands
// there; with fewer than four sets the idle waves only load (and, for int8
// pools, convert).
// The K/V of a sequence is read by all of its work-groups, so these loads are
// ordinary (cached) ones.  No partial results meet: a wave finishes its own
// columns.
template <typename E, int D, int kTiles>
__global__ __launch_bounds__(kMultiWaves* kWave, kTiles == 1 ? 3 : 2) void chunk_mfma_kernel(
    MultiArgs a) {
  using S = typename E::storage;
  constexpr int KI = MfmaShape<D>::KI;
  constexpr int MC = MfmaShape<D>::MC;
  constexpr int kSetCols = kHeadsPerTile * kTiles;
  constexpr int kThreads = kMultiWaves * kWave;
  constexpr int kTileElems = kBlockTokens * D;
  constexpr bool kInt8 = E::kKind == Kind::kInt8;
  constexpr int kTileUnits = kTileElems * int(sizeof(S)) / 16;    // 16-byte units of one tile
  // a stage: K tile, V tile, and for int8 the 16 K then 16 V row scales
  constexpr int kScaleUnits = kBlockTokens * int(sizeof(float)) / 16;  // per tile
  constexpr int kUnits = 2 * kTileUnits + (kInt8 ? 2 * kScaleUnits : 0);
  // bf16 / fp8: wave w loads units 64w + kThreads k.  int8: wave w loads
  // code units kCodeUnits w .. + kCodeUnits - 1 (all K or all V), then two of
  // the eight scale units (waves 0, 1 K's, waves 2, 3 V's), so every wave
  // issues the same number of loads per block.
  constexpr int kCodeUnits = 2 * kTileUnits / kMultiWaves;
  static_assert(kTileUnits % kCodeUnits == 0 && kScaleUnits == kMultiWaves, "int8 stage split");
  constexpr int kPer = kInt8 ? (kCodeUnits + kWave - 1) / kWave + 1
                             : (kUnits + kThreads - 1) / kThreads;  // loads per thread per block
  // Blocks are computed in pairs (one 32-deep P V product per pair;
  // compute_pair_lds).  Measured against single blocks: 512-token prefill
  // chunks 0.975 -> 0.866 ms (bf16), 1.052 -> 0.957 ms (fp8); verification of
  // 8 draft tokens at g = 8, 528 -> 518 us (bf16), 416 -> 380 us (fp8).  One
  // tile per wave stays at three work-groups per CU.
  // The table window: int8 pools take a smaller one, so three work-groups
  // with one tile per wave fit a CU with their bf16 buffers (below).
  constexpr int kTabWin = kInt8 ? 512 : 1024;
  // bf16 and fp8 pairs on the software-pipelined path (see below) take eight
  // stages where the work-groups of a CU still fit its 160 KiB of LDS (two
  // with two tiles per wave, three with one); the others six.
  constexpr int kStageBytes = kUnits * 16;
  constexpr bool kPipe =
      !kInt8 && (kTiles == 2 ? 2 : 3) * (8 * kStageBytes + 4 * kTabWin + 1024) <= 160 * 1024;
  constexpr int kStages = kPipe ? 8 : 6;
  __shared__ uint4 sm_kv[kStages][kUnits];
  __shared__ int sm_tab[kTabWin];
  // int8: the blocks are converted to bf16 once per work-group (each
  // thread one or two 16-byte units of codes per block) into sm_cv, and the
  // waves take their operands from there (C, the compute type, keeps the row
  // scales).  sm_cv holds six bf16 tiles, with kBT the bytes of one:
  //   [K a][V a, slot 0][K b][V b, slot 0][V a, slot 1][V b, slot 1]
  // then the row scales: K's of a, b (16 floats each), V's of slot 0, V's of
  // slot 1.  A pair converted for the general loop below takes the first four
  // tiles (block a's K and V adjacent, as is b's) and keeps its row scales in
  // the ring stages; the pipelined path converts each pair one pair ahead, K
  // into the K tiles and V into the slot the pair being computed does not
  // read, with the row scales beside them.
  constexpr bool kConvert = kInt8;
  using C = std::conditional_t<kConvert, Int8AsBf16, E>;
  constexpr int kCvUnits = 2 * kTileElems * 2 / 16;  // one bf16 block, K and V
  constexpr uint32_t kBT = kTileElems * 2;            // one bf16 tile
  constexpr int kCvScaleUnits = 3 * 2 * kScaleUnits;   // K's, V's of two slots
  __shared__ uint4 sm_cv[kConvert ? 3 * kCvUnits + kCvScaleUnits : 1];

  __shared__ int sm_order[kOrderBuckets + kMultiWaves + 1];
  const int b = __builtin_amdgcn_readfirstlane(
      a.B <= kMaxOrderedSeqs
          ? sequence_of_rank<kThreads>(a.context_lens, a.B, a.max_nb, blockIdx.z, sm_order)
          : int(blockIdx.z));
  const int kvh = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  __builtin_assume(w >= 0 && w < kMultiWaves);
  const int n = lane & 15, q = lane >> 4;
  const int g = a.H / a.num_kv_heads;

  const int32_t q0 = a.query_start[b], q1 = a.query_start[b + 1];
  if (q0 < 0 || q1 > a.num_rows || q1 <= q0) return;
  const int nq = q1 - q0;
  const int ctx = a.context_lens[b];
  const int ncols = min(nq, a.max_query_len) * g;
  const int nsets = (ncols + kSetCols - 1) / kSetCols;
  const int s0 = blockIdx.x * kMultiWaves;
  if (s0 >= nsets) return;
  const int cs = min(kMultiWaves, nsets - s0);

  // element offset of column c's row (token c / g, head c % g) in query / out
  auto row_at = [&](int c) -> int64_t {
    return ((int64_t(q0) + c / g) * a.H + kvh * g + c % g) * D;
  };
  uint16_t* out = static_cast<uint16_t*>(a.out);
  const uint16_t* query = static_cast<const uint16_t*>(a.query);
  const int cbeg = s0 * kSetCols;
  const int cend = min(cbeg + cs * kSetCols, ncols);
  if (nq > ctx || nq > a.max_query_len || ctx > a.max_nb * kBlockTokens) {
    for (int idx = tid; idx < (cend - cbeg) * D; idx += kThreads)
      out[row_at(cbeg + idx / D) + idx % D] = 0x7fc0;
    return;
  }

  const bool active = w < cs;
  const int scb = (s0 + w) * kSetCols;
  const int sce = active ? min(scb + kSetCols, ncols) : scb;
  const int pos0 = ctx - nq;
  const int kmin = pos0 + scb / g;
  const int kend = active ? pos0 + (sce - 1) / g + 1 : 0;
  const int klo = window_first(kmin, a.window);
  const int klo_max = active ? window_first(kend - 1, a.window) : 0;
  const int ntiles = active ? (sce - scb + kHeadsPerTile - 1) / kHeadsPerTile : 0;
  // the work-group's blocks: wave 0 sees the lowest positions, the last set
  // the highest
  const int wjb = window_first(pos0 + cbeg / g, a.window) / kBlockTokens;
  const int wje = (pos0 + (cend - 1) / g + 1 + kBlockTokens - 1) / kBlockTokens;

  int limit[kTiles], lo[kTiles];
  bool col_ok[kTiles];
  bf16x8_t qop[kTiles][KI];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const int c = scb + tt * kHeadsPerTile + n;
    col_ok[tt] = c < sce;
    limit[tt] = col_ok[tt] ? pos0 + c / g : kend - 1;
    lo[tt] = window_first(limit[tt], a.window);
    const uint16_t* qrow = query + row_at(col_ok[tt] ? c : scb);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (col_ok[tt]) raw = *reinterpret_cast<const uint4*>(qrow + query_dim0<C>(i, q));
      qop[tt][i] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  MfmaState<D> st[kTiles];
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) st[tt].o[mc] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    st[tt].m = -INFINITY;
    st[tt].l = 0.f;
  }
  int bad = 0;

  const int32_t* table = a.block_tables + int64_t(b) * a.max_nb;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  constexpr int64_t kTileBytes = int64_t(kTileElems) * sizeof(S);
  // Block j's two tiles arrive in LDS by direct global-to-LDS loads
  // (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at the wave's
  // LDS address + 16 i), kStages - 1 blocks ahead of the block computing, so
  // several blocks are in flight without holding registers.  A stage holds
  // the K tile's units, then V's (then, for int8, the row scales); the units
  // of one wave-wide load are all K, all V or all scales of one tile.
  // Block j's ring stage, counted from the work-group's first block (so a
  // loop that advances eight blocks per trip sees the same stages every trip).
  auto stage_of = [&](int jj) { return unsigned(jj - wjb) % kStages; };
  auto stage_addr = [&](int jj) { return lds_offset(&sm_kv[stage_of(jj)][0]); };
  // e: the block's table word as staged (see fill_tab): its tile's index, bit
  // 31 set for an entry outside the pool (whose tile index is then kvh's in
  // block 0, loaded but never used).
  auto issue = [&](unsigned stage, int e) {
    const int64_t pt = int64_t(e & 0x7fffffff);  // tile index p H_kv + kvh
    const int64_t tile = pt * kTileBytes;
    uint4* ring = &sm_kv[stage][0];
    if constexpr (kInt8) {
      // the tile's 16 row scales: floats 16 (p H_kv + kvh) .. of the scale region
      const int cu0 = w * kCodeUnits;  // uniform: all K or all V
      const char* src = (cu0 < kTileUnits ? kc : vc) + pt * kTileBytes +
                        int64_t((cu0 % kTileUnits) + lane) * 16;
#pragma unroll
      for (int k = 0; k < kPer - 1; ++k)
        if (lane < kCodeUnits - k * kWave)  // d = 64: half a wave-load
          __builtin_amdgcn_global_load_lds(
              src + k * kWave * 16,
              (__attribute__((address_space(3))) void*)(ring + cu0 + k * kWave), 16, 0, 0);
      const int su0 = 2 * w;  // scale units su0, su0 + 1: 0..3 K's, 4..7 V's
      const char* ssrc = (w < kMultiWaves / 2 ? kc : vc) + a.scales_offset +
                         pt * kBlockTokens * int64_t(sizeof(float)) +
                         ((su0 % kScaleUnits) + lane) * 16;
      if (lane < 2)
        __builtin_amdgcn_global_load_lds(
            ssrc, (__attribute__((address_space(3))) void*)(ring + 2 * kTileUnits + su0), 16, 0,
            0);
    } else {
      // Buffer loads: the tile's address in a resource (scalar registers), the
      // wave's first unit a scalar offset and the lane's 16 bytes a vector
      // offset that never changes, so no lane holds a 64-bit address.
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int u0 = w * kWave + k * kThreads;  // uniform
        if (u0 < kUnits) {
          const bool is_k = u0 < kUnits / 2;
          const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<char*>((is_k ? kc : vc) + tile), 0, int(kTileBytes), kRawBufferWord3);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsrc, (__attribute__((address_space(3))) void*)(ring + u0), 16, lane * 16,
              (is_k ? u0 : u0 - kUnits / 2) * 16, 0, 0);
        }
      }
    }
  };

  // the query operands are in registers before any block load is issued
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  // The table entries of the work-group's blocks are staged in LDS, kTabWin at
  // a time, so the loop below consumes no vector-load result (the compiler
  // would wait for every load in flight before one); a refill (one barrier
  // that drains the loads in flight) comes once per kTabWin blocks.
  // Each word is validated as it is staged: the tile index p H_kv + kvh of
  // the entry p, or kvh's tile of block 0 with bit 31 set where p lies outside
  // the pool (the launch checks that tile indices fit 31 bits).
  int tb = wjb;
  int any_bad = 0;  // some word staged so far lay outside the pool
  auto fill_tab = [&]() {
    // (the first block through readfirstlane: the compiler then keeps no
    // pointer per call site stepping along with the loops that call it)
    const int32_t* row = table + __builtin_amdgcn_readfirstlane(tb);
    int inval = 0;
    for (int i = tid; i < kTabWin && tb + i < wje; i += kThreads) {
      const int p = row[i];
      const bool ok = p >= 0 && p < a.num_blocks;
      sm_tab[i] = ((ok ? p : 0) * a.num_kv_heads + kvh) | (ok ? 0 : int(0x80000000u));
      inval |= ok ? 0 : 1;
    }
    any_bad |= __syncthreads_or(inval);
  };
  fill_tab();
  // The words of blocks wb .. wb + 63 in a register (lane i: block wb + i),
  // read from sm_tab once per 64 blocks; a block's word is then one lane read,
  // with no LDS wait.
  int wb = -(1 << 30), win = 0;
  auto table_word = [&](int jn) -> int {  // uniform
    if (jn - tb >= kTabWin) {
      tb = jn;
      fill_tab();
      wb = -(1 << 30);
    }
    if (jn - wb >= kWave) {
      wb = jn;
      const int i = jn - tb + lane;
      win = i < kTabWin ? sm_tab[i] : 0;
    }
    return __builtin_amdgcn_readlane(win, jn - wb);
  };
  // Block j of the wave's range, alone: the per-block arithmetic.
  // (operands: where block j's K and V are, in the layout of C)
  auto single = [&](int j, uint32_t operands) {
    const int key0 = j * kBlockTokens;
    if (!(active && key0 < kend && key0 + kBlockTokens > klo)) return;  // uniform per wave
    MfmaFrag<C, D> f;
    const uint32_t stage = stage_addr(j);
    load_block_lds_asm<C, D>(f, operands, lane);
    if constexpr (kInt8) load_scales_lds_asm<E, D>(f, stage, lane);
    const int nvalid = kend - key0;
    const int nfirst = klo - key0;
    const bool open =
        nvalid >= kBlockTokens && key0 + kBlockTokens - 1 <= kmin && key0 >= klo_max;
    // The branch encloses the tiles' work, so the masked path's (the V
    // operands' masking, shared by the tiles) stays inside it instead of
    // being computed ahead of the branch for every block.  Both tiles run
    // phase by phase in one pass; a set with one tile of columns runs one.
    if (kTiles == 1 || ntiles == kTiles) {
      if (open)
        compute_block_tiles<C, D, false, false, kTiles>(f, qop, st, 0, nvalid, a.scale_log2, lane,
                                                        0, lo, limit);
      else
        compute_block_tiles<C, D, true, true, kTiles>(f, qop, st, nfirst, nvalid, a.scale_log2,
                                                      lane, key0, lo, limit);
    } else {
      if (open)
        compute_block_tiles<C, D, false, false, 1>(f, qop, st, 0, nvalid, a.scale_log2, lane, 0,
                                                   lo, limit);
      else
        compute_block_tiles<C, D, true, true, 1>(f, qop, st, nfirst, nvalid, a.scale_log2, lane,
                                                 key0, lo, limit);
    }
  };
  auto issue_at = [&](int jn) {  // uniform
    issue(stage_of(jn), table_word(jn));
  };
  // int8: blocks jj and jj + 1 (if in the range) in bf16 into sm_cv (after
  // the barrier that makes them visible, before the one that hands them to
  // the waves); where each one's operands are
  const uint32_t cv0 = lds_offset(&sm_cv[0]);
  auto convert_pair = [&](int jj) {
    if constexpr (kConvert) {
      const int units = (jj + 1 < wje ? 2 : 1) * 2 * kTileUnits;
      for (int u = tid; u < units; u += kThreads) {
        const int h = u / (2 * kTileUnits);
        const uint32_t cvk = cv0 + uint32_t(h) * kCvUnits * 16;
        convert_int8_unit_lds<D>(stage_addr(jj + h), cvk, cvk + kBT, u - h * 2 * kTileUnits);
      }
    }
  };
  auto operands_of = [&](int jj, int h) {  // block jj + h (h = 0, 1)
    return kConvert ? cv0 + uint32_t(h) * kCvUnits * 16 : stage_addr(jj + h);
  };
  {
    // blocks wjb .. wjb + 3 in flight; at pair (j, j + 1) the two after it
    // may still be loading
    for (int t = 0; t < kStages - 2 && wjb + t < wje; ++t) issue_at(wjb + t);
    int j = wjb;
    // First the pairs every column of the work-group sees whole (all of a
    // prefill chunk's or a verification's blocks but those on its diagonal):
    // one straight path, an active wave computing all its tiles (a partial
    // set computes on zero queries and writes nothing; a block whose entry
    // lies outside the pool computes on tile 0 and turns the columns NaN), an
    // inactive one only keeping the loads and barriers in step.  With the
    // branches of the general loop below (open or masked pair, a single
    // block, nothing) the compiler moved the output accumulators between
    // registers at every join: about 100 moves per pair.
    {
      const int kmin_wg = pos0 + cbeg / g;                                // first column's position
      const int klo_wg = window_first(pos0 + (cend - 1) / g, a.window);  // last column's first key
      auto open = [&](int jj) {
        return jj + 1 < wje && jj * kBlockTokens >= klo_wg &&
               jj * kBlockTokens + 2 * kBlockTokens - 1 <= kmin_wg;
      };
      if constexpr (kPipe) {
        // Software-pipelined: while pair j's weights and P V products run, the
        // scores of pair j + 2 are computed, so a wave has matrix products
        // independent of its exponentials.  Eight stages (four pairs): at pair
        // j the scores need pair j + 2 in LDS, pair j's V is still read, and
        // the pair issued (j + 6, j + 7) reuses the stages of pair j - 2,
        // which every wave has finished once past the barrier.  Invariant at
        // the top of an iteration: blocks below j + kStages - 2 are issued.
        if (open(j)) {
          // Iterations: pairs j = wjb, wjb + 2, ... while pair j + 2 is whole
          // for every column and blocks j + 6, j + 7 exist (so both issues
          // happen and exactly two blocks load after pair j + 2's: a fixed
          // count to wait for).  open(wjb) already holds the window bound.
          const int jmax = min(wje - 8, ((kmin_wg - (2 * kBlockTokens - 1)) >> 4) - 2);
          const int n_iter = jmax >= j ? (jmax - j) / 2 + 1 : 0;
          // stage byte offsets and the lane's addresses in stage 0
          const uint32_t ring0 = lds_offset(&sm_kv[0][0]);
          const uint32_t kl = ring0 + uint32_t(lane) * 16;
          const uint32_t vl = ring0 + uint32_t(kTileBytes) +
                              uint32_t((n * kBlockTokens + 4 * q) * int(sizeof(S)));
          // blocks jn, jn + 1 (both in the range) into stages kS, kS + 1: one
          // window check for the two table words
          auto issue_pair = [&](int jn, auto stag) {
            constexpr unsigned kS = decltype(stag)::value;
            if (jn + 1 - tb >= kTabWin) {
              tb = jn;
              fill_tab();
              wb = -(1 << 30);
            }
            if (jn + 1 - wb >= kWave) {
              wb = jn;
              const int i = jn - tb + lane;
              win = i < kTabWin ? sm_tab[i] : 0;
            }
            const int e0 = __builtin_amdgcn_readlane(win, jn - wb);
            const int e1 = __builtin_amdgcn_readlane(win, jn + 1 - wb);
            issue(kS, e0);
            issue(kS + 1, e1);
          };
          auto run = [&](auto act) {
            constexpr bool kAct = decltype(act)::value;
            // the state's reference in raw score units (the state is fresh:
            // m = -inf)
            float thr[kTiles];
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) thr[tt] = (st[tt].m + kRescaleSlack) / a.scale_log2;
            auto rescale = [&](floatx4_t (*sc)[kTiles]) {
              pair_rescale<D, false, false, kTiles>(sc, st, 0, 2 * kBlockTokens, a.scale_log2,
                                                    lane, 0, lo, limit, nullptr, thr);
            };
            // pair j landed; the blocks after it may still be loading
            wait_vm_later<kStages - 4, kPer>(min(kStages - 4, max(wje - 2 - j, 0)));
            lds_barrier();
            floatx4_t s0[2][kTiles], s1[2][kTiles];
            if constexpr (kAct) {
              pair_scores<C, D, kTiles>(stage_addr(j), stage_addr(j + 1), qop, s0, lane);
              rescale(s0);
            }
            // Iteration M (mod 4) of the path: pair j (stages 2M, 2M + 1 of
            // the ring, counted from wjb) has its scores, rescaled for, in sc.
            // The rescale for pair j + 2 comes last, after pair j's products,
            // as the output accumulators then pass one branch per pair, in
            // place.
            auto iter = [&](auto mtag, floatx4_t (*sc)[kTiles], floatx4_t (*sn)[kTiles]) {
              constexpr unsigned M = decltype(mtag)::value;
              constexpr unsigned kStage = kStageBytes;
              __builtin_amdgcn_s_waitcnt(vm_wait_imm((kStages - 6) * kPer));
              lds_barrier();
              issue_pair(j + kStages - 2, std::integral_constant<unsigned, (2 * M + 6) % 8>{});
              if constexpr (kAct) {
                pair_pipelined<C, D, kTiles, ((2 * M + 2) % 8) * kStage, ((2 * M + 3) % 8) * kStage,
                               (2 * M) * kStage, (2 * M + 1) * kStage>(kl, vl, qop, sc, sn, st,
                                                                       a.scale_log2);
                rescale(sn);
              }
              j += 2;
            };
            // the last pair of the path: its weights and products, and the
            // issue that keeps the invariant of the general loop below
            auto last = [&](floatx4_t (*sc)[kTiles]) {
              lds_barrier();
              if (j + kStages - 2 < wje) issue_at(j + kStages - 2);
              if (j + kStages - 1 < wje) issue_at(j + kStages - 1);
              if constexpr (kAct) {
                pair_pv<C, D, false, false, kTiles>(stage_addr(j), stage_addr(j + 1), sc, st, 0,
                                                    2 * kBlockTokens, a.scale_log2, lane);
              }
              j += 2;
            };
            using I0 = std::integral_constant<unsigned, 0>;
            using I1 = std::integral_constant<unsigned, 1>;
            using I2 = std::integral_constant<unsigned, 2>;
            using I3 = std::integral_constant<unsigned, 3>;
            // Four iterations per trip: the stages repeat, and the score
            // buffers swap roles without copies.  Then two more if at least
            // two are left (the stages of a trip's first half); the one pair
            // that may remain goes through the general loop below.  Every path
            // ends on the same score buffer: a remainder of one or three taken
            // here put the accumulators through joins the compiler resolved
            // by spilling.
            int it = 0;
            for (; it + 4 <= n_iter; it += 4) {
              iter(I0{}, s0, s1);
              iter(I1{}, s1, s0);
              iter(I2{}, s0, s1);
              iter(I3{}, s1, s0);
            }
            if (it + 2 <= n_iter) {
              iter(I0{}, s0, s1);
              iter(I1{}, s1, s0);
            }
            last(s0);
          };
          if (active) run(std::true_type{});
          else run(std::false_type{});
        }
      } else if constexpr (kConvert) {
        // int8, software-pipelined as above on the bf16 copies: at pair j the
        // work-group converts pair j + 2 (K into the K tiles, V into the slot
        // pair j does not read, the row scales beside them), then each wave
        // computes pair j + 2's scores and pair j's weights and products.
        // Six ring stages: pair j + 2 converting, pair j + 4 loading, and the
        // pair issued, j + 6, takes the stages of pair j, converted one pair
        // earlier.  Invariant at the top of an iteration: blocks below j + 6
        // are issued.  Two barriers per pair: one before the conversion (pair
        // j + 2 landed for every wave, every wave done with what the
        // conversion overwrites), one after it.
        if (open(j)) {
          // Iterations: pairs j = wjb, wjb + 2, ... while pair j + 2 is whole
          // for every column and blocks j + 6, j + 7 exist; an even count, so
          // that every path ends on the same score buffer and V slot.
          const int jmax = min(wje - 8, ((kmin_wg - (2 * kBlockTokens - 1)) >> 4) - 2);
          const int n_iter = jmax >= j ? ((jmax - j) / 2 + 1) & ~1 : 0;
          const uint32_t kl = cv0 + uint32_t(lane) * 16;
          const uint32_t vl = cv0 + uint32_t((n * kBlockTokens + 4 * q) * 2);
          constexpr uint32_t kScaleBytes = kBlockTokens * sizeof(float);  // one tile's
          const uint32_t ks0 = cv0 + 6 * kBT;  // K row scales of a, then b
          auto vs_at = [&](int slot) { return ks0 + uint32_t(1 + slot) * 2 * kScaleBytes; };
          // All LDS reads of a thread's share first (its code units, and for
          // threads 0..15 one unit of row scales), one wait, then the writes.
          auto convert_ahead = [&](int jn, int slot) {
            constexpr int kBlockUnits = 2 * kTileUnits;  // code units of one block
            constexpr int kU = (2 * kBlockUnits + kThreads - 1) / kThreads;
            static_assert(2 * kBlockUnits % kThreads == 0, "every thread converts kU units");
            u32x4_t c[kU], sc;
#pragma unroll
            for (int k = 0; k < kU; ++k) {
              const int u = tid + k * kThreads, h = u / kBlockUnits;
              __asm__ volatile("ds_read_b128 %0, %1"
                               : "=v"(c[k])
                               : "v"(stage_addr(jn + h) + uint32_t(u - h * kBlockUnits) * 16));
            }
            const bool copies = tid < 4 * kScaleUnits;  // (block h, unit r: K's, then V's)
            const int sh = tid / (2 * kScaleUnits), sr = tid % (2 * kScaleUnits);
            if (copies)
              __asm__ volatile("ds_read_b128 %0, %1"
                               : "=v"(sc)
                               : "v"(stage_addr(jn + sh) + uint32_t(2 * kTileUnits + sr) * 16));
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int k = 0; k < kU; ++k) {
              __asm__ volatile("" : "+v"(c[k]));
              const int u = tid + k * kThreads, h = u / kBlockUnits;
              const uint32_t vt = cv0 + uint32_t(slot ? 4 + h : 1 + 2 * h) * kBT;
              write_int8_unit_lds<D>(c[k], cv0 + uint32_t(2 * h) * kBT, vt, u - h * kBlockUnits);
            }
            if (copies) {
              __asm__ volatile("" : "+v"(sc));
              const uint32_t to = (sr < kScaleUnits ? ks0 : vs_at(slot)) +
                                  uint32_t(sh) * kScaleBytes + uint32_t(sr % kScaleUnits) * 16;
              __asm__ volatile("ds_write_b128 %0, %1" ::"v"(to), "v"(sc) : "memory");
            }
          };
          auto run = [&](auto act) {
            constexpr bool kAct = decltype(act)::value;
            float thr[kTiles];
#pragma unroll
            for (int tt = 0; tt < kTiles; ++tt) thr[tt] = (st[tt].m + kRescaleSlack) / a.scale_log2;
            // vcur: the V row scales of the pair whose products come next
            float vcur[2][4];
            // the pair converted last (its V in `slot`): its scores' rescale,
            // and its V row scales into vcur
            auto rescale = [&](floatx4_t (*sc)[kTiles], int slot) {
              float ks[2][4];
              read_pair_scales_lds(ks0, vs_at(slot), lane, ks, vcur);
              pair_rescale<D, false, false, kTiles, true>(sc, st, 0, 2 * kBlockTokens,
                                                          a.scale_log2, lane, 0, lo, limit, ks, thr);
            };
            // pair j landed (the two blocks after it may still be loading)
            wait_vm_later<kStages - 4, kPer>(min(kStages - 4, max(wje - 2 - j, 0)));
            lds_barrier();
            convert_ahead(j, 0);
            if (j + 4 < wje) issue_at(j + 4);
            if (j + 5 < wje) issue_at(j + 5);
            lds_barrier();
            floatx4_t s0[2][kTiles], s1[2][kTiles];
            if constexpr (kAct) {
              pair_scores<C, D, kTiles>(cv0, cv0 + 2 * kBT, qop, s0, lane);
              rescale(s0, 0);
            }
            // iteration M (mod 2): pair j's V in slot M, its scores in sc
            auto iter = [&](auto mtag, floatx4_t (*sc)[kTiles], floatx4_t (*sn)[kTiles]) {
              constexpr unsigned M = decltype(mtag)::value;
              __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kPer));  // pair j + 2 landed
              lds_barrier();
              issue_at(j + 6);
              issue_at(j + 7);
              convert_ahead(j + 2, 1 - M);
              lds_barrier();
              if constexpr (kAct) {
                pair_pipelined<C, D, kTiles, 0, 2 * kBT, (M ? 4 : 1) * kBT, (M ? 5 : 3) * kBT,
                               true>(kl, vl, qop, sc, sn, st, a.scale_log2, vcur);
                rescale(sn, 1 - M);
              }
              j += 2;
            };
            using I0 = std::integral_constant<unsigned, 0>;
            using I1 = std::integral_constant<unsigned, 1>;
            for (int it = 0; it < n_iter; it += 2) {
              iter(I0{}, s0, s1);
              iter(I1{}, s1, s0);
            }
            // the last pair of the path (V in slot 0): its weights and products
            if constexpr (kAct)
              pair_pv<C, D, false, false, kTiles, true>(cv0, cv0 + 2 * kBT, s0, st, 0,
                                                        2 * kBlockTokens, a.scale_log2, lane, vcur);
            j += 2;
          };
          if (active) run(std::true_type{});
          else run(std::false_type{});
        }
      } else {
        auto step = [&](int jj) {
          wait_vm_later<kStages - 4, kPer>(min(kStages - 4, max(wje - 2 - jj, 0)));
          lds_barrier();
          if (jj + kStages - 2 < wje) issue_at(jj + kStages - 2);
          if (jj + kStages - 1 < wje) issue_at(jj + kStages - 1);
        };
        if (active) {
          for (; open(j); j += 2) {
            step(j);
            compute_pair_lds<C, D, false, false, kTiles>(stage_addr(j), stage_addr(j + 1), qop, st,
                                                         0, 2 * kBlockTokens, a.scale_log2, lane,
                                                         0, lo, limit);
          }
        } else {
          for (; open(j); j += 2) step(j);
        }
      }
    }
    for (; j < wje; j += 2) {
      wait_vm_later<kStages - 4, kPer>(min(kStages - 4, max(wje - 2 - j, 0)));
      // blocks j, j + 1 are in LDS for every wave, and every wave is done with
      // the previous pair, whose buffers the next issues reuse
      lds_barrier();
      if (j + kStages - 2 < wje) issue_at(j + kStages - 2);
      if (j + kStages - 1 < wje) issue_at(j + kStages - 1);
      if constexpr (kConvert) {
        convert_pair(j);
        lds_barrier();  // the bf16 blocks are complete
      }
      const uint32_t sa = operands_of(j, 0);
      const uint32_t sb = operands_of(j, 1);
      const uint32_t ra = stage_addr(j), rb = stage_addr(j + 1);
      const int key0 = j * kBlockTokens;
      const bool in_a = active && key0 < kend && key0 + kBlockTokens > klo;
      const bool in_b = j + 1 < wje && active && key0 + kBlockTokens < kend &&
                        key0 + 2 * kBlockTokens > klo;
      if (in_a && in_b) {  // uniform per wave
        const int nvalid = kend - key0;
        const int nfirst = klo - key0;
        const bool open =
            nvalid >= 2 * kBlockTokens && key0 + 2 * kBlockTokens - 1 <= kmin && key0 >= klo_max;
        if (ntiles == kTiles) {
          if (open)
            compute_pair_lds<C, D, false, false, kTiles>(sa, sb, qop, st, 0, nvalid,
                                                         a.scale_log2, lane, 0, lo, limit, ra, rb);
          else
            compute_pair_lds<C, D, true, true, kTiles>(sa, sb, qop, st, nfirst, nvalid,
                                                       a.scale_log2, lane, key0, lo, limit, ra,
                                                       rb);
        } else {
          if (open)
            compute_pair_lds<C, D, false, false, 1>(sa, sb, qop, st, 0, nvalid, a.scale_log2,
                                                    lane, 0, lo, limit, ra, rb);
          else
            compute_pair_lds<C, D, true, true, 1>(sa, sb, qop, st, nfirst, nvalid, a.scale_log2,
                                                  lane, key0, lo, limit, ra, rb);
        }
      } else if (in_a) {
        single(j, sa);
      } else if (in_b) {
        single(j + 1, sb);
      }
    }
  }

  // A staged table word lay outside the pool: the wave's columns turn NaN if
  // their keys reach such a block (the blocks of positions klo .. kend - 1,
  // all of which the loops above computed, a bad one on tile 0).  Rare, so
  // the entries are read again here instead of tracked block by block.
  if (any_bad && active) {
    int inval = 0;
    for (int jj = klo / kBlockTokens + lane; jj * kBlockTokens < kend; jj += kWave) {
      const int p = table[jj];
      inval |= (p >= 0 && p < a.num_blocks) ? 0 : 1;
    }
    bad = __builtin_amdgcn_ballot_w64(inval != 0) != 0 ? 1 : 0;
  }

  // Each wave finishes its own columns: lane (q, n) holds dims 16mc + 4q .. +3
  // of column n.
#pragma unroll
  for (int tt = 0; tt < kTiles; ++tt) {
    const float L = cross_row_sum(st[tt].l);
    if (!active || !col_ok[tt]) continue;
    uint16_t* orow = out + row_at(scb + tt * kHeadsPerTile + n);
    const float inv = a.v_scale / L;
    // (the hardware's conversion rounds to nearest even, as f32_to_bf16_rne)
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
      *reinterpret_cast<uint2*>(orow + 16 * mc + 4 * q) =
          bad ? make_uint2(0x7fc07fc0u, 0x7fc07fc0u)
              : make_uint2(pack_bf16x2(st[tt].o[mc][0] * inv, st[tt].o[mc][1] * inv),
                           pack_bf16x2(st[tt].o[mc][2] * inv, st[tt].o[mc][3] * inv));
  }
}

template <typename E, int kTiles>
void (*chunk_kernel(int head_dim))(MultiArgs) {
  if (head_dim == 128) return chunk_mfma_kernel<E, 128, kTiles>;
  if (head_dim == 64) return chunk_mfma_kernel<E, 64, kTiles>;
  return nullptr;
}

template <typename E, int kTiles>
void (*multi_kernel(int head_dim))(MultiArgs) {
  if (head_dim == 128) return multi_mfma_kernel<E, 128, kTiles>;
  if (head_dim == 64) return multi_mfma_kernel<E, 64, kTiles>;
  return nullptr;
}

template <typename E>
void (*multi_kernel(int head_dim, int tiles))(MultiArgs) {
  return tiles == 1 ? multi_kernel<E, 1>(head_dim) : multi_kernel<E, 2>(head_dim);
}

}  // namespace

hipError_t launch_multi_mfma(const MultiArgs& a, Kind kind, int head_dim, hipStream_t s) {
  if (a.tiles_per_set < 1 || a.tiles_per_set > 2 || a.sets_per_group < 1 ||
      a.sets_per_group > kMaxSetsPerGroup)
    return hipErrorInvalidValue;
  // tile indices p H_kv + kvh are staged as 31-bit words
  if (int64_t(a.num_blocks) * a.num_kv_heads > (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int g = a.H / a.num_kv_heads;
  const int64_t set_cols = int64_t(kHeadsPerTile) * a.tiles_per_set;
  const int64_t sets = (int64_t(a.max_query_len) * g + set_cols - 1) / set_cols;
  // The LDS-staged kernel loads each block once for all columns of a
  // work-group.  Measured against the per-wave kernel: 21% faster on 512-token
  // prefill chunks of a bf16 pool and 11% for fp8 (two tiles per wave, four
  // sets).  With 3 or 4 tiles of columns (draft verification with g * K of
  // 33..64) each of the four waves takes one tile (148 VGPRs: three
  // work-groups per CU): against two waves with two tiles each, 12% faster for
  // bf16 at K = 8, g = 8, and against the per-wave kernel 11-22% faster for
  // fp8 and 2-10% for int8 (whose stages add the row scales).  One tile per
  // wave measured slower with two tiles of columns (8%, bf16) and on fp8
  // prefill chunks (2.5%), and equal on bf16 prefill chunks.  int8 pools take
  // it since their blocks are converted to bf16 once per work-group (two tiles
  // per wave then fit 256 VGPRs): 512-token prefill chunks 1.456 -> 1.298 ms
  // against the per-wave kernel.
  const int64_t tiles = (int64_t(a.max_query_len) * g + kHeadsPerTile - 1) / kHeadsPerTile;
  const bool chunk1 = tiles >= 3 && tiles <= kMultiWaves;
  const bool chunk = !chunk1 && a.tiles_per_set == 2 &&
                     ((kind == Kind::kBf16 && sets >= 2) ||
                      ((kind == Kind::kFp8 || kind == Kind::kInt8) && sets >= kMultiWaves));
  const bool bf16 = kind == Kind::kBf16;
  void (*kern)(MultiArgs) =
      chunk1  ? (bf16                 ? chunk_kernel<Bf16, 1>(head_dim)
                 : kind == Kind::kFp8 ? chunk_kernel<Fp8, 1>(head_dim)
                 : kind == Kind::kInt8 ? chunk_kernel<Int8, 1>(head_dim)
                                       : nullptr)
      : chunk ? (bf16                 ? chunk_kernel<Bf16, 2>(head_dim)
                 : kind == Kind::kFp8 ? chunk_kernel<Fp8, 2>(head_dim)
                                      : chunk_kernel<Int8, 2>(head_dim))
              : (bf16                  ? multi_kernel<Bf16>(head_dim, a.tiles_per_set)
                 : kind == Kind::kFp8  ? multi_kernel<Fp8>(head_dim, a.tiles_per_set)
                 : kind == Kind::kInt8 ? multi_kernel<Int8>(head_dim, a.tiles_per_set)
                                       : nullptr);
  if (!kern) return hipErrorInvalidValue;
  if (a.B == 0 || a.max_query_len == 0) return hipSuccess;
  const int64_t per_group = chunk1 || chunk ? kMultiWaves : a.sets_per_group;
  const int64_t groups =
      chunk1 ? (tiles + kMultiWaves - 1) / kMultiWaves : (sets + per_group - 1) / per_group;
  hipLaunchKernelGGL(kern, dim3(unsigned(groups), unsigned(a.num_kv_heads), unsigned(a.B)),
                     dim3(kMultiWaves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
