// Paged decode attention on the vector ALUs: one query head per work-group.
//
// What it computes ("MLSys Engineer - Inference Systems Q&A", Q1 and Q4; the
// "LLM inference and serving" workbook's incremental decoder): for query head h
// of sequence b, out = softmax_t(scale * q . K[t]) V[t] over the ctx tokens of
// the sequence, K[t] and V[t] read through the block table.  Scores stay in
// registers; a running max and denominator are rescaled whenever the max
// rises (online softmax); everything accumulates in fp32.
//
// Work decomposition: a work-group of 8 wavefronts takes one (partition, query
// head, sequence); wave w walks the partition's blocks w, w+8, w+16, ...
// keeping its own (m, l, O), and the eight are merged through LDS at the end.
// The next block's K and V are loaded while the current one is computed.
//
// Lane mapping for one 16-token block (see the pool layout in pagedkv.h):
//   K tile [d/X][16][X]: load i gives lane l the 16-byte chunk 4i + l/16 of
//     token l%16; each lane forms a partial dot over its chunks, and two
//     cross-row shuffles complete the score of token l%16 in every row.
//   V tile [d][16]: lane l owns dims l and l+64; each 16-byte load gives it X
//     consecutive tokens of one dim, and the tokens are the same for every lane,
//     so the 16 probabilities are broadcast once per block (readlane) and
//     each lane does plain fp32 FMAs.
#include "device_common.h"
#include "launch.h"
#include "row_write.h"
#include "work_list.h"

namespace pagedkv {
namespace {

constexpr int kWaves = 8;

template <typename Tr, int D>
struct ValuShape {
  static constexpr int X = Tr::kChunk;  // elements per 16-byte chunk
  static constexpr int C = D / X;       // chunks per token row
  static constexpr int KL = C / 4;      // K loads per lane per block
  static constexpr int XK = D / 64;     // output dims per lane
  static constexpr int R = 16 / X;      // 16-byte pieces per V row (16 tokens)
  static constexpr int VL = XK * R;     // V loads per lane per block
};

// int8 caches also carry the K and V scales of the lane's token (l % 16).
template <typename Tr, bool kScaled = Tr::kKind == Kind::kInt8>
struct RowScales {
  float ks, vs;
};
template <typename Tr>
struct RowScales<Tr, false> {};

template <typename Tr, int D>
struct BlockFrag : RowScales<Tr> {
  uint4 k[ValuShape<Tr, D>::KL];
  uint4 v[ValuShape<Tr, D>::VL];
};

// ksr / vsr: the tile's 16 row scales (int8 caches only).
template <typename Tr, int D>
__device__ __forceinline__ void load_block(BlockFrag<Tr, D>& f, const typename Tr::storage* kt,
                                           const typename Tr::storage* vt, int lane,
                                           const float* ksr = nullptr,
                                           const float* vsr = nullptr) {
  using Sh = ValuShape<Tr, D>;
  if constexpr (Tr::kKind == Kind::kInt8) {
    f.ks = __builtin_nontemporal_load(ksr + (lane & 15));
    f.vs = __builtin_nontemporal_load(vsr + (lane & 15));
  }
#pragma unroll
  for (int i = 0; i < Sh::KL; ++i)
    f.k[i] = load_tile16(kt + (i * kWave + lane) * Sh::X);
#pragma unroll
  for (int xk = 0; xk < Sh::XK; ++xk)
#pragma unroll
    for (int th = 0; th < Sh::R; ++th)
      f.v[xk * Sh::R + th] =
          load_tile16(vt + ((xk * kWave + lane) * kBlockTokens + th * Sh::X));
}

struct WaveState {
  float m;    // running max (base-2 units), uniform across the wave
  float l;    // this lane's share of the denominator (token lane%16)
};

// The query slice a lane contracts with: the dims of K chunks 4i + lane/16 of
// the head row.  bf16 keeps the stored pairs (the dot2 instruction takes them
// as they are); fp32 keeps floats; an fp8 cache's 16-element chunk pairs with
// 16 bf16 query values, two 16-byte pieces.
template <typename Tr, int D>
struct QueryFrag {
  static constexpr int kPieces = kByteCodes<Tr> ? 2 : 1;
  uint4 c[ValuShape<Tr, D>::KL][kPieces];
};

// One 16-byte piece of 16 one-byte codes (E4M3 or int8) as 8 bf16 pairs (lo:
// codes 0..7, hi: codes 8..15), exact.
template <Kind kK>
__device__ __forceinline__ void codes16_to_bf16(const uint4& v, uint4& lo, uint4& hi) {
  lo = make_uint4(code2_to_bf16x2<kK, false>(v.x), code2_to_bf16x2<kK, true>(v.x),
                  code2_to_bf16x2<kK, false>(v.y), code2_to_bf16x2<kK, true>(v.y));
  hi = make_uint4(code2_to_bf16x2<kK, false>(v.z), code2_to_bf16x2<kK, true>(v.z),
                  code2_to_bf16x2<kK, false>(v.w), code2_to_bf16x2<kK, true>(v.w));
}

// Zero the bf16 V values of tokens outside [nfirst, nvalid) inside one 16-byte
// piece holding tokens first..first+7 of one dim (the same tokens in every
// lane).
__device__ __forceinline__ uint4 mask_tokens(uint4 v, int first, int nfirst, int nvalid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t0 = first + 2 * c;
    const bool keep_lo = t0 >= nfirst && t0 < nvalid;
    const bool keep_hi = t0 + 1 >= nfirst && t0 + 1 < nvalid;
    w[c] = (keep_lo ? (w[c] & 0x0000ffffu) : 0u) | (keep_hi ? (w[c] & 0xffff0000u) : 0u);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One block of 16 tokens.  With kTail only tokens nfirst .. nvalid-1 (uniform
// bounds) are inside the range: the block holding the end of the range, or the
// first position of a sliding window.
template <typename Tr, int D, bool kTail>
__device__ __forceinline__ void compute_block(const BlockFrag<Tr, D>& f, const QueryFrag<Tr, D>& qf,
                                              float (&o)[ValuShape<Tr, D>::XK], WaveState& st,
                                              int nfirst, int nvalid, float scale_log2, int lane) {
  using Sh = ValuShape<Tr, D>;
  constexpr bool kBytes = kByteCodes<Tr>;             // one-byte codes, converted to bf16
  constexpr bool kInt8 = Tr::kKind == Kind::kInt8;    // per-token row scales
  constexpr bool kPacked = Tr::kKind != Kind::kF32;  // bf16 pairs into dot2
  // ---- scores: this lane's chunks of token lane%16, then the 4 rows combined
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < Sh::KL; ++i) {
    if constexpr (kBytes) {
      uint4 klo, khi;
      codes16_to_bf16<Tr::kKind>(f.k[i], klo, khi);
      dot = dot2_bf16(klo.x, qf.c[i][0].x, dot);
      dot = dot2_bf16(klo.y, qf.c[i][0].y, dot);
      dot = dot2_bf16(klo.z, qf.c[i][0].z, dot);
      dot = dot2_bf16(klo.w, qf.c[i][0].w, dot);
      dot = dot2_bf16(khi.x, qf.c[i][1].x, dot);
      dot = dot2_bf16(khi.y, qf.c[i][1].y, dot);
      dot = dot2_bf16(khi.z, qf.c[i][1].z, dot);
      dot = dot2_bf16(khi.w, qf.c[i][1].w, dot);
    } else if constexpr (kPacked) {
      dot = dot2_bf16(f.k[i].x, qf.c[i][0].x, dot);
      dot = dot2_bf16(f.k[i].y, qf.c[i][0].y, dot);
      dot = dot2_bf16(f.k[i].z, qf.c[i][0].z, dot);
      dot = dot2_bf16(f.k[i].w, qf.c[i][0].w, dot);
    } else {
      dot = fmaf(__uint_as_float(f.k[i].x), __uint_as_float(qf.c[i][0].x), dot);
      dot = fmaf(__uint_as_float(f.k[i].y), __uint_as_float(qf.c[i][0].y), dot);
      dot = fmaf(__uint_as_float(f.k[i].z), __uint_as_float(qf.c[i][0].z), dot);
      dot = fmaf(__uint_as_float(f.k[i].w), __uint_as_float(qf.c[i][0].w), dot);
    }
  }
  dot = cross_row_sum(dot);
  const int t = lane & 15;
  float s = dot * scale_log2;
  if constexpr (kInt8) s *= f.ks;  // the token's K row scale
  const bool masked = kTail && (t >= nvalid || t < nfirst);
  if (masked) s = -INFINITY;  // select: the slot may hold NaN
  // ---- online softmax over the block's 16 tokens (one per lane of a row)
  const float m_new = fmaxf(st.m, row16_max(s));
  const float alpha = fast_exp2(st.m - m_new);
  const float p = fast_exp2(s - m_new);
  st.m = m_new;
#pragma unroll
  for (int xk = 0; xk < Sh::XK; ++xk) o[xk] *= alpha;
  if constexpr (kPacked) {
    // weights rounded to bf16 pairs (tokens 2k, 2k+1); the denominator sums
    // the same rounded values.  int8: the values the products take are p
    // times the token's V row scale (0 where masked: the scale may be NaN),
    // the denominator sums p alone.
    const uint32_t packed = pack_bf16x2(p, dpp_mov<kDppQuadXor1>(p));
    st.l = fmaf(st.l, alpha, __uint_as_float(packed << 16));
    uint32_t packed_v = packed;
    if constexpr (kInt8) {
      const float pv = masked ? 0.f : p * f.vs;
      packed_v = pack_bf16x2(pv, dpp_mov<kDppQuadXor1>(pv));
    }
    uint32_t pp[kBlockTokens / 2];
#pragma unroll
    for (int k = 0; k < kBlockTokens / 2; ++k)
      pp[k] = __builtin_amdgcn_readlane(packed_v, 2 * k);
    auto accumulate = [&](uint4 v, int th, float& acc) {  // tokens 8th .. 8th+7
      if (kTail) v = mask_tokens(v, th * 8, nfirst, nvalid);
      acc = dot2_bf16(v.x, pp[th * 4 + 0], acc);
      acc = dot2_bf16(v.y, pp[th * 4 + 1], acc);
      acc = dot2_bf16(v.z, pp[th * 4 + 2], acc);
      acc = dot2_bf16(v.w, pp[th * 4 + 3], acc);
    };
#pragma unroll
    for (int xk = 0; xk < Sh::XK; ++xk) {
      if constexpr (kBytes) {
        uint4 vlo, vhi;
        codes16_to_bf16<Tr::kKind>(f.v[xk], vlo, vhi);
        accumulate(vlo, 0, o[xk]);
        accumulate(vhi, 1, o[xk]);
      } else {
#pragma unroll
        for (int th = 0; th < Sh::R; ++th) accumulate(f.v[xk * Sh::R + th], th, o[xk]);
      }
    }
  } else {
    st.l = fmaf(st.l, alpha, p);
    float ps[kBlockTokens];
#pragma unroll
    for (int tt = 0; tt < kBlockTokens; ++tt)
      ps[tt] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), tt));
#pragma unroll
    for (int xk = 0; xk < Sh::XK; ++xk) {
#pragma unroll
      for (int th = 0; th < Sh::R; ++th) {
        const uint4 v = f.v[xk * Sh::R + th];
        const float vf[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                             __uint_as_float(v.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tt = th * 4 + e;
          if (!kTail || (tt < nvalid && tt >= nfirst)) o[xk] = fmaf(ps[tt], vf[e], o[xk]);
        }
      }
    }
  }
}

// q . k of the newest position's key row (in LDS, as the cache holds it: for
// one-byte caches the codes' bf16 values, in dim order) over this lane's
// query chunks, the four 16-lane rows combined: the same value in every lane.
template <typename Tr, int D>
__device__ __forceinline__ float fresh_score(const typename Tr::act* krow,
                                             const QueryFrag<Tr, D>& qf, int lane) {
  using Sh = ValuShape<Tr, D>;
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < Sh::KL; ++i) {
#pragma unroll
    for (int pc = 0; pc < QueryFrag<Tr, D>::kPieces; ++pc) {
      const uint4 k =
          *reinterpret_cast<const uint4*>(krow + (4 * i + lane / 16) * Sh::X + pc * 8);
      if constexpr (Tr::kKind == Kind::kF32) {
        dot = fmaf(__uint_as_float(k.x), __uint_as_float(qf.c[i][pc].x), dot);
        dot = fmaf(__uint_as_float(k.y), __uint_as_float(qf.c[i][pc].y), dot);
        dot = fmaf(__uint_as_float(k.z), __uint_as_float(qf.c[i][pc].z), dot);
        dot = fmaf(__uint_as_float(k.w), __uint_as_float(qf.c[i][pc].w), dot);
      } else {
        dot = dot2_bf16(k.x, qf.c[i][pc].x, dot);
        dot = dot2_bf16(k.y, qf.c[i][pc].y, dot);
        dot = dot2_bf16(k.z, qf.c[i][pc].z, dot);
        dot = dot2_bf16(k.w, qf.c[i][pc].w, dot);
      }
    }
  }
  return cross_row_sum(dot);
}

// One work item: partition `part` of sequence b, query head h.
template <typename Tr, int D>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, const int part, const int h,
                                          const int b) {
  using S = typename Tr::storage;
  using A = typename Tr::act;
  using Sh = ValuShape<Tr, D>;
  constexpr int X = Sh::X;

  __shared__ float sm_o[kWaves][D];
  __shared__ float sm_m[kWaves];
  __shared__ float sm_l[kWaves];
  __shared__ int sm_bad[kWaves];
  // fused step: the newest position's K and V rows, its score, and whether its
  // block's table entry lies outside the pool
  __shared__ __attribute__((aligned(16))) A sm_fresh[2][D];
  __shared__ float sm_fresh_scale[2];  // int8: the rows' scales (K, V)
  __shared__ float sm_fresh_s;
  __shared__ int sm_fresh_bad;

  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int kvh = h / (a.H / a.num_kv_heads);
  const int ctx = a.context_lens[b];
  const bool split = a.partition_size > 0;
  const int first = ctx > 0 ? window_first(ctx - 1, a.window) : 0;  // first visible token
  const int rs = range_start(ctx, a.window);
  const int nparts = split ? (ctx > 0 ? (ctx - rs + a.partition_size - 1) / a.partition_size : 0) : 1;
  const bool bad_len = ctx > a.max_nb * kBlockTokens || (split && nparts > a.num_partitions);
  const size_t row = (size_t(b) * a.H + h) * D;
  A* out = static_cast<A*>(a.out) + row;
  const size_t prow = (size_t(b) * a.H + h) * a.num_partitions + part;

  if (!split && (ctx <= 0 || bad_len)) {
    const float fill = ctx <= 0 ? 0.f : __int_as_float(0x7fc00000);
    for (int x = threadIdx.x; x < D; x += blockDim.x) out[x] = Tr::from_f32(fill);
    return;
  }
  if (split && bad_len) {
    if (part >= nparts) return;
    const float nan = __int_as_float(0x7fc00000);
    if (nparts == 1) {
      for (int x = threadIdx.x; x < D; x += blockDim.x) out[x] = Tr::from_f32(nan);
    } else {
      for (int x = threadIdx.x; x < D; x += blockDim.x) a.ws_o[prow * D + x] = nan;
      if (threadIdx.x == 0) { a.ws_m[prow] = 0.f; a.ws_l[prow] = 1.f; }
    }
    return;
  }
  if (split && part >= nparts) return;

  const int tb = rs + (split ? part * a.partition_size : 0);
  int te = split ? min(tb + a.partition_size, ctx) : ctx;
  // Fused step: the item holding position ctx - 1 takes that position from
  // the fresh rows (folded in at the merge) and walks the cache up to ctx - 2
  // only; with no cached position left in its range it walks nothing.
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

  // This lane's slice of the query: the dims of chunks 4i + lane/16.
  QueryFrag<Tr, D> qf;
  {
    const A* qrow = static_cast<const A*>(a.query) + row;
#pragma unroll
    for (int i = 0; i < Sh::KL; ++i)
#pragma unroll
      for (int pc = 0; pc < QueryFrag<Tr, D>::kPieces; ++pc)
        qf.c[i][pc] = *reinterpret_cast<const uint4*>(qrow + (4 * i + lane / 16) * X + pc * 8);
  }
  if (fold && w == 0) fetch_fresh<Tr, D>(a, b, kvh, lane, sm_fresh, sm_fresh_bad, sm_fresh_scale);

  const S* kc = static_cast<const S*>(a.k_cache);
  const S* vc = static_cast<const S*>(a.v_cache);
  const int64_t tile_elems = int64_t(kBlockTokens) * D;

  WaveState st{-INFINITY, 0.f};
  float o[Sh::XK];
#pragma unroll
  for (int xk = 0; xk < Sh::XK; ++xk) o[xk] = 0.f;
  int bad_blk = 0;

  // Block n of this wave's walk, from the current window of table entries
  // (lane i of `win` holds entry n0 + i).  No branch around the loads: an entry
  // outside the pool loads tile 0 instead (always valid memory) and is
  // reported as -1, so every load in the loop below is unconditional and the
  // compiler can keep the next block's loads in flight while one computes.
  int n0 = 0;
  auto fetch = [&](int n, BlockFrag<Tr, D>& f) -> int64_t {
    const int p = __builtin_amdgcn_readlane(win, n - n0);
    const bool ok = p >= 0 && p < a.num_blocks;
    const int64_t tile = (int64_t(ok ? p : 0) * a.num_kv_heads + kvh) * tile_elems;
    if constexpr (Tr::kKind == Kind::kInt8) {
      const int64_t row0 = tile / D;  // the tile's first (block, head, slot) row
      load_block<Tr, D>(f, kc + tile, vc + tile, lane, row_scales(a.k_cache, a.scales_offset) + row0,
                        row_scales(a.v_cache, a.scales_offset) + row0);
    } else {
      load_block<Tr, D>(f, kc + tile, vc + tile, lane);
    }
    return ok ? tile : -1;
  };
  auto consume = [&](int j, int64_t tile, const BlockFrag<Tr, D>& f) {
    if (tile < 0) { bad_blk = 1; return; }
    const int nvalid = te - j * kBlockTokens;
    const int nfirst = first - j * kBlockTokens;  // > 0 only where a window starts
    if (nvalid >= kBlockTokens && nfirst <= 0)
      compute_block<Tr, D, false>(f, qf, o, st, 0, nvalid, a.scale_log2, lane);
    else
      compute_block<Tr, D, true>(f, qf, o, st, nfirst, nvalid, a.scale_log2, lane);
  };
  // Ping-pong over two register buffers: block n+1 is in flight while n
  // computes.  Windows of 64 blocks; inside one, every iteration has a next
  // block to fetch (the last one or two are peeled off).
  const int nblk = je - jb - w > 0 ? (je - jb - w + kWaves - 1) / kWaves : 0;
  BlockFrag<Tr, D> fa, fb;
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
    float sf = fresh_score<Tr, D>(sm_fresh[0], qf, lane) * a.scale_log2;
    if constexpr (Tr::kKind == Kind::kInt8) sf *= sm_fresh_scale[0];  // as the blocks' ks
    if (lane == 0) sm_fresh_s = sf;
  }
  // Wave totals: the denominator is spread over the 16 token lanes of a row.
  const float lsum = row16_sum(st.l);
  if (lane == 0) {
    sm_m[w] = st.m;
    sm_l[w] = lsum;
    sm_bad[w] = bad_blk;
  }
#pragma unroll
  for (int xk = 0; xk < Sh::XK; ++xk) sm_o[w][xk * kWave + lane] = o[xk];
  __syncthreads();

  for (int x = threadIdx.x; x < D; x += blockDim.x) {
    float M = -INFINITY;
    int bad = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      M = fmaxf(M, sm_m[ww]);
      bad |= sm_bad[ww];
    }
    if (fold) {  // the newest position joins as one more partial: m = its score, l = 1
      M = fmaxf(M, sm_fresh_s);
      bad |= sm_fresh_bad;
    }
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      if (sm_m[ww] == -INFINITY) continue;  // a wave that saw no block
      const float sc = fast_exp2(sm_m[ww] - M);
      L = fmaf(sm_l[ww], sc, L);
      acc = fmaf(sm_o[ww][x], sc, acc);
    }
    if (fold) {
      const float sc = fast_exp2(sm_fresh_s - M);
      L += sc;
      float v = act_to_f32<Tr>(sm_fresh[1][x]);
      if constexpr (Tr::kKind == Kind::kInt8) v *= sm_fresh_scale[1];  // as the blocks' vs
      acc = fmaf(v, sc, acc);
    }
    float res = acc / L * a.v_scale;
    if (bad) res = __int_as_float(0x7fc00000);
    if (!split || nparts == 1) {
      out[x] = Tr::from_f32(res);
    } else {
      a.ws_o[prow * D + x] = res;
      if (x == 0) {
        a.ws_m[prow] = bad ? 0.f : M;
        a.ws_l[prow] = bad ? 1.f : L;
      }
    }
  }
}

// Single pass (kSplit = false): grid (1, head tiles, B), one work-group per
// sequence and head tile, sequences taken longest first.  Split (kSplit = true): grid (resident workers, head
// tiles, 1) walking the work list.  Two instantiations keep each one's
// register allocation that of a single inlined item.
//
// Fused step: append_groups more work-groups write the new rows, dispatched
// after every decode work-group (single pass: z-slabs past the sequences;
// split: y-slabs past the heads), so their stores meet the end of the read
// stream.  The decode never waits for them: it takes the newest position from
// the fresh rows.  (The scattered partial-line stores of a write slow a read
// stream they overlap: placed first, or spread over the decode work-groups,
// they cost the 7B-shape step 20-24 us; placed last, 8 us.)
template <typename Tr, int D, bool kSplit>
__global__ __launch_bounds__(kWaves * kWave) void decode_valu_kernel(DecodeArgs a) {
  if constexpr (!kSplit) {
    const int z = blockIdx.z;
    if (a.append_groups > 0 && z >= a.B) {
      append_group<Tr>(a.append, int64_t(z - a.B) * gridDim.y + blockIdx.y);
      return;
    }
    __shared__ int sm_order[kOrderBuckets + kWaves + 1];
    const int b = a.B <= kMaxOrderedSeqs
        ? sequence_of_rank<kWaves * kWave>(a.context_lens, a.B, a.max_nb, z, sm_order)
        : z;
    valu_item<Tr, D>(a, 0, blockIdx.y, b);
  } else {
    if (int(blockIdx.y) >= a.H) {
      append_group<Tr>(a.append, int64_t(blockIdx.y - a.H) * gridDim.x + blockIdx.x);
      return;
    }
    __shared__ int sm_starts[kMaxSplitSeqs + 1];
    const int n_items = build_work_list(a, sm_starts);
    for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
      int b, part;
      locate_item(sm_starts, a.B, i, b, part);
      valu_item<Tr, D>(a, part, blockIdx.y, b);
      __syncthreads();  // the next item reuses the merge buffers
    }
  }
}

}  // namespace

template <typename Tr>
void (*valu_kernel(int head_dim, bool split))(DecodeArgs) {
  if (head_dim == 128)
    return split ? decode_valu_kernel<Tr, 128, true> : decode_valu_kernel<Tr, 128, false>;
  if (head_dim == 64)
    return split ? decode_valu_kernel<Tr, 64, true> : decode_valu_kernel<Tr, 64, false>;
  return nullptr;
}

hipError_t launch_decode_valu(const DecodeArgs& a, Kind kind, int head_dim, hipStream_t s) {
  const bool split = a.partition_size > 0;
  void (*kern)(DecodeArgs) = kind == Kind::kBf16   ? valu_kernel<Bf16>(head_dim, split)
                             : kind == Kind::kF32  ? valu_kernel<F32>(head_dim, split)
                             : kind == Kind::kInt8 ? valu_kernel<Int8>(head_dim, split)
                                                   : valu_kernel<Fp8>(head_dim, split);
  if (!kern) return hipErrorInvalidValue;
  const dim3 block(kWaves * kWave);
  dim3 grid(1, a.H, a.B);
  if (a.partition_size > 0) {
    const int64_t most = int64_t(a.B) * a.num_partitions;
    const int workers = resident_workers(reinterpret_cast<const void*>(kern), block.x, a.H);
    grid = dim3(unsigned(most < workers ? most : workers), a.H, 1);
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
