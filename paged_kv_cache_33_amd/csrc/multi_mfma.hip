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
    load_block<E, D>(f, kc + tile, vc + tile, lane);
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
  void (*kern)(MultiArgs) = kind == Kind::kBf16  ? multi_kernel<Bf16>(head_dim, a.tiles_per_set)
                            : kind == Kind::kFp8 ? multi_kernel<Fp8>(head_dim, a.tiles_per_set)
                                                 : nullptr;
  if (!kern) return hipErrorInvalidValue;
  if (a.B == 0 || a.max_query_len == 0) return hipSuccess;
  const int g = a.H / a.num_kv_heads;
  const int64_t set_cols = int64_t(kHeadsPerTile) * a.tiles_per_set;
  const int64_t sets = (int64_t(a.max_query_len) * g + set_cols - 1) / set_cols;
  const int64_t groups = (sets + a.sets_per_group - 1) / a.sets_per_group;
  hipLaunchKernelGGL(kern, dim3(unsigned(groups), unsigned(a.num_kv_heads), unsigned(a.B)),
                     dim3(kMultiWaves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
