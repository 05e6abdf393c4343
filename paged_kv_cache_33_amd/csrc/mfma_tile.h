// MFMA tile code shared by the decode kernel (decode_mfma.hip) and the
// multi-token kernel (multi_mfma.hip): per 16-token block, S = K Q^T and
// O^T += V^T P^T as gfx950 matrix-core tiles with the online softmax between.
//
// Operand layouts (wave64, lane l, q = l / 16, n = l % 16):
//   16x16x32 bf16: A row n, k = 8q..8q+7; B column n, k = 8q..8q+7;
//   16x16x16 bf16: A row n, k = 4q..4q+3; B column n, k = 4q..4q+3;
//   accumulator: register j holds row 4q + j, column n.
// K's [d/8][16][8] tile puts the 8 dims of chunk 4i + q of token n in one
// 16-byte load (a coalesced 1 KiB per wave); the contraction runs over dims in
// that chunk order, and Q's operand is loaded in the same order.  V's [d][16]
// tile puts tokens 4q..4q+3 of dim 16mc + n in one 8-byte load (a coalesced
// 512 B per wave).  The S accumulator (tokens 4q+j of head n) is already the
// P^T operand of the second product, so no data moves between lanes.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace pagedkv {
namespace {

constexpr int kHeadsPerTile = 16;
constexpr float kRescaleSlack = 8.f;  // see compute_block

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short short4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef float floatx4_t __attribute__((__vector_size__(4 * sizeof(float))));

template <int D>
struct MfmaShape {
  static constexpr int KI = D / 32;  // QK products per block (= 16-byte K loads per lane)
  static constexpr int MC = D / 16;  // PV products per block (= 8-byte V loads per lane)
};

// One block's K and V as loaded by one lane.  bf16: 16-byte K chunk 4i + q of
// token n is operand i of S = K Q^T as stored; 8 bytes of V (tokens 4q..4q+3
// of dim 16mc + n) are operand mc of O^T = V^T P^T.  One-byte codes (fp8 E4M3
// or int8): one 16-byte load holds chunk q + 4j (16 dims) and becomes operands
// 2j, 2j+1 (dims 8 and 8 more); 4 bytes of V become operand mc.  The codes
// convert to bf16 exactly, so every cache feeds the same bf16 products.  An
// int8 cache adds the K and V row scales of the tokens 4q..4q+3 whose S rows
// the lane holds: each lane loads one scale of each (token 4q + n % 4, 4 bytes)
// and a quad of lanes shares its four by DPP broadcasts (quad_bcast).  Loading
// all four per lane (16 bytes, identical in 16 lanes) made every wave-wide
// scale load return 1 KiB for 64 unique bytes and measured 5% slower on the
// GQA batch-256 workload.
template <typename E, bool kScaled = E::kKind == Kind::kInt8>
struct MfmaScales {
  float ks, vs;  // of token 4q + (n & 3)
};
template <typename E>
struct MfmaScales<E, false> {};

// The value of lane J of this lane's quad (DPP quad_perm [J, J, J, J]).
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), J * 0x55, 0xF, 0xF, false));
}

// The four row scales of a quad's tokens 4q .. 4q + 3 (lane n % 4 of the quad
// holds token 4q + n % 4's, see MfmaScales), for every lane, where a lane uses
// them under a mask.  A broadcast reads another lane, so it must run with the
// whole wave active: left to itself the compiler may compute it under the
// mask, where only the lanes that use it are on, and a broadcast from a lane
// that is off returns 0 (seen in an int8 kernel: the weights of some causally
// masked columns came out 0).  The empty asm statement makes the values exist
// here, before any masking.
__device__ __forceinline__ void quad_scales(float v, float (&out)[4]) {
  out[0] = quad_bcast<0>(v);
  out[1] = quad_bcast<1>(v);
  out[2] = quad_bcast<2>(v);
  out[3] = quad_bcast<3>(v);
  __asm__ volatile("" : "+v"(out[0]), "+v"(out[1]), "+v"(out[2]), "+v"(out[3]));
}

template <typename E, int D>
struct MfmaFrag : MfmaScales<E> {
  static constexpr bool kFp8 = kByteCodes<E>;  // one-byte codes
  static constexpr int KL = kFp8 ? D / 64 : D / 32;  // 16-byte K loads per lane
  using VPiece = std::conditional_t<kFp8, uint32_t, uint2>;
  uint4 k[KL];
  VPiece v[MfmaShape<D>::MC];
};

// ksr / vsr: the tile's 16 row scales (int8 caches only).
template <typename E, int D>
__device__ __forceinline__ void load_block(MfmaFrag<E, D>& f, const typename E::storage* kt,
                                           const typename E::storage* vt, int lane,
                                           const float* ksr = nullptr,
                                           const float* vsr = nullptr) {
  constexpr int X = E::kChunk;
  if constexpr (E::kKind == Kind::kInt8) {
    const int tok = 4 * (lane >> 4) + (lane & 3);
    f.ks = __builtin_nontemporal_load(ksr + tok);
    f.vs = __builtin_nontemporal_load(vsr + tok);
  }
#pragma unroll
  for (int i = 0; i < MfmaFrag<E, D>::KL; ++i)
    f.k[i] = load_tile16(kt + (i * kWave + lane) * X);
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mc = 0; mc < MfmaShape<D>::MC; ++mc) {
    if constexpr (MfmaFrag<E, D>::kFp8)
      f.v[mc] = load_tile4(vt + (16 * mc + n) * kBlockTokens + 4 * q);
    else
      f.v[mc] = load_tile8(vt + (16 * mc + n) * kBlockTokens + 4 * q);
  }
}

// load_block from a copy of the two tiles in LDS (same layouts).
template <typename E, int D>
__device__ __forceinline__ void load_block_lds(MfmaFrag<E, D>& f, const typename E::storage* kt,
                                               const typename E::storage* vt, int lane) {
  constexpr int X = E::kChunk;
#pragma unroll
  for (int i = 0; i < MfmaFrag<E, D>::KL; ++i)
    f.k[i] = *reinterpret_cast<const uint4*>(kt + (i * kWave + lane) * X);
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int mc = 0; mc < MfmaShape<D>::MC; ++mc)
    f.v[mc] = *reinterpret_cast<const typename MfmaFrag<E, D>::VPiece*>(
        vt + (16 * mc + n) * kBlockTokens + 4 * q);
}

// Operand i of S = K Q^T and operand mc of O^T = V^T P^T, as bf16.
template <typename E, int D>
__device__ __forceinline__ bf16x8_t k_operand(const MfmaFrag<E, D>& f, int i) {
  if constexpr (MfmaFrag<E, D>::kFp8) {
    constexpr Kind kK = E::kKind;
    const uint4 c = f.k[i >> 1];
    const uint32_t w0 = (i & 1) ? c.z : c.x, w1 = (i & 1) ? c.w : c.y;
    return __builtin_bit_cast(bf16x8_t, make_uint4(code2_to_bf16x2<kK, false>(w0),
                                                   code2_to_bf16x2<kK, true>(w0),
                                                   code2_to_bf16x2<kK, false>(w1),
                                                   code2_to_bf16x2<kK, true>(w1)));
  } else {
    return __builtin_bit_cast(bf16x8_t, f.k[i]);
  }
}
template <typename E, int D>
__device__ __forceinline__ uint2 v_operand(const MfmaFrag<E, D>& f, int mc) {
  if constexpr (MfmaFrag<E, D>::kFp8)
    return make_uint2(code2_to_bf16x2<E::kKind, false>(f.v[mc]),
                      code2_to_bf16x2<E::kKind, true>(f.v[mc]));
  else
    return f.v[mc];
}

// First query dim of the 8 that pair with K operand i in lane quarter q.
template <typename E>
__device__ __forceinline__ int query_dim0(int i, int q) {
  if constexpr (kByteCodes<E>)
    return (q + 4 * (i >> 1)) * 16 + (i & 1) * 8;
  else
    return (4 * i + q) * 8;
}

template <int D>
struct MfmaState {
  floatx4_t o[MfmaShape<D>::MC];  // O^T[16mc + 4q + j][head n]
  float m;                        // reference max of head n (base 2): within 8 of the max
  float l;                        // denominator share of head n over tokens 4q..4q+3
};

__device__ __forceinline__ uint32_t zero_masked_pair(uint32_t w, bool keep_lo, bool keep_hi) {
  return (keep_lo ? (w & 0x0000ffffu) : 0u) | (keep_hi ? (w & 0xffff0000u) : 0u);
}

// One 16-token block for kT column tiles that share its K/V operands: S =
// K Q^T, the online softmax per column, O^T += V^T P^T.  The work runs phase
// by phase over the tiles (every tile's score products, then every tile's
// softmax, then the PV products), so the tiles' dependent chains interleave.
// With kTail only tokens nfirst .. nvalid-1 of the block (uniform bounds) are
// inside the range; the rest get no weight and their V is zeroed (their slots
// may hold NaN).  kCausal: the block's first token is at key position key0 and
// tile tt's lane column may see positions lo[tt] .. limit[tt] only.
template <typename E, int D, bool kTail, bool kCausal, int kT>
__device__ __forceinline__ void compute_block_tiles(const MfmaFrag<E, D>& f,
                                                    const bf16x8_t (*qop)[MfmaShape<D>::KI],
                                                    MfmaState<D>* st, int nfirst, int nvalid,
                                                    float scale_log2, int lane, int key0,
                                                    const int* lo, const int* limit) {
  const int q = lane >> 4;
  floatx4_t s[kT];
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) s[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MfmaShape<D>::KI; ++i) {
    const bf16x8_t kop = k_operand<E, D>(f, i);
#pragma unroll
    for (int tt = 0; tt < kT; ++tt)
      s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[tt][i], s[tt], 0, 0, 0);
  }
  constexpr bool kInt8 = E::kKind == Kind::kInt8;
  // sc[j]: the score of token 4q + j in base 2, -inf where masked (by select:
  // the slot may hold NaN).  Without per-token scales the multiply by
  // scale_log2 is folded into the exponent's argument below, and the block
  // maximum scaled once (scale_log2 > 0, so max and rounding commute).
  float sc[kT][4];
  bool masked[kT][4];
  float lmax[kT];
  bool exceeds = false;
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[tt][j] = s[tt][j];
      if constexpr (kInt8) {  // token 4q + j's K row scale (used by every lane)
        const float ks[4] = {quad_bcast<0>(f.ks), quad_bcast<1>(f.ks), quad_bcast<2>(f.ks),
                             quad_bcast<3>(f.ks)};
        sc[tt][j] = sc[tt][j] * scale_log2 * ks[j];
      }
      masked[tt][j] = (kTail && (4 * q + j >= nvalid || 4 * q + j < nfirst)) ||
                      (kCausal && (key0 + 4 * q + j > limit[tt] || key0 + 4 * q + j < lo[tt]));
      if (masked[tt][j]) sc[tt][j] = -INFINITY;
    }
    // (maximum, not fmaxf: gfx950's v_maximum3_f32 needs no NaN quieting of
    // the matrix-core results; a NaN score makes its column NaN either way)
    lmax[tt] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(sc[tt][0], sc[tt][1]),
                                             __builtin_elementwise_maximum(sc[tt][2], sc[tt][3]));
    if constexpr (!kInt8) lmax[tt] *= scale_log2;
    exceeds = exceeds || lmax[tt] > st[tt].m + kRescaleSlack;
  }
  // The reference max st.m moves only when a head's block max exceeds it by
  // more than kRescaleSlack (base-2 units), so weights 2^(s - m) stay below 2^8
  // and most blocks skip rescaling O (32 multiplies at d = 128).  Softmax does
  // not depend on the reference, so only rounding changes.  The column's max
  // over its four lanes is needed only when one of them exceeds the reference
  // by that much, so the wave first asks whether any lane's own max does.
  if (__builtin_amdgcn_ballot_w64(exceeds) != 0) {  // wave-uniform
#pragma unroll
    for (int tt = 0; tt < kT; ++tt) {
      const float mx = cross_row_max(lmax[tt]);
      const bool grow = mx > st[tt].m + kRescaleSlack;
      // Only growing columns rescale.  The others keep factor 1 (exact): a
      // column that has seen no key yet (m = -inf, possible under causal and
      // window masks) would otherwise get 2^(-inf - -inf) = NaN.
      const float alpha = grow ? fast_exp2(st[tt].m - mx) : 1.f;
      st[tt].l *= alpha;
#pragma unroll
      for (int mc = 0; mc < MfmaShape<D>::MC; ++mc) st[tt].o[mc] *= alpha;
      st[tt].m = grow ? mx : st[tt].m;
    }
  }
  // weights rounded to bf16 for the matrix core; the denominator sums the
  // same rounded values.  Causal: a column that has seen no position yet
  // (every score -inf) takes weight 0, not 2^(-inf - -inf).
  float vs[4];  // int8: the V row scales of tokens 4q + j
  if constexpr (kInt8) quad_scales(f.vs, vs);
  short4_t pop[kT];
#pragma unroll
  for (int tt = 0; tt < kT; ++tt) {
    const float mref = (kCausal && st[tt].m == -INFINITY) ? 0.f : st[tt].m;
    float pw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pw[j] = kInt8 ? fast_exp2(sc[tt][j] - mref)
                    : fast_exp2(__builtin_fmaf(sc[tt][j], scale_log2, -mref));
    const uint32_t p01 = pack_bf16x2(pw[0], pw[1]);
    const uint32_t p23 = pack_bf16x2(pw[2], pw[3]);
    // the rounded weights summed by two packed dot products with ones (the
    // bf16 products are exact in fp32)
    constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
    st[tt].l = dot2_bf16(p23, kOnes, dot2_bf16(p01, kOnes, st[tt].l));
    uint32_t q01 = p01, q23 = p23;
    if constexpr (kInt8) {
      // the products take p times the token's V row scale (0 where masked:
      // the scale may be NaN there); the denominator above sums p alone
      float pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[j] = masked[tt][j] ? 0.f : pw[j] * vs[j];
      q01 = pack_bf16x2(pv[0], pv[1]);
      q23 = pack_bf16x2(pv[2], pv[3]);
    }
    pop[tt] = __builtin_bit_cast(short4_t, make_uint2(q01, q23));
  }
#pragma unroll
  for (int mc = 0; mc < MfmaShape<D>::MC; ++mc) {
    uint2 v = v_operand<E, D>(f, mc);
    if (kTail) {  // tokens outside the range get weight 0; their V must be 0, not NaN
      const int t = 4 * q;
      v.x = zero_masked_pair(v.x, t >= nfirst && t < nvalid, t + 1 >= nfirst && t + 1 < nvalid);
      v.y = zero_masked_pair(v.y, t + 2 >= nfirst && t + 2 < nvalid,
                             t + 3 >= nfirst && t + 3 < nvalid);
    }
#pragma unroll
    for (int tt = 0; tt < kT; ++tt)
      st[tt].o[mc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(short4_t, v), pop[tt], st[tt].o[mc], 0, 0, 0);
  }
}

// compute_block_tiles for one column tile.
template <typename E, int D, bool kTail, bool kCausal = false>
__device__ __forceinline__ void compute_block(const MfmaFrag<E, D>& f,
                                              const bf16x8_t (&qop)[MfmaShape<D>::KI],
                                              MfmaState<D>& st, int nfirst, int nvalid,
                                              float scale_log2, int lane, int key0 = 0,
                                              int lo = 0, int limit = 0) {
  compute_block_tiles<E, D, kTail, kCausal, 1>(f, &qop, &st, nfirst, nvalid, scale_log2, lane,
                                               key0, &lo, &limit);
}

// Work-group barrier for data exchanged through LDS only: this wave's LDS
// operations complete (lgkmcnt 0; the gfx9 s_waitcnt encoding with vmcnt and
// expcnt at their maxima, i.e. not waited for), then s_barrier.  Unlike
// __syncthreads it leaves global loads in flight.  The empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  constexpr int kLgkm0 = 0xF | (3 << 14) | (7 << 4);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Walk a wave's blocks j = first, first + stride, ... < je.  Table entries are
// read 64 at a time into one register (lane i holds the entry of the wave's
// block n0 + i) so no tile load waits on a dependent table load.
// fetch(entry, frag) loads a block's tiles (unconditionally: an entry outside
// the pool loads tile 0 and is reported as -1) and returns its tile offset or
// -1; consume(j, tile, frag) computes it.  Two register buffers ping-pong, and
// inside a window every iteration has a next block to fetch (the last one or
// two are peeled off), so the loads of block n+1 stay in flight while block n
// computes.
template <typename Frag, typename Fetch, typename Consume>
__device__ __forceinline__ void walk_blocks(int first, int stride, int je, int lane,
                                            const int32_t* table, Fetch&& fetch,
                                            Consume&& consume) {
  const int nblk = je > first ? (je - first + stride - 1) / stride : 0;
  Frag fa, fb;
  for (int n0 = 0; n0 < nblk; n0 += kWave) {
    const int cnt = min(kWave, nblk - n0);
    const int win = lane < cnt ? table[first + stride * (n0 + lane)] : -1;
    const int j0 = first + stride * n0;
    int64_t tile_a = fetch(__builtin_amdgcn_readlane(win, 0), fa), tile_b;
    int n = 0;
    for (; n + 2 < cnt; n += 2) {
      tile_b = fetch(__builtin_amdgcn_readlane(win, n + 1), fb);
      consume(j0 + stride * n, tile_a, fa);
      tile_a = fetch(__builtin_amdgcn_readlane(win, n + 2), fa);
      consume(j0 + stride * (n + 1), tile_b, fb);
    }
    if (n + 1 < cnt) {
      tile_b = fetch(__builtin_amdgcn_readlane(win, n + 1), fb);
      consume(j0 + stride * n, tile_a, fa);
      consume(j0 + stride * (n + 1), tile_b, fb);
    } else {
      consume(j0 + stride * n, tile_a, fa);
    }
  }
}

}  // namespace
}  // namespace pagedkv
