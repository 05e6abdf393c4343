// Work list of split-KV decode: the (sequence, partition) items that exist.
//
// A sequence of ctx tokens has ceil((ctx - r) / P) partitions of P tokens, r
// the start of its range (0 without a sliding window).  Sizing a
// grid by the longest sequence would launch mostly empty work-groups when
// lengths differ (100,000 and 17 tokens in one batch); instead every
// work-group builds the prefix sum of the per-sequence partition counts in LDS
// and walks the real items i = blockIdx.x, blockIdx.x + gridDim.x, ...  The
// grid holds as many work-groups as the GPU keeps resident, so each one starts
// at once and the items, all of nearly equal size, are dealt round-robin.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace pagedkv {

// Fills starts[0..B] with the exclusive prefix sum of the per-sequence item
// counts (min(ceil((ctx - r)/P), P_max); 0 for ctx <= 0) and returns the total.
// Must be called by every thread of the work-group.
__device__ __forceinline__ int build_work_list(const DecodeArgs& a, int* starts) {
  const int B = a.B;
  const int P = a.partition_size;
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const int ctx = a.context_lens[t];
    const int np = ctx > 0 ? (ctx - range_start(ctx, a.window) + P - 1) / P : 0;
    starts[t + 1] = min(np, a.num_partitions);
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int per = (B + kWave - 1) / kWave;
    const int lo = min(lane * per, B), hi = min(lo + per, B);
    int sum = 0;
    for (int k = lo; k < hi; ++k) sum += starts[k + 1];
    int incl = sum;  // inclusive scan of the 64 chunk sums
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += v;
    }
    int run = incl - sum;
    for (int k = lo; k < hi; ++k) {
      run += starts[k + 1];
      starts[k + 1] = run;
    }
    if (lane == 0) starts[0] = 0;
  }
  __syncthreads();
  return starts[B];
}

// Sequence b and partition of item i: starts[b] <= i < starts[b + 1].
__device__ __forceinline__ void locate_item(const int* starts, int B, int i, int& b, int& part) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (starts[mid] <= i) lo = mid; else hi = mid;
  }
  b = lo;
  part = i - starts[lo];
}


// Single-pass decode takes sequences longest first.  Work-groups are dispatched
// in index order, so when work-group z takes the z-th longest sequence the
// dispatcher itself deals the work longest-processing-time first: the long
// sequences start at once and the short ones fill the gaps at the end, where a
// long sequence drawn late would otherwise run alone on a draining GPU.  Every
// work-group derives the same order from context_lens: sequences are bucketed
// by block count (kOrderBuckets equal-width buckets over [0, max_nb]), longer
// buckets first, index order inside a bucket.  Any order is correct (each
// sequence is still taken by exactly one work-group); this one balances load.
constexpr int kOrderBuckets = 32;
constexpr int kMaxOrderedSeqs = 4096;

// Sequence of rank r (0 <= r < B <= kMaxOrderedSeqs) in that order.  sh: LDS of
// kOrderBuckets + kThreads / 64 + 1 ints.  Called by every thread of the
// work-group (it synchronises).
template <int kThreads>
__device__ __forceinline__ int sequence_of_rank(const int32_t* __restrict__ context_lens, int B,
                                                int max_nb, int r, int* sh) {
  constexpr int kW = kThreads / kWave;
  // each thread keys kMaxIters sequences: the work-group must cover all of them
  static_assert(kMaxOrderedSeqs % kThreads == 0, "kMaxIters * kThreads == kMaxOrderedSeqs");
  constexpr int kMaxIters = kMaxOrderedSeqs / kThreads;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int* total = sh;                      // [kOrderBuckets] members per bucket
  int* wave_cnt = sh + kOrderBuckets;   // [kW] members of the wanted bucket per wave
  int* result = wave_cnt + kW;
  for (int k = tid; k < kOrderBuckets; k += kThreads) total[k] = 0;
  if (tid == 0) *result = r;  // always a valid index
  // Wave w owns sequences [w * per_wave, (w + 1) * per_wave), 64 per iteration.
  const int iters = (B + kThreads - 1) / kThreads;
  const int per_wave = iters * kWave;
  int key[kMaxIters];
#pragma unroll
  for (int it = 0; it < kMaxIters; ++it) {
    key[it] = -1;
    const int j = w * per_wave + it * kWave + lane;
    if (it < iters && j < B) {
      const int n = context_lens[j];
      const int64_t nb = n > 0 ? min((int64_t(n) + kBlockTokens - 1) / kBlockTokens, int64_t(max_nb)) : 0;
      // (32-bit arithmetic where it cannot overflow: far cheaper than 64-bit
      // division)
      key[it] = max_nb < (1 << 26)
                    ? int(unsigned(nb) * unsigned(kOrderBuckets) / unsigned(max_nb + 1))
                    : int(nb * kOrderBuckets / (int64_t(max_nb) + 1));
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kMaxIters; ++it)
    if (key[it] >= 0) atomicAdd(&total[key[it]], 1);
  __syncthreads();
  // Bucket holding rank r, from the longest bucket down, and r's index in it:
  // lane i takes bucket kOrderBuckets - 1 - i, a prefix sum over the lanes
  // gives each bucket's last rank, and the first lane past r holds it (one
  // LDS read and five shuffles, where a bucket-by-bucket walk waited for up
  // to 32 dependent LDS reads).
  static_assert(kOrderBuckets <= kWave, "one lane per bucket");
  const int t = lane < kOrderBuckets ? total[kOrderBuckets - 1 - lane] : 0;
  int incl = t;
#pragma unroll
  for (int off = 1; off < kOrderBuckets; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  const uint64_t past = __ballot(lane < kOrderBuckets && r < incl);
  int want_key = 0, before = 0;
  if (past != 0) {
    const int i = __ffsll(static_cast<unsigned long long>(past)) - 1;
    want_key = kOrderBuckets - 1 - i;
    before = __shfl(incl - t, i, kWave);
  }
  const int want = r - before;
  int cnt = 0;
#pragma unroll
  for (int it = 0; it < kMaxIters; ++it)
    cnt += __popcll(__ballot(key[it] == want_key));
  if (lane == 0) wave_cnt[w] = cnt;
  __syncthreads();
  int base = 0;
  for (int ww = 0; ww < w; ++ww) base += wave_cnt[ww];
  if (want >= base && want < base + cnt) {
    int seen = base;
#pragma unroll
    for (int it = 0; it < kMaxIters; ++it) {
      const uint64_t m = __ballot(key[it] == want_key);
      const int c = __popcll(m);
      if (want < seen + c) {
        const bool mine = (m >> lane) & 1;
        if (mine && __popcll(m & ((uint64_t(1) << lane) - 1)) == want - seen)
          *result = w * per_wave + it * kWave + lane;
        break;
      }
      seen += c;
    }
  }
  __syncthreads();
  return *result;
}

}  // namespace pagedkv
