// Work list of split-KV decode: the (sequence, partition) items that exist.
//
// A sequence of ctx tokens has ceil(ctx / P) partitions of P tokens.  Sizing a
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
// counts (min(ceil(ctx/P), P_max); 0 for ctx <= 0) and returns the total.
// Must be called by every thread of the work-group.
__device__ __forceinline__ int build_work_list(const DecodeArgs& a, int* starts) {
  const int B = a.B;
  const int P = a.partition_size;
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const int ctx = a.context_lens[t];
    const int np = ctx > 0 ? (ctx + P - 1) / P : 0;
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

}  // namespace pagedkv
