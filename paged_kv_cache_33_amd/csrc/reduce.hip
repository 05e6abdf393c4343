// Log-sum-exp merge of split-KV partials.
//
// Each partition k of a sequence left (o_k, m_k, l_k): its normalised partial
// output, its max score and its denominator, in base-2 units.  Rescaling every
// partition to the common max M = max_k m_k is the online-softmax rule of
// "MLSys Engineer - Inference Systems Q&A", Q4 (multiply by exp(m_old - m_new)),
// applied to whole partitions:
//   w_k = l_k * 2^(m_k - M),   out = sum_k w_k o_k / sum_k w_k.
// One work-group per (query head, sequence); the weights are computed once into
// LDS, then the threads split the partitions and the output dims.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {
namespace {

constexpr int kReduceThreads = 256;

// Block-wide max / sum of one value per thread (256 threads = 4 waves).
__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = cross_row_max(row16_max(v));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < kReduceThreads / kWave; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  v = cross_row_sum(row16_sum(v));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) scratch[w] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < kReduceThreads / kWave; ++i) r += scratch[i];
  return r;
}

// Thread t owns the four output dims 4*(t % R) .. +3 (one 16-byte load per
// partition row, R = D / 4 threads per row) and partitions k = t / R,
// t / R + G, ... with G = 256 / R groups; four independent accumulators keep
// four partition rows in flight per thread, and the G group sums meet in LDS.
template <typename Tr, int D>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_kernel(ReduceArgs a) {
  constexpr int R = D / 4;
  constexpr int G = kReduceThreads / R;
  extern __shared__ float sm_w[];  // [num_partitions] weights
  __shared__ float sm_red[kReduceThreads / kWave];
  __shared__ __attribute__((aligned(16))) float sm_part[G][D];
  using S = typename Tr::storage;

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int ctx = a.context_lens[b];
  const int nparts =
      ctx > 0 ? (ctx - range_start(ctx, a.window) + a.partition_size - 1) / a.partition_size : 0;
  S* out = static_cast<S*>(a.out) + (size_t(b) * a.H + h) * D;

  if (nparts == 1) return;  // the decode kernel wrote this row itself
  if (nparts == 0 || nparts > a.num_partitions) {
    const float fill = nparts == 0 ? 0.f : __int_as_float(0x7fc00000);
    for (int x = threadIdx.x; x < D; x += blockDim.x) out[x] = Tr::from_f32(fill);
    return;
  }
  const size_t base = (size_t(b) * a.H + h) * a.num_partitions;
  const float* m = a.ws_m + base;
  const float* l = a.ws_l + base;
  const float4* o = reinterpret_cast<const float4*>(a.ws_o + base * D);

  float mx = -INFINITY;
  for (int k = threadIdx.x; k < nparts; k += kReduceThreads) mx = fmaxf(mx, m[k]);
  const float M = block_max(mx, sm_red);

  float tot = 0.f;
  for (int k = threadIdx.x; k < nparts; k += kReduceThreads) {
    const float wk = l[k] * fast_exp2(m[k] - M);
    sm_w[k] = wk;
    tot += wk;
  }
  const float total = block_sum(tot, sm_red);  // its barriers also publish sm_w

  const int xv = threadIdx.x % R;
  const int kg = threadIdx.x / R;
  float4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fma4 = [](float w, const float4 v, float4& c) {
    c.x = fmaf(w, v.x, c.x);
    c.y = fmaf(w, v.y, c.y);
    c.z = fmaf(w, v.z, c.z);
    c.w = fmaf(w, v.w, c.w);
  };
  int k = kg;
  for (; k + 3 * G < nparts; k += 4 * G) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = o[size_t(k + u * G) * R + xv];
#pragma unroll
    for (int u = 0; u < 4; ++u) fma4(sm_w[k + u * G], v[u], acc[u]);
  }
  for (; k < nparts; k += G) fma4(sm_w[k], o[size_t(k) * R + xv], acc[0]);
  float4 r;
  r.x = (acc[0].x + acc[1].x) + (acc[2].x + acc[3].x);
  r.y = (acc[0].y + acc[1].y) + (acc[2].y + acc[3].y);
  r.z = (acc[0].z + acc[1].z) + (acc[2].z + acc[3].z);
  r.w = (acc[0].w + acc[1].w) + (acc[2].w + acc[3].w);
  *reinterpret_cast<float4*>(&sm_part[kg][4 * xv]) = r;
  __syncthreads();
  for (int x = threadIdx.x; x < D; x += kReduceThreads) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) sum += sm_part[g][x];
    out[x] = Tr::from_f32(sum / total);
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, bool bf16_out, hipStream_t s) {
  if (a.B == 0 || a.H == 0) return hipSuccess;
  const dim3 grid(a.H, a.B);
  const dim3 block(kReduceThreads);
  const size_t shmem = size_t(a.num_partitions) * sizeof(float);
  if (bf16_out && a.head_dim == 128)
    hipLaunchKernelGGL((lse_reduce_kernel<Bf16, 128>), grid, block, shmem, s, a);
  else if (bf16_out && a.head_dim == 64)
    hipLaunchKernelGGL((lse_reduce_kernel<Bf16, 64>), grid, block, shmem, s, a);
  else if (!bf16_out && a.head_dim == 128)
    hipLaunchKernelGGL((lse_reduce_kernel<F32, 128>), grid, block, shmem, s, a);
  else if (!bf16_out && a.head_dim == 64)
    hipLaunchKernelGGL((lse_reduce_kernel<F32, 64>), grid, block, shmem, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pagedkv
