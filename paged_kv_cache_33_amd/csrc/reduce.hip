// Log-sum-exp merge of split-KV partials.
//
// Each partition k of a sequence left (o_k, m_k, l_k): its normalised partial
// output, its max score and its denominator, in base-2 units.  Rescaling every
// partition to the common max M = max_k m_k is the online-softmax rule of
// "MLSys Engineer - Inference Systems Q&A", Q4 (multiply by exp(m_old - m_new)),
// applied to whole partitions:
//   w_k = l_k * 2^(m_k - M),   out = sum_k w_k o_k / sum_k w_k.
// One work-group per (query head, sequence); the weights are computed once into
// LDS, then each thread owns one or more output dims.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {
namespace {

constexpr int kReduceThreads = 128;

template <typename Tr>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_kernel(ReduceArgs a) {
  extern __shared__ float sm_w[];  // [num_partitions] weights
  __shared__ float sm_red[kReduceThreads / kWave];
  __shared__ float sm_total;
  using S = typename Tr::storage;

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int D = a.head_dim;
  const int ctx = a.context_lens[b];
  const int nparts = ctx > 0 ? (ctx + a.partition_size - 1) / a.partition_size : 0;
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
  const float* o = a.ws_o + base * D;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;

  // M = max_k m_k
  float mx = -INFINITY;
  for (int k = threadIdx.x; k < nparts; k += blockDim.x) mx = fmaxf(mx, m[k]);
  for (int off = 32; off >= 1; off >>= 1) mx = wave_xor_max(mx, off);
  if (lane == 0) sm_red[w] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < kReduceThreads / kWave; ++i) M = fmaxf(M, sm_red[i]);
  __syncthreads();

  // w_k and their sum
  float tot = 0.f;
  for (int k = threadIdx.x; k < nparts; k += blockDim.x) {
    const float wk = l[k] * fast_exp2(m[k] - M);
    sm_w[k] = wk;
    tot += wk;
  }
  for (int off = 32; off >= 1; off >>= 1) tot = wave_xor_add(tot, off);
  if (lane == 0) sm_red[w] = tot;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < kReduceThreads / kWave; ++i) t += sm_red[i];
    sm_total = t;
  }
  __syncthreads();
  const float inv = 1.f / sm_total;

  for (int x = threadIdx.x; x < D; x += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < nparts; ++k) acc = fmaf(sm_w[k], o[size_t(k) * D + x], acc);
    out[x] = Tr::from_f32(acc * inv);
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, bool bf16_out, hipStream_t s) {
  if (a.B == 0 || a.H == 0) return hipSuccess;
  const dim3 grid(a.H, a.B);
  const size_t shmem = size_t(a.num_partitions) * sizeof(float);
  if (bf16_out)
    hipLaunchKernelGGL(lse_reduce_kernel<Bf16>, grid, dim3(kReduceThreads), shmem, s, a);
  else
    hipLaunchKernelGGL(lse_reduce_kernel<F32>, grid, dim3(kReduceThreads), shmem, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
