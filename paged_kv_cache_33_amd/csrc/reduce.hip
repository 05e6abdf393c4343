// Log-sum-exp merge of split-KV partials.
//
// Each partition k of a sequence left (o_k, m_k, l_k): its normalised partial
// output, its max score and its denominator, in base-2 units.  Rescaling every
// partition to the common max M = max_k m_k is the online-softmax rule of
// "MLSys Engineer - Inference Systems Q&A", Q4 (multiply by exp(m_old - m_new)),
// applied to whole partitions:
//   w_k = l_k * 2^(m_k - M),   out = sum_k w_k o_k / sum_k w_k.
#include "device_common.h"
#include "launch.h"

namespace pagedkv {
namespace {

constexpr int kReduceThreads = 512;

// One work-group per (query head, sequence).  Thread t owns the four output
// dims 4*(t % R) .. +3 (one 16-byte load per partition row, R = D / 4
// threads per row) and partitions k = t / R, t / R + G, ... (G = 512 / R
// groups).  Each thread merges its partitions as it loads them (the same
// rule, one partition at a time: a running max, the denominator and the sum
// rescaled whenever the max rises), four partitions' loads in flight at a
// time, so one pass over the partials suffices; the G group results meet in
// LDS, merged by the same rule.  A sequence of 196 partitions (100,000
// tokens in 512-token partitions) is 7 partitions per thread.
template <typename Tr, int D>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_kernel(ReduceArgs a) {
  constexpr int R = D / 4;
  constexpr int G = kReduceThreads / R;
  constexpr int U = 4;  // partitions in flight per thread
  __shared__ float sm_m[G];
  __shared__ float sm_l[G];
  __shared__ __attribute__((aligned(16))) float sm_o[G][D];
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

  const int xv = threadIdx.x % R;
  const int kg = threadIdx.x / R;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto merge = [&](float mk, float lk, float4 ok) {
    const float Mn = fmaxf(M, mk);
    const float so = fast_exp2(M - Mn);   // 0 while nothing is merged (M = -inf)
    const float wk = lk * fast_exp2(mk - Mn);
    L = fmaf(L, so, wk);
    acc.x = fmaf(acc.x, so, wk * ok.x);
    acc.y = fmaf(acc.y, so, wk * ok.y);
    acc.z = fmaf(acc.z, so, wk * ok.z);
    acc.w = fmaf(acc.w, so, wk * ok.w);
    M = Mn;
  };
  int k = kg;
  for (; k + (U - 1) * G < nparts; k += U * G) {
    float mk[U], lk[U];
    float4 ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mk[u] = m[k + u * G];
      lk[u] = l[k + u * G];
      ok[u] = o[size_t(k + u * G) * R + xv];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) merge(mk[u], lk[u], ok[u]);
  }
  for (; k < nparts; k += G) merge(m[k], l[k], o[size_t(k) * R + xv]);

  if (xv == 0) {
    sm_m[kg] = M;
    sm_l[kg] = L;
  }
  *reinterpret_cast<float4*>(&sm_o[kg][4 * xv]) = acc;
  __syncthreads();
  for (int x = threadIdx.x; x < D; x += blockDim.x) {
    float Mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) Mx = fmaxf(Mx, sm_m[g]);
    float tot = 0.f, sum = 0.f;
#pragma unroll 8
    for (int g = 0; g < G; ++g) {
      if (sm_m[g] == -INFINITY) continue;  // a group with no partition
      const float sc = fast_exp2(sm_m[g] - Mx);
      tot = fmaf(sm_l[g], sc, tot);
      sum = fmaf(sm_o[g][x], sc, sum);
    }
    out[x] = Tr::from_f32(sum / tot);
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, bool bf16_out, hipStream_t s) {
  if (a.B == 0 || a.H == 0) return hipSuccess;
  const dim3 grid(a.H, a.B);
  const dim3 block(kReduceThreads);
  const size_t shmem = 0;
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
