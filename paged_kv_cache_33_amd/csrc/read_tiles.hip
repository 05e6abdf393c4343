// Read-only pass over listed K/V tiles: the bandwidth ceiling of the decode's
// access pattern.  The decode step reads each (block, KV head) tile of both
// caches once, in an order fixed by the block tables; this kernel reads the
// same tiles with the same loads (non-temporal, 16 bytes per lane, one 4 KiB
// tile = four wave-wide loads) and does no arithmetic beyond folding the words
// into a checksum, so its rate is what the pool's layout and the HBM can give
// a kernel that only streams those tiles.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace pagedkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadWaves = kReadThreads / 64;

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Wave w of the grid takes entries w, w + W, ... (W = waves in the grid), two
// at a time so 2 x 2 x (tile_bytes / 1 KiB) loads are in flight per lane.
// Each work-group stores the XOR of every 32-bit word it read into
// sink[blockIdx.x] (a plain store: the loads cannot be dropped, and one word
// per work-group is all it writes).
template <int kChunks>  // wave-wide 16-byte loads per tile (tile bytes / 1 KiB)
__global__ __launch_bounds__(kReadThreads) void read_tiles_kernel(ReadTilesArgs a) {
  __shared__ uint32_t sm[kReadWaves];
  const int lane = threadIdx.x % 64;
  const int wv = threadIdx.x / 64;
  const int64_t nwaves = int64_t(gridDim.x) * kReadWaves;
  const char* kc = static_cast<const char*>(a.k_cache);
  const char* vc = static_cast<const char*>(a.v_cache);
  uint32_t acc = 0;
  auto tile_ok = [&](int32_t t) { return t >= 0 && int64_t(t) < a.pool_tiles; };
  int64_t e = int64_t(blockIdx.x) * kReadWaves + wv;
  for (; e + nwaves < a.n; e += 2 * nwaves) {
    const int32_t t0 = a.tiles[e], t1 = a.tiles[e + nwaves];
    const int64_t o0 = (tile_ok(t0) ? int64_t(t0) : 0) * a.tile_bytes + 16 * lane;
    const int64_t o1 = (tile_ok(t1) ? int64_t(t1) : 0) * a.tile_bytes + 16 * lane;
    uint32_t x0 = 0, x1 = 0;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int64_t off = int64_t(c) * 1024;
      x0 ^= fold(load_tile16(kc + o0 + off));
      x0 ^= fold(load_tile16(vc + o0 + off));
      x1 ^= fold(load_tile16(kc + o1 + off));
      x1 ^= fold(load_tile16(vc + o1 + off));
    }
    acc ^= (tile_ok(t0) ? x0 : 0u) ^ (tile_ok(t1) ? x1 : 0u);
  }
  if (e < a.n) {
    const int32_t t0 = a.tiles[e];
    if (tile_ok(t0)) {
      const int64_t o0 = int64_t(t0) * a.tile_bytes + 16 * lane;
  #pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t off = int64_t(c) * 1024;
        acc ^= fold(load_tile16(kc + o0 + off));
        acc ^= fold(load_tile16(vc + o0 + off));
      }
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc ^= uint32_t(__shfl_xor(int(acc), s));
  if (lane == 0) sm[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kReadWaves; ++w) x ^= sm[w];
    a.sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_read_tiles(const ReadTilesArgs& a, int groups, hipStream_t s) {
  if (groups <= 0) return hipSuccess;
  void (*k)(ReadTilesArgs) = nullptr;
  switch (a.tile_bytes) {
    case 1024: k = read_tiles_kernel<1>; break;
    case 2048: k = read_tiles_kernel<2>; break;
    case 4096: k = read_tiles_kernel<4>; break;
    case 8192: k = read_tiles_kernel<8>; break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(k, dim3(unsigned(groups)), dim3(kReadThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
