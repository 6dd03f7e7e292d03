// Whole-block copies between two block arrays, each in device memory or in
// pinned host memory: the data movement of swapping KV blocks out to host memory
// and back ("Dismantling the Memory Wall", "Cross-Tier Memory Offloading": blocks
// that overflow the GPU go down to CPU memory and are brought back before
// attention needs them).
//
// Work-groups take (listed block, array) items in turn, one per work-group by
// default or a capped number looping over them; 256 threads move a block in
// 16-byte pieces, four loads in flight each.  Reads from host memory cross the
// host link with microseconds of latency: the bytes in flight across the
// work-groups keep the link busy.  A cap leaves the rest of the chip to
// kernels running beside the copy (a prefetch under decode).  Ids outside
// either array are skipped.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int64_t items = static_cast<int64_t>(a.n) * a.num_arrays;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int32_t i = static_cast<int32_t>(it / a.num_arrays);
    const int32_t k = static_cast<int32_t>(it % a.num_arrays);
    const int32_t s = a.src_ids[i];
    const int32_t d = a.dst_ids[i];
    if (s < 0 || s >= a.src_blocks || d < 0 || d >= a.dst_blocks) continue;
    const int64_t nv = a.block_bytes[k] / 16;
    const u32x4* __restrict__ sp =
        reinterpret_cast<const u32x4*>(a.src[k] + static_cast<int64_t>(s) * a.block_bytes[k]);
    u32x4* __restrict__ dp = reinterpret_cast<u32x4*>(a.dst[k] + static_cast<int64_t>(d) * a.block_bytes[k]);
    constexpr int64_t T = 256;
    int64_t j = threadIdx.x;
    for (; j + 3 * T < nv; j += 4 * T) {
      const u32x4 x0 = __builtin_nontemporal_load(sp + j);
      const u32x4 x1 = __builtin_nontemporal_load(sp + j + T);
      const u32x4 x2 = __builtin_nontemporal_load(sp + j + 2 * T);
      const u32x4 x3 = __builtin_nontemporal_load(sp + j + 3 * T);
      dp[j] = x0;
      dp[j + T] = x1;
      dp[j + 2 * T] = x2;
      dp[j + 3 * T] = x3;
    }
    for (; j < nv; j += T) dp[j] = __builtin_nontemporal_load(sp + j);
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.n <= 0 || a.num_arrays <= 0) return hipSuccess;
  const int64_t items = static_cast<int64_t>(a.n) * a.num_arrays;
  const int64_t grid = a.max_workgroups > 0 ? std::min<int64_t>(items, a.max_workgroups) : items;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
