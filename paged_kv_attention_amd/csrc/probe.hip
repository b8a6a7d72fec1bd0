// HBM streaming-read probe: a measurement aid for the decode roofline, not
// part of the attention path.  It reads a device buffer once with 16-byte
// nontemporal loads, four per thread in flight, over a grid of 16384
// workgroups (64 per CU), and folds what it read into one word per
// workgroup so the loads cannot be dropped.  The rate it reaches is the
// practical ceiling for a kernel that streams K/V pages from HBM.
#include <stddef.h>
#include <stdint.h>

#include "pa_device.h"
#include "pagedattn.h"

namespace pa {

constexpr int kProbeBlocks = 16384;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, size_t n, uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * 256 * kProbeUnroll;
  for (size_t i = (size_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; i < n; i += stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int m = 32; m >= 1; m >>= 1) r ^= (uint32_t)__shfl_xor((int)r, m);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace pa

extern "C" pa_status pa_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || ((uintptr_t)sink & 3) != 0) return PA_ERR_SHAPE;
  if (sink_bytes < (size_t)pa::kProbeBlocks * 4) return PA_ERR_WORKSPACE;
  if (bytes == 0) return PA_OK;
  hipLaunchKernelGGL(pa::read_probe_kernel, dim3(pa::kProbeBlocks), dim3(256), 0, (hipStream_t)stream,
                     (const pa::u32x4*)buf, bytes / 16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
