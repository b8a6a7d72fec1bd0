// The 16-row-wave tile's kernel and its launches; the tile itself (what
// one workgroup computes, and why) is prefill16_tile.h.
#include "prefill16_tile.h"

namespace pa {

template <int D, int NW, bool WIN, int MODE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void prefill16_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[tile16_lds_bytes<D>()];
  prefill16_tile<D, NW, WIN, MODE>(p, (PA_LDS char*)smem, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x);
}

// 256-dim heads over bf16 pools: the prefill tiles.
hipError_t launch_prefill16(const AttnParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.num_qtiles * p.num_kv_heads * p.num_seqs;
  if (p.window > 0)
    hipLaunchKernelGGL((prefill16_kernel<256, 8, true, T16_PREFILL>), dim3((unsigned)total), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((prefill16_kernel<256, 8, false, T16_PREFILL>), dim3((unsigned)total), dim3(512), 0, st, p);
  return hipGetLastError();
}

// A short prefill (few 256-row tiles for the chip) over 64-row tiles,
// 128-dim heads; p.tok_per_tile and p.num_qtiles describe 64-row tiles.
hipError_t launch_prefill16_small(const AttnParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)p.num_qtiles * p.num_kv_heads));   // compact tile slots
  if (p.head_dim != 128) return hipErrorInvalidValue;
  if (p.window > 0) hipLaunchKernelGGL((prefill16_kernel<128, 4, true, T16_PREFILL>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((prefill16_kernel<128, 4, false, T16_PREFILL>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// The cascade's prefix pass over 64-row tiles of the flat token range
// (128- and 256-dim heads; p.num_qtiles counts the tiles).
hipError_t launch_prefix16(const AttnParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)p.num_qtiles * p.num_kv_heads * p.prefix_splits));
  if (p.head_dim == 128) hipLaunchKernelGGL((prefill16_kernel<128, 4, false, T16_CASCADE>), grid, dim3(256), 0, st, p);
  else if (p.head_dim == 256) hipLaunchKernelGGL((prefill16_kernel<256, 4, false, T16_CASCADE>), grid, dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Verification tiles of up to 64 rows over bf16 pools (128- and 256-dim
// heads): grid (splits, KV heads, sequences) as the decode tiles'.
bool verify16_supported(int head_dim) { return head_dim == 128 || head_dim == 256; }

template <int D>
static hipError_t launch_verify16_t(const AttnParams& p, hipStream_t st) {
  const dim3 grid(p.num_splits, p.num_kv_heads, p.num_seqs);
  if (p.window > 0) hipLaunchKernelGGL((prefill16_kernel<D, 4, true, T16_VERIFY>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((prefill16_kernel<D, 4, false, T16_VERIFY>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_verify16(const AttnParams& p, hipStream_t st) {
  switch (p.head_dim) {
    case 128: return launch_verify16_t<128>(p, st);
    case 256: return launch_verify16_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
