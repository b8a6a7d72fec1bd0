// The decode / verification tile's kernel and its launches; the tile itself
// (what one workgroup computes, and why) is decode_tile.h.
#include "decode_tile.h"

namespace pa {

// Grid: (split, KV head, sequence), (KV head, sequence, split) for a batch of
// 16-row tiles alone, or (KV head, bal_wgs) for a balanced launch.
template <int D, int NT, bool WIN, int KQ, int NB = 0, bool FW = false, bool BAL = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 256 && (WIN || KQ != KV_BF16 || NT == 2) ? 1 : 2)))
void decode_splitkv_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[DecodeLds<D, NT, KQ>::BYTES];
  decode_tile<D, NT, WIN, KQ, NB, FW, BAL>(p, (PA_LDS char*)smem, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int D, int NT, int KQ, int NB, bool FW, bool BAL>
static void launch_k(const AttnParams& p, bool win, dim3 grid, hipStream_t st) {
  if (win) hipLaunchKernelGGL((decode_splitkv_kernel<D, NT, true, KQ, NB, FW, BAL>), grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL((decode_splitkv_kernel<D, NT, false, KQ, NB, FW, BAL>), grid, dim3(256), 0, st, p);
}

template <int D, int NT, bool BAL>
static void launch_decode_b(const AttnParams& p, dim3 grid, hipStream_t st) {
  const bool win = p.window > 0 || p.key_lo > 0;
  switch (p.kv_code) {
    case KV_INT8:
      launch_k<D, NT, KV_INT8, 0, false, BAL>(p, win, grid, st);
      break;
    case KV_FP8:
      launch_k<D, NT, KV_FP8, 0, false, BAL>(p, win, grid, st);
      break;
    default:
      // Two chunks per wave in flight (see the main loop) for heads of up to
      // 128 dims: always in 16-row tiles, in 32- and 64-row tiles when the
      // launch has several splits; 256-dim heads do not have the registers
      if constexpr (NT == 1 && !BAL) {
        if (p.new_k) {                           // the step's new rows written by this launch
          launch_k<D, NT, KV_BF16, D <= 128 ? 2 : 0, true, false>(p, win, grid, st);
          break;
        }
      }
      if constexpr (D <= 128) {
        if (NT == 1 || p.num_splits > 1) {
          launch_k<D, NT, KV_BF16, 2, false, BAL>(p, win, grid, st);
          break;
        }
      }
      if constexpr (NT > 1 || D > 128) launch_k<D, NT, KV_BF16, 0, false, BAL>(p, win, grid, st);
  }
}

template <int D, int NT>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t st) {
  if constexpr (NT == 1) {
    if (p.bal_wgs > 0) {
      launch_decode_b<D, NT, true>(p, dim3(p.num_kv_heads, p.bal_wgs), st);
      return hipGetLastError();
    }
  }
  const dim3 grid = NT == 1 && p.head_first ? dim3(p.num_kv_heads, p.num_seqs, p.num_splits)
                                            : dim3(p.num_splits, p.num_kv_heads, p.num_seqs);
  launch_decode_b<D, NT, false>(p, grid, st);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnParams& p, int nt, hipStream_t st) {
  switch (p.head_dim) {
    case 64:
      return nt == 1 ? launch_decode_t<64, 1>(p, st) : nt == 2 ? launch_decode_t<64, 2>(p, st) : launch_decode_t<64, 4>(p, st);
    case 128:
      return nt == 1 ? launch_decode_t<128, 1>(p, st) : nt == 2 ? launch_decode_t<128, 2>(p, st) : launch_decode_t<128, 4>(p, st);
    case 256:
      return nt == 1 ? launch_decode_t<256, 1>(p, st) : nt == 2 ? launch_decode_t<256, 2>(p, st) : launch_decode_t<256, 4>(p, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pa
