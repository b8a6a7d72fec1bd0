// A mixed batch in one launch: the workgroups of its three tile classes --
// 16-row decode tiles, 64-row tiles of a short prefill chunk and verification
// tiles -- make up one grid, so they share the chip without side streams or
// the events that fork and join them (page "32. Production attention
// kernels", One kernel for the whole batch: one launch serves every sequence
// class).  The flat workgroup index picks the class: decode tiles first, so
// they are dealt to the CUs before anything else, then prefill tiles (a
// compact grid of the batch's tiles, heaviest first inside a sequence), then
// verification tiles.  Beside a prefill class a balanced decode launch has
// about one workgroup per CU, whose four waves stream the batch's K/V from
// the start while the CU's other slot takes the prefill and verification
// tiles.  Each workgroup runs the same tile code as the class's own kernel,
// with the class's argument block.  Classes without sequences have no
// workgroups.
#include "decode_tile.h"
#include "prefill16_tile.h"

namespace pa {

template <int D> struct MixedLds {
  static constexpr int DEC = DecodeLds<D, 1, KV_BF16>::BYTES;
  static constexpr int T16 = tile16_lds_bytes<D>();
  static constexpr int BYTES = DEC > T16 ? DEC : T16;
};

// WIN: sliding window; BAL: the decode tiles run as a balanced launch.
template <bool WIN, bool BAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mixed_kernel(const AttnParams pp, const AttnParams pv, const AttnParams pd, const int n_pre, const int n_ver) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(1024))) char smem[MixedLds<D>::BYTES];
  PA_LDS char* lds = (PA_LDS char*)smem;
  // decode tiles take the first workgroups of the grid; f is the index in
  // the order prefill, verification, decode that the argument counts use
  const int n_dec = (int)gridDim.x - n_pre - n_ver;
  const int f = (int)blockIdx.x < n_dec ? n_pre + n_ver + (int)blockIdx.x : (int)blockIdx.x - n_dec;
  if (f < n_pre) {
    prefill16_tile<D, 4, WIN, T16_PREFILL>(pp, lds, f, 0, 0, n_pre);
  } else if (f < n_pre + n_ver) {
    // verification grid (split, KV head, sequence), split fastest
    const int i = f - n_pre, S = pv.num_splits, H = pv.num_kv_heads;
    prefill16_tile<D, 4, WIN, T16_VERIFY>(pv, lds, i % S, (i / S) % H, i / (S * H), 0);
  } else {
    const int i = f - n_pre - n_ver, H = pd.num_kv_heads;
    if constexpr (BAL) {
      // balanced grid (KV head, bal_wgs), KV head fastest
      decode_tile<D, 1, WIN, KV_BF16, 2, false, true>(pd, lds, i % H, i / H, 0);
    } else {
      // split grid (split, KV head, sequence), split fastest
      const int S = pd.num_splits;
      decode_tile<D, 1, WIN, KV_BF16, 2, false, false>(pd, lds, i % S, (i / S) % H, i / (S * H));
    }
  }
}

bool mixed_supported(int head_dim) { return head_dim == 128; }

// pp: prefill tiles (64-row tiles, pp.num_qtiles per (sequence, KV head)) or
// none (have_pre false); pv: verification tiles (pv.num_splits) or none; pd:
// 16-row decode tiles (balanced when pd.bal_wgs > 0) or none.
hipError_t launch_mixed(const AttnParams& pp, bool have_pre, const AttnParams& pv, bool have_ver,
                        const AttnParams& pd, bool have_dec, hipStream_t st) {
  if (pd.head_dim != 128) return hipErrorInvalidValue;
  const int64_t n_pre = have_pre ? (int64_t)pp.num_qtiles * pp.num_kv_heads : 0;   // compact tile slots
  const int64_t n_ver = have_ver ? (int64_t)pv.num_splits * pv.num_kv_heads * pv.num_seqs : 0;
  const bool bal = have_dec && pd.bal_wgs > 0;
  const int64_t n_dec = !have_dec ? 0
                        : bal ? (int64_t)pd.num_kv_heads * pd.bal_wgs
                              : (int64_t)pd.num_splits * pd.num_kv_heads * pd.num_seqs;
  const int64_t total = n_pre + n_ver + n_dec;
  if (total <= 0) return hipSuccess;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const bool win = pd.window > 0 || pd.key_lo > 0;
  const dim3 grid((unsigned)total);
  if (win) {
    if (bal) hipLaunchKernelGGL((mixed_kernel<true, true>), grid, dim3(256), 0, st, pp, pv, pd, (int)n_pre, (int)n_ver);
    else hipLaunchKernelGGL((mixed_kernel<true, false>), grid, dim3(256), 0, st, pp, pv, pd, (int)n_pre, (int)n_ver);
  } else {
    if (bal) hipLaunchKernelGGL((mixed_kernel<false, true>), grid, dim3(256), 0, st, pp, pv, pd, (int)n_pre, (int)n_ver);
    else hipLaunchKernelGGL((mixed_kernel<false, false>), grid, dim3(256), 0, st, pp, pv, pd, (int)n_pre, (int)n_ver);
  }
  return hipGetLastError();
}

}  // namespace pa
