// Float32 paged attention, GQA-packed, on the fp32 matrix cores (gfx950).
//
// One workgroup per (split x 16-row tile, KV head g, sequence b).  The rows of
// a tile are the sequence's step tokens times the G query heads that share KV
// head g, row r = token (r / G), head g*G + r % G; a sequence with more than
// 16 such rows takes several tiles.  Every K/V row of the split is read once
// for all rows of the tile (page "Attention kernels", Decode: GQA packing and
// split-KV; page "Attention and KV Cache", Multi-head, GQA, and MQA: the
// heads of a group read the same K/V).
//
// The tile's keys are cut into 16-key chunks; wave w of NW takes chunks w,
// w + NW, ... with its own online-softmax state, two chunks in registers at
// a time (the next one is loaded while this one is computed).  Per chunk:
//   S^T[16 keys x 16 rows] = K . Q^T    v_mfma_f32_16x16x4_f32, K loaded from
//                                       the page in 16-byte pieces straight
//                                       into the A operand, Q^T held in the B
//                                       operand (4 dims per k-step);
//   mask (only chunks that reach the causal diagonal, the range end or a
//   window edge); m' = max(m, rowmax), alpha = exp2(m - m'),
//   p = exp2(s - m') with the -inf guard;
//   O^T[D x 16 rows] += V^T . P^T       the same MFMA; P^T is already in the
//                                       B-operand layout of S^T's accumulator
//                                       registers, and lane (i, k) reads the
//                                       value V[key 4k + r][dim 16 t + i];
// V rows outside the tile's key range are selected to zero first, so a NaN
// in an unused slot never reaches an output.  Everything stays float32 (page
// "paged-attn-xpu", Requirements and limits: scores, softmax state and split
// partials in float32).  The waves merge their states in LDS in a fixed
// order.  With one split the normalised rows are written directly (one
// launch, no combine); otherwise the unnormalised partial (acc, m, l) goes to
// the workspace, and a split without keys writes the neutral (0, -inf, 0).
// A sliding window starts the key range at the tile's first window start and
// masks per row; split 0 folds an attention sink into its state as one more
// score with no value row (page "32. Production attention kernels", window
// mask and Stretch exercises).
#include <limits.h>

#include "pa_device.h"

namespace pa {

// Waves per workgroup: enough to spread a short context over the CU, with
// room for two register chunks per wave.
template <int D> struct F32Shape;
template <> struct F32Shape<64> { static constexpr int NW = 8; };
template <> struct F32Shape<128> { static constexpr int NW = 8; };
template <> struct F32Shape<256> { static constexpr int NW = 4; };

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
struct F32Chunk {
  f32x4 k[D / 16];                               // K[k0 + l16][16c + 4 q4 .. + 3]
  float v[D / 16][4];                            // V[k0 + 4 q4 + r][16t + l16]
};

template <int D, bool WIN>
__global__ __launch_bounds__(64 * F32Shape<D>::NW) void attn_f32_kernel(const AttnParams p) {
  constexpr int NW = F32Shape<D>::NW;
  constexpr int DC = D / 16;                     // 16-dim groups
  constexpr int ORS = D + 4;                     // merge buffer row stride (floats)
  __shared__ __attribute__((aligned(16))) float smem[NW * 16 * ORS + 2 * NW * 16];

  // grid: x = split + S * row tile, y = KV head, z = sequence
  const int S = p.num_splits;
  const int split = blockIdx.x % S, rt = blockIdx.x / S;
  const int g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;

  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  const int G = p.group;
  const int r0 = 16 * rt;
  // tokens past the host bound max_query_len (= p.ws_tok, invalid input) are
  // not computed: their workspace rows do not exist
  const int nq = min(n, p.ws_tok);
  if (nq <= 0 || r0 >= nq * G) return;
  const int nrows = min(16, nq * G - r0);

  const int ps = p.page_size;
  const int L = clampi(p.context_lens[b], 0, p.table_width * ps);
  const int diag = L - n;                        // token t sees keys j <= diag + t
  const int causal = p.causal;
  const int t_first = r0 / G, t_last = (r0 + nrows - 1) / G;
  const int window = WIN ? p.window : 0;
  // keys some row of the tile may see: [wlo, hi)
  const int hi = causal ? clampi(diag + t_last + 1, 0, L) : L;
  const int wlo = WIN && window > 0 ? max(0, diag + t_first - window + 1) : 0;
  // the split's pages (counted from the sequence's first window start)
  const int pg0 = split_page_base(L, n, window, ps) + split * p.pages_per_split;
  const int k_begin = max(pg0 * ps, wlo & ~15);  // 16-key chunks never straddle a page
  const int k_end = min(min((pg0 + p.pages_per_split) * ps, L), hi);
  const int nchunks = k_end > k_begin ? (k_end - k_begin + 15) / 16 : 0;
  // keys below mask_lim are visible to every row, and keys at or above
  // win_all lie inside every row's window
  const int mask_lim = min(k_end, causal ? diag + t_first + 1 : L);
  const int win_all = WIN && window > 0 ? diag + t_last - window + 1 : INT_MIN;

  // ---- Q^T as the B operand: lane (l16, q4) holds Q[row l16][16c + 4 q4 .. + 3]
  f32x4 qv[DC];
  const int my_row = r0 + l16;
  const int my_tok = my_row / G;                 // token of this lane's row
  if (l16 < nrows) {
    const float* qp = (const float*)p.q + (int64_t)(s0 + my_tok) * p.q_stride_tok +
                      (int64_t)(g * G + my_row % G) * p.q_stride_head + 4 * q4;
#pragma unroll
    for (int c = 0; c < DC; ++c) qv[c] = *(const f32x4*)(qp + 16 * c);
  } else {
#pragma unroll
    for (int c = 0; c < DC; ++c) qv[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  f32x4 acc[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const float* kbase = (const float*)p.k_pool + (int64_t)g * p.kv_stride_head;
  const float* vbase = (const float*)p.v_pool + (int64_t)g * p.kv_stride_head;
  auto slot_off = [&](int j) -> int64_t {        // key j of a chunk inside the sequence's pages
    const int lp = j / ps;
    return (int64_t)page_of(p, b, lp) * p.kv_stride_page + (int64_t)(j - lp * ps) * p.kv_stride_slot;
  };

  auto load = [&](int c, F32Chunk<D>& ch) {
    const int k0 = k_begin + 16 * c;
    // the chunk lies in one page: its page id is uniform
    const int64_t pbase = slot_off(k0);
    const float* kp = kbase + pbase + (int64_t)l16 * p.kv_stride_slot + 4 * q4;
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) ch.k[cc] = *(const f32x4*)(kp + 16 * cc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* vp = vbase + pbase + (int64_t)(4 * q4 + r) * p.kv_stride_slot + l16;
#pragma unroll
      for (int t = 0; t < DC; ++t) ch.v[t][r] = vp[16 * t];
    }
  };

  auto process = [&](int c, const F32Chunk<D>& ch) {
    const int k0 = k_begin + 16 * c;
    const bool need_mask = k0 + 16 > mask_lim || k0 < win_all;
    // S^T = K . Q^T
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < DC; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) st = mfma_f32(ch.k[cc][e], qv[cc][e], st);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = st[r] * p.scale_log2;
      if (need_mask) {
        const int j = k0 + 4 * q4 + r;
        const bool vis = j < k_end && (!causal || j <= diag + my_tok) &&
                         (!WIN || window <= 0 || j > diag + my_tok - window);
        v = vis ? v : kNegInf;
      }
      x[r] = v;
    }
    float cmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    cmax = fmaxf(cmax, shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_safe = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_safe);
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(x[r] - m_safe);
    l_run = alpha * l_run + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
    for (int t = 0; t < DC; ++t) acc[t] *= alpha;
    // O^T += V^T . P^T; value rows outside [wlo, k_end) are selected to zero
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = k0 + 4 * q4 + r;
      const bool live = !need_mask || (j < k_end && j >= wlo);
#pragma unroll
      for (int t = 0; t < DC; ++t) acc[t] = mfma_f32(live ? ch.v[t][r] : 0.f, pr[r], acc[t]);
    }
  };

  // two chunks per wave in registers: chunk c + NW is loaded while c is computed
  F32Chunk<D> buf[2];
  if (wave < nchunks) load(wave, buf[0]);
  for (int base = wave; base < nchunks; base += 2 * NW) {
    if (base + NW < nchunks) load(base + NW, buf[1]);
    process(base, buf[0]);
    if (base + NW < nchunks) {
      if (base + 2 * NW < nchunks) load(base + 2 * NW, buf[0]);
      process(base + NW, buf[1]);
    }
  }

  // ---- merge the waves' states (fixed order: bitwise repeatable)
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  float* Ob = smem;                              // [NW][16][ORS]
  float* Mw = smem + NW * 16 * ORS;              // [NW][16]
  float* Lw = Mw + NW * 16;                      // [NW][16]
  if (q4 == 0) Mw[wave * 16 + l16] = m_run;
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, Mw[w * 16 + l16]);
    const float e = fast_exp2(m_run - (M == kNegInf ? 0.f : M));
    if (q4 == 0) Lw[wave * 16 + l16] = l_run * e;
    // lane (l16, q4) holds O^T[16t + 4 q4 + r][row l16]
#pragma unroll
    for (int t = 0; t < DC; ++t)
      *(f32x4*)(Ob + (wave * 16 + l16) * ORS + 16 * t + 4 * q4) = acc[t] * e;
  }
  __syncthreads();

  const int64_t NH = (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;   // workspace rows per split
  for (int it = threadIdx.x; it < nrows * (D / 4); it += 64 * NW) {
    const int row = it / (D / 4), c4 = it % (D / 4);
    const int tok = (r0 + row) / G, head = g * G + (r0 + row) % G;
    float M = kNegInf, Lt = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      M = fmaxf(M, Mw[w * 16 + row]);
      Lt += Lw[w * 16 + row];
      o += *(const f32x4*)(Ob + (w * 16 + row) * ORS + 4 * c4);
    }
    if (p.sinks && split == 0) {
      // the sink joins split 0 as one more score with no value row
      const float s2 = p.sinks[head] * kLog2e;
      const float Mn = fmaxf(M, s2);
      const float Ms = Mn == kNegInf ? 0.f : Mn;
      const float e = fast_exp2(M - Ms);
      Lt = Lt * e + fast_exp2(s2 - Ms);
      o *= e;
      M = Mn;
    }
    if (S == 1) {
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
      float* op = (float*)p.out + (int64_t)(s0 + tok) * p.o_stride_tok + (int64_t)head * p.o_stride_head + 4 * c4;
      *(f32x4*)op = o * inv;
    } else {
      const int64_t ri = (int64_t)split * NH + ((int64_t)b * p.ws_tok + tok) * p.num_q_heads + head;
      *(f32x4*)(p.ws_acc + ri * D + 4 * c4) = o;
      if (c4 == 0) *(f32x2*)(p.ws_ml + ri * 2) = f32x2{M, Lt};
    }
  }
}

template <int D>
static hipError_t launch_f32_t(const AttnParams& p, hipStream_t st) {
  const int64_t gx = (int64_t)p.num_splits * p.num_qtiles;
  const dim3 grid((unsigned)gx, p.num_kv_heads, p.num_seqs), block(64 * F32Shape<D>::NW);
  if (p.window > 0) hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

// p.num_qtiles: 16-row tiles per sequence (ceil(max_query_len * G / 16)).
hipError_t launch_f32(const AttnParams& p, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_f32_t<64>(p, st);
    case 128: return launch_f32_t<128>(p, st);
    case 256: return launch_f32_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Split combine.  For output row (token, head) with partials (acc_s, m_s, l_s):
//   M = max_s m_s (0 if every split is empty), w_s = exp2(m_s - M),
//   out = sum_s w_s acc_s / sum_s w_s l_s, and zero when the sum is zero.
// This is the log-sum-exp merge of page "32. Production attention kernels"
// (Long contexts: split the keys) written for unnormalised partials, as in
// page "Attention and KV Cache" (Split-KV decode, Combine).
// A 256-thread workgroup merges one row at a time (the rows of a query head
// and sequence, every COMB_TSLOTS-th token): the threads form 256 / (D/4) groups,
// group k takes splits k, k + groups, ... (each thread 4 dims), and the
// first eight splits of every group arrive together with their (m, l) pairs,
// so a row with up to 8 * groups splits costs one memory latency.  The
// groups' sums are added in LDS in group order, so the result does not
// depend on scheduling.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) int32_t i32x2;

template <int D, bool BF16>
__device__ __attribute__((always_inline)) void combine_row(const AttnParams& p, const int h, const int t, const int b) {
  constexpr int CPR = D / 4;                     // threads per partial row (4 dims each)
  constexpr int NGR = 256 / CPR;                 // split groups
  constexpr int PB = 8;                          // splits of a group per batch
  constexpr int BATCH = PB * NGR;                // splits whose loads are in flight at once
  __shared__ float red[NGR][D + 4];
  __shared__ float red_m[NGR], red_l[NGR];
  const int grp = threadIdx.x / CPR, c4 = threadIdx.x % CPR;
  // the sequence's token range and, after a balanced launch, its partial
  // slots are requested together
  const bool bal = p.bal_wgs > 0;
  i32x2 meta = {0, 0};
  if (bal) meta = *(const i32x2*)(p.bal_meta + 2 * b);
  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  if (t >= n || n > p.comb_max_n) return;
  const int tok = s0 + t;
  // rows of the 16-row decode tile and of the verify tile may use different
  // split counts; a class with one split was written by its decode kernel
  int S = n * p.group <= 16 ? p.comb_splits_small : p.comb_splits_big;
  const float* acc_p = p.ws_acc;
  const float* ml_p = p.ws_ml;
  // workspace rows per split: (sequence, step token) slots, or flat tokens
  int64_t NH = p.ws_flat ? (int64_t)p.num_tokens * p.num_q_heads : (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;
  int64_t row = p.ws_flat ? (int64_t)tok * p.num_q_heads + h : ((int64_t)b * p.ws_tok + t) * p.num_q_heads + h;
  int s_base = 0;
  if (bal && n * p.group <= 16) {
    // balanced 16-row tiles: the sequence's pieces hold slots s_base ..
    // s_base + S - 1 of ws_tok * Hq rows each (one piece: written by the
    // decode kernel)
    s_base = meta[0];
    S = meta[1];
    acc_p = p.bal_acc;
    ml_p = p.bal_ml;
    NH = (int64_t)p.ws_tok * p.num_q_heads;
    row = (int64_t)t * p.num_q_heads + h;
  }
  if (S <= 1) return;
  // Group grp takes splits grp, grp + NGR, ...; the first BATCH splits'
  // (m, l) pairs and partial rows are loaded at once and kept, so a row with
  // up to BATCH splits costs one memory latency.  Padding entries are
  // (-inf, 0) and leave every sum bit for bit unchanged.
  auto load = [&](int s, f32x2 (&ml)[PB], f32x4 (&av)[PB]) {
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int sj = s + j * NGR;
      if (sj < S) {
        const int64_t ri = (s_base + sj) * NH + row;
        ml[j] = *(const f32x2*)(ml_p + ri * 2);
        av[j] = *(const f32x4*)(acc_p + ri * D + 4 * c4);
      } else {
        ml[j] = f32x2{kNegInf, 0.f};
        av[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  f32x2 ml0[PB];
  f32x4 av0[PB];
  load(grp, ml0, av0);
  float M = kNegInf;
#pragma unroll
  for (int j = 0; j < PB; ++j) M = fmaxf(M, ml0[j][0]);
  for (int s = grp + BATCH; s < S; s += BATCH) {
    float m[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) m[j] = s + j * NGR < S ? ml_p[((s_base + s + j * NGR) * NH + row) * 2] : kNegInf;
#pragma unroll
    for (int j = 0; j < PB; ++j) M = fmaxf(M, m[j]);
  }
  if (c4 == 0) red_m[grp] = M;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NGR; ++k) M = fmaxf(M, red_m[k]);
  const float Ms = M == kNegInf ? 0.f : M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
#pragma unroll
  for (int j = 0; j < PB; ++j) {
    const float w = fast_exp2(ml0[j][0] - Ms);
    l = fmaf(w, ml0[j][1], l);
    acc += w * av0[j];
  }
  for (int s = grp + BATCH; s < S; s += BATCH) {
    f32x2 ml[PB];
    f32x4 av[PB];
    load(s, ml, av);
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const float w = fast_exp2(ml[j][0] - Ms);
      l = fmaf(w, ml[j][1], l);
      acc += w * av[j];
    }
  }
  *(f32x4*)&red[grp][4 * c4] = acc;
  if (c4 == 0) red_l[grp] = l;
  __syncthreads();
  if (grp != 0) return;
  acc = *(const f32x4*)&red[0][4 * c4];
  l = red_l[0];
#pragma unroll
  for (int k = 1; k < NGR; ++k) {
    acc += *(const f32x4*)&red[k][4 * c4];
    l += red_l[k];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (BF16) {
    __bf16* op = (__bf16*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + 4 * c4;
    *(u32x2*)op = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  } else {
    float* op = (float*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + 4 * c4;
    *(f32x4*)op = acc * inv;
  }
}

// Grid: (query head, token slot, sequence) with at most COMB_TSLOTS token
// slots; slot y takes the sequence's tokens y, y + COMB_TSLOTS, ...  A grid
// with a slot for every token of the longest step idles most of its
// workgroups beside one-token steps (a mixed batch with a 16-token bound:
// 16,384 workgroups for 1,120 rows; 118.4-119.1 -> 116.5-118.0 us with four
// slots, 119.8-121.0 us with one, where a verification step's rows run in
// turn).
constexpr int COMB_TSLOTS = 4;

template <int D, bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const AttnParams p) {
  const int n = p.query_start_loc[blockIdx.z + 1] - p.query_start_loc[blockIdx.z];
  if (n > p.comb_max_n) return;
  for (int t = blockIdx.y; t < n; t += gridDim.y) combine_row<D, BF16>(p, blockIdx.x, t, blockIdx.z);
}

template <int D>
static hipError_t launch_combine_t(const AttnParams& p, bool bf16, hipStream_t st) {
  dim3 grid(p.num_q_heads, p.comb_tokens < COMB_TSLOTS ? p.comb_tokens : COMB_TSLOTS, p.num_seqs);
  if (bf16)
    hipLaunchKernelGGL((combine_kernel<D, true>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((combine_kernel<D, false>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine(const AttnParams& p, bool bf16, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_combine_t<64>(p, bf16, st);
    case 128: return launch_combine_t<128>(p, bf16, st);
    case 256: return launch_combine_t<256>(p, bf16, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// KV write: token i's K and V rows ([Hkv, D]) go to flat slot s =
// slot_mapping[i] = page * ps + offset of both pools; s < 0 writes nothing
// (page "Attention and KV Cache", Paged KV: the write map, -1 for padding
// tokens; the work scales with the step's tokens, never with the pool size).  One workgroup per token,
// 16-byte copies; slots outside the pool are skipped.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteParams p) {
  const int i = blockIdx.x;
  const int slot = p.slot_mapping[i];
  if (slot < 0 || slot >= p.num_pages * p.page_size) return;
  const int page = slot / p.page_size, off = slot % p.page_size;
  const int cpr = p.head_dim * p.elem_bytes / 16;     // 16-byte chunks per head row
  const int total = p.num_kv_heads * cpr;
  const int64_t eb = p.elem_bytes;
  const char* ksrc = (const char*)p.k_new + i * p.new_stride_tok * eb;
  const char* vsrc = (const char*)p.v_new + i * p.new_stride_tok * eb;
  char* kdst = (char*)p.k_pool + ((int64_t)page * p.kv_stride_page + (int64_t)off * p.kv_stride_slot) * eb;
  char* vdst = (char*)p.v_pool + ((int64_t)page * p.kv_stride_page + (int64_t)off * p.kv_stride_slot) * eb;
  for (int c = threadIdx.x; c < total; c += 256) {
    const int hh = c / cpr, cc = c % cpr;
    const int64_t so = hh * p.new_stride_head * eb + cc * 16;
    const int64_t dst = hh * p.kv_stride_head * eb + cc * 16;
    *(u32x4*)(kdst + dst) = *(const u32x4*)(ksrc + so);
    *(u32x4*)(vdst + dst) = *(const u32x4*)(vsrc + so);
  }
}

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t st) {
  hipLaunchKernelGGL(kv_write_kernel, dim3(p.num_tokens), dim3(256), 0, st, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantizing KV write (page "32. Production attention kernels", Quantized KV
// caches: quantize on write, once per token, one scale per (token, KV head)).
// One workgroup per token, one wave per (head, K or V) vector: each lane
// holds D/64 elements in float32; keys are divided by their smoothing
// factors; amax = max(max |x|, 1e-8) by a wave reduction (exact);
// scale = amax / q_max; code = x / scale rounded half-to-even and clamped to
// +-127 (int8) or converted to float8 E4M3 by the hardware's round-to-nearest-
// even conversion.  Each step is one correctly rounded float32 operation.
// ---------------------------------------------------------------------------
template <int D, int KQ>
__global__ __launch_bounds__(256) void kv_write_quant_kernel(const KvWriteParams p) {
  constexpr int EPL = D / 64;                    // elements per lane
  const int i = blockIdx.x;
  const int slot = p.slot_mapping[i];
  if (slot < 0 || slot >= p.num_pages * p.page_size) return;
  const int page = slot / p.page_size, off = slot % p.page_size;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float q_max = KQ == KV_INT8 ? 127.f : 448.f;
  for (int item = wave; item < 2 * p.num_kv_heads; item += 4) {
    const int h = item >> 1;
    const bool is_v = item & 1;
    const int64_t src = (int64_t)i * p.new_stride_tok + (int64_t)h * p.new_stride_head + lane * EPL;
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if (p.elem_bytes == 2) x[e] = (float)((const __bf16*)(is_v ? p.v_new : p.k_new))[src + e];
      else x[e] = ((const float*)(is_v ? p.v_new : p.k_new))[src + e];
    }
    if (!is_v && p.k_smooth) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[e] = x[e] / p.k_smooth[(int64_t)h * D + lane * EPL + e];
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
    a = wave_max(a);
    const float scale = fmaxf(a, 1e-8f) / q_max;
    uint8_t code[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float y = x[e] / scale;
      if constexpr (KQ == KV_INT8) {
        const float r = fminf(fmaxf(rintf(y), -127.f), 127.f);
        code[e] = (uint8_t)(int8_t)(int)r;
      } else {
        code[e] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xff);
      }
    }
    uint8_t* dst = (uint8_t*)(is_v ? p.v_pool : p.k_pool) + (int64_t)page * p.kv_stride_page +
                   (int64_t)off * p.kv_stride_slot + (int64_t)h * p.kv_stride_head + lane * EPL;
    if constexpr (EPL == 1) {
      dst[0] = code[0];
    } else if constexpr (EPL == 2) {
      *(uint16_t*)dst = (uint16_t)(code[0] | (code[1] << 8));
    } else {
      *(uint32_t*)dst = (uint32_t)code[0] | ((uint32_t)code[1] << 8) | ((uint32_t)code[2] << 16) |
                        ((uint32_t)code[3] << 24);
    }
    if (lane == 0)
      (is_v ? p.v_scale : p.k_scale)[(int64_t)page * p.sc_stride_page + (int64_t)off * p.sc_stride_slot +
                                     (int64_t)h * p.sc_stride_head] = scale;
  }
}

template <int D>
static hipError_t launch_kv_write_quant_t(const KvWriteParams& p, hipStream_t st) {
  if (p.kv_code == KV_INT8)
    hipLaunchKernelGGL((kv_write_quant_kernel<D, KV_INT8>), dim3(p.num_tokens), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((kv_write_quant_kernel<D, KV_FP8>), dim3(p.num_tokens), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_kv_write_quant(const KvWriteParams& p, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_kv_write_quant_t<64>(p, st);
    case 128: return launch_kv_write_quant_t<128>(p, st);
    case 256: return launch_kv_write_quant_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
