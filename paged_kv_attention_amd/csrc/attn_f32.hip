// Float32 paged attention on the vector ALUs (gfx950).
//
// Float32 has no MFMA path worth its precision cost here, so each query row
// (token, query head, split) is one wave.  The wave walks its split's keys in
// chunks of 64: lane j scores key j of the chunk against the row's query
// (held in LDS, read as a broadcast), the chunk's maximum and the softmax
// state are wave reductions, and lane d accumulates output dims d, d+64, ...
// with the chunk's probabilities read lane by lane.  Everything stays float32
// (page "paged-attn-xpu", Requirements and limits: scores and softmax state
// float32, split partials float32) and only keys below the row's visible end
// are ever read, so slots past the context are never touched.  With a
// sliding window a row also starts at its own window start; split 0 folds an
// attention sink into its state as one more score with no value row (page
// "32. Production attention kernels", window mask and Stretch exercises).
#include "pa_device.h"

namespace pa {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnParams p) {
  constexpr int DPL = D / 64;                    // output dims per lane
  __shared__ float qs[D];
  // grid: x = split + S * (head + Hq * token_slot), y = sequence
  const int S = p.num_splits;
  int x = blockIdx.x;
  const int split = x % S;
  x /= S;
  const int h = x % p.num_q_heads;
  const int t = x / p.num_q_heads;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;

  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  if (t >= n) return;
  const int ps = p.page_size;
  const int L = clampi(p.context_lens[b], 0, p.table_width * ps);
  const int kend = p.causal ? clampi(L - n + t + 1, 0, L) : L;
  const int kpp = p.pages_per_split * ps;
  // splits cut the pages from the sequence's first window start (page 0
  // without a window); this row reads only its own window
  const int k_split = (split_page_base(L, n, p.window, ps) + split * p.pages_per_split) * ps;
  const int k_begin = p.window > 0 ? max(k_split, L - n + t - p.window + 1) : k_split;
  const int k_stop = min(k_split + kpp, kend);
  const int g = h / p.group;
  const int tok = s0 + t;

  const float* qp = (const float*)p.q + (int64_t)tok * p.q_stride_tok + (int64_t)h * p.q_stride_head;
  for (int d = lane; d < D; d += 64) qs[d] = qp[d];
  __syncthreads();

  const float* kb = (const float*)p.k_pool + (int64_t)g * p.kv_stride_head;
  const float* vb = (const float*)p.v_pool + (int64_t)g * p.kv_stride_head;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  for (int j0 = k_begin; j0 < k_stop; j0 += 64) {
    const int j = j0 + lane;
    float s = kNegInf;
    int64_t off = 0;
    if (j < k_stop) {
      const int lp = j / ps;
      off = (int64_t)page_of(p, b, lp) * p.kv_stride_page + (int64_t)(j - lp * ps) * p.kv_stride_slot;
      const f32x4* kr = (const f32x4*)(kb + off);
      float dot = 0.f;
#pragma unroll 4
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const f32x4 kv = kr[d4];
        dot = fmaf(qs[4 * d4], kv[0], dot);
        dot = fmaf(qs[4 * d4 + 1], kv[1], dot);
        dot = fmaf(qs[4 * d4 + 2], kv[2], dot);
        dot = fmaf(qs[4 * d4 + 3], kv[3], dot);
      }
      s = dot * p.scale_log2;
    }
    const float cmax = wave_max(s);
    const float m_new = fmaxf(m_run, cmax);
    const float m_safe = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_safe);
    const float pj = fast_exp2(s - m_safe);
    l_run = alpha * l_run + wave_sum(pj);
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    const int cnt = min(64, k_stop - j0);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj));
      const int64_t o = (int64_t)__builtin_amdgcn_readlane((int)(off & 0xffffffff), jj) |
                        ((int64_t)__builtin_amdgcn_readlane((int)(off >> 32), jj) << 32);
      const float* vr = vb + o;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pw, vr[lane + 64 * i], acc[i]);
    }
  }

  if (p.sinks && split == 0) {
    // the sink joins split 0 as one more score with no value row
    const float s2 = p.sinks[h] * kLog2e;
    const float mn = fmaxf(m_run, s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float e = fast_exp2(m_run - ms);
    l_run = l_run * e + fast_exp2(s2 - ms);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= e;
    m_run = mn;
  }
  const int64_t NH = (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;   // workspace rows per split
  if (S == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = (float*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head;
#pragma unroll
    for (int i = 0; i < DPL; ++i) op[lane + 64 * i] = acc[i] * inv;
  } else {
    const int64_t ri = (int64_t)split * NH + ((int64_t)b * p.ws_tok + t) * p.num_q_heads + h;
#pragma unroll
    for (int i = 0; i < DPL; ++i) p.ws_acc[ri * D + lane + 64 * i] = acc[i];
    if (lane == 0) {
      p.ws_ml[ri * 2] = m_run;
      p.ws_ml[ri * 2 + 1] = l_run;
    }
  }
}

template <int D>
static hipError_t launch_f32_t(const AttnParams& p, int max_q, hipStream_t st) {
  const int64_t gx = (int64_t)p.num_splits * p.num_q_heads * max_q;
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3((unsigned)gx, p.num_seqs), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_f32(const AttnParams& p, int max_q, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_f32_t<64>(p, max_q, st);
    case 128: return launch_f32_t<128>(p, max_q, st);
    case 256: return launch_f32_t<256>(p, max_q, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Split combine.  For output row (token, head) with partials (acc_s, m_s, l_s):
//   M = max_s m_s (0 if every split is empty), w_s = exp2(m_s - M),
//   out = sum_s w_s acc_s / sum_s w_s l_s, and zero when the sum is zero.
// This is the log-sum-exp merge of page "32. Production attention kernels"
// (Long contexts: split the keys) written for unnormalised partials, as in
// page "Attention and KV Cache" (Split-KV decode, Combine).  Splits are summed
// in index order, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(64) void combine_kernel(const AttnParams p) {
  constexpr int DPL = D / 64;
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  if (t >= n || n > p.comb_max_n) return;
  // rows of the 16-row decode tile and of the verify tile may use different
  // split counts; a class with one split was written by its decode kernel
  const int S = n * p.group <= 16 ? p.comb_splits_small : p.comb_splits_big;
  if (S <= 1) return;
  const int tok = s0 + t;
  // workspace rows per split: (sequence, step token) slots, or flat tokens
  const int64_t NH = p.ws_flat ? (int64_t)p.num_tokens * p.num_q_heads : (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;
  const int64_t row = p.ws_flat ? (int64_t)tok * p.num_q_heads + h : ((int64_t)b * p.ws_tok + t) * p.num_q_heads + h;
  // Splits are read in groups of 8 whose loads are all issued before any is
  // used (one memory latency per group and pass rather than one per split);
  // padding entries (-inf, 0) leave the sums bit for bit unchanged.
  float M = kNegInf;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = s0 + j < S ? p.ws_ml[((s0 + j) * NH + row) * 2] : kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) M = fmaxf(M, m[j]);
  }
  const float Ms = M == kNegInf ? 0.f : M;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float l = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float mv[8], lv[8], av[8][DPL];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t ri = (s0 + j) * NH + row;
      const bool in = s0 + j < S;
      mv[j] = in ? p.ws_ml[ri * 2] : kNegInf;
      lv[j] = in ? p.ws_ml[ri * 2 + 1] : 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) av[j][i] = in ? p.ws_acc[ri * D + lane * DPL + i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float w = fast_exp2(mv[j] - Ms);
      l = fmaf(w, lv[j], l);
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, av[j][i], acc[i]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (BF16) {
    __bf16* op = (__bf16*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) op[i] = (__bf16)(acc[i] * inv);
  } else {
    float* op = (float*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + lane * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) op[i] = acc[i] * inv;
  }
}

template <int D>
static hipError_t launch_combine_t(const AttnParams& p, bool bf16, hipStream_t st) {
  dim3 grid(p.num_q_heads, p.comb_tokens, p.num_seqs);
  if (bf16)
    hipLaunchKernelGGL((combine_kernel<D, true>), grid, dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((combine_kernel<D, false>), grid, dim3(64), 0, st, p);
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
