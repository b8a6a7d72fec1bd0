// Prefill-chunk attention for gfx950 (bf16 Q/K/V, MFMA 32x32x16).
//
// A workgroup of 4 waves owns one tile of 128 query rows of one sequence and
// one KV head g.  Rows are GQA-packed like the decode tile: row r of the tile
// is token t0 + r / G and query head g*G + r % G, so a K/V block staged in
// LDS serves all G heads of the group (page "Attention kernels", Open
// questions: GQA packing in the prefill kernel; page "32. Production attention
// kernels", One kernel for the whole batch).  Each wave owns 32 rows.
//
// The tile walks the sequence's pages in 64-key blocks, stopping at the key
// its last token can see (same page, "The key loop stops at the tile's last
// query").  Blocks are staged through a double-buffered LDS ring: the next
// block's K and V are fetched into registers while the current block is
// computed.  Per block and wave:
//   S^T[64 keys x 32 rows] = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS);
//   mask only blocks that reach the diagonal or the context end (page
//   "Attention kernels", Walking the block table: only pages that overlap the
//   diagonal are masked);
//   online softmax in float32 with exp2 (scale*log2 e folded in);
//   P rounded to bf16, O^T[D x 32 rows] += V^T . P^T on MFMA, V^T read
//   transposed from LDS (ds_read_b64_tr_b16), P^T taken straight from the
//   S^T accumulator registers.
// Keys past the context end are zero-filled in LDS, never loaded.
//
// Tiles with more keys run first (page "Attention kernels", Open questions:
// heaviest causal blocks first), and the flat block index is remapped so
// that the tiles of one (sequence, KV head) land on the same XCD and share
// its L2.
#include "pa_device.h"

namespace pa {

template <int D>
struct PrefillCfg {
  static constexpr int BM = 128;                 // rows per workgroup (4 waves x 32)
  static constexpr int KB = 64;                  // keys per block
  static constexpr int DS = D / 16;              // k-steps of QK^T
  static constexpr int DT = D / 32;              // 32-dim output tiles
  static constexpr int CPL = D / 8;              // 16-byte chunks per key row
  static constexpr int LOADS = KB * CPL / 256;   // 16-byte loads per thread per tensor
  static constexpr int KRS = D * 2 + 16;         // K row stride (bytes)
  static constexpr int VRS = D * 2 + 32;         // V row stride (bytes)
  static constexpr int KBYTES = KB * KRS;
  static constexpr int STAGE = KBYTES + KB * VRS;
  static constexpr int LDS = 2 * STAGE;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(const AttnParams p) {
  using C = PrefillCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  // ---- XCD-aware block order: consecutive logical tiles share an XCD
  const int total = gridDim.x;
  const int id = blockIdx.x;
  const int xcd = id & 7, per = total >> 3, rem = total & 7;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (id >> 3);
  const int nqt = p.num_qtiles;
  const int qt = nqt - 1 - logical % nqt;       // heaviest tile of a sequence first
  const int rest = logical / nqt;
  const int g = rest % p.num_kv_heads;
  const int b = rest / p.num_kv_heads;

  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  if (n <= p.dec_max_n) return;                 // decode class (or empty)
  const int G = p.group;
  const int TPT = p.tok_per_tile;
  const int t0 = qt * TPT;
  if (t0 >= n) return;
  const int tcount = min(TPT, n - t0);
  const int rows_valid = tcount * G;

  const int ps = p.page_size;
  const int L = clampi(p.context_lens[b], 0, p.table_width * ps);
  const int causal = p.causal;
  const int diag = L - n;
  const int k_hi = causal ? clampi(diag + t0 + tcount, 0, L) : L;   // keys any row can see
  const int full_lim = causal ? clampi(diag + t0 + 1, 0, L) : L;    // keys every row sees
  const int nblk = (k_hi + C::KB - 1) / C::KB;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int rl = 32 * wave + l32;               // row within the tile
  const bool row_ok = rl < rows_valid;
  const int my_tok = t0 + rl / G;               // token index within the sequence
  const int my_head = g * G + rl % G;

  // ---- Q^T as the B operand of S^T = K . Q^T
  bf16x8 qB[C::DS];
  if (row_ok) {
    const __bf16* qp = (const __bf16*)p.q + (int64_t)(s0 + my_tok) * p.q_stride_tok +
                       (int64_t)my_head * p.q_stride_head + 8 * h2;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) qB[s] = *(const bf16x8*)(qp + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < C::DS; ++s) qB[s] = bf16x8{};
  }

  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  const __bf16* kbase = (const __bf16*)p.k_pool + (int64_t)g * p.kv_stride_head;
  const __bf16* vbase = (const __bf16*)p.v_pool + (int64_t)g * p.kv_stride_head;
  PA_LDS char* lds = (PA_LDS char*)smem;

  u32x4 rk[C::LOADS], rv[C::LOADS];
  auto gload = [&](int blk) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * 256 + threadIdx.x;
      const int kl = idx / C::CPL, cc = idx % C::CPL;
      const int j = blk * C::KB + kl;
      if (j < L) {
        const int lp = j / ps;
        const int pg = page_of(p, b, lp);
        const int64_t off = (int64_t)pg * p.kv_stride_page + (int64_t)(j - lp * ps) * p.kv_stride_slot + 8 * cc;
        rk[i] = *(const u32x4*)(kbase + off);
        rv[i] = *(const u32x4*)(vbase + off);
      } else {
        rk[i] = u32x4{0u, 0u, 0u, 0u};
        rv[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto lstore = [&](int buf) {
    PA_LDS char* kl_ = lds + buf * C::STAGE;
    PA_LDS char* vl_ = kl_ + C::KBYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * 256 + threadIdx.x;
      const int kl = idx / C::CPL, cc = idx % C::CPL;
      *(PA_LDS u32x4*)(kl_ + kl * C::KRS + cc * 16) = rk[i];
      *(PA_LDS u32x4*)(vl_ + kl * C::VRS + cc * 16) = rv[i];
    }
  };

  if (nblk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int blk = 0; blk < nblk; ++blk) {
    const bool more = blk + 1 < nblk;
    if (more) gload(blk + 1);
    const PA_LDS char* kl_ = lds + (blk & 1) * C::STAGE;
    const PA_LDS char* vl_ = kl_ + C::KBYTES;
    const int kb0 = blk * C::KB;

    // S^T = K . Q^T for two 32-key tiles
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 a;
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = 0.f;
      const PA_LDS char* kr = kl_ + (32 * kt + l32) * C::KRS + 16 * h2;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        const bf16x8 ka = *(const PA_LDS bf16x8*)(kr + 32 * s);
        a = mfma32(ka, qB[s], a);
      }
      st[kt] = a;
    }

    const bool need_mask = kb0 + C::KB > full_lim;
    float cmax = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = st[kt][r] * p.scale_log2;
        if (need_mask) {
          const int j = kb0 + 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const bool vis = j < L && (!causal || j <= diag + my_tok);
          v = vis ? v : kNegInf;
        }
        st[kt][r] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float m_safe = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_safe);
    m_run = m_new;

    u32x4 pk[2][2][2];   // [kt][ks][half]: bf16 P^T operand, 8 values per (kt, ks)
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r0 = 8 * ks + 4 * hh;
          const uint32_t w0 = pack_bf16x2(fast_exp2(st[kt][r0] - m_safe), fast_exp2(st[kt][r0 + 1] - m_safe));
          const uint32_t w1 = pack_bf16x2(fast_exp2(st[kt][r0 + 2] - m_safe), fast_exp2(st[kt][r0 + 3] - m_safe));
          psum += (bf16_lo(w0) + bf16_hi(w0)) + (bf16_lo(w1) + bf16_hi(w1));
          pk[kt][ks][hh] = u32x4{w0, w1, 0u, 0u};
        }
    l_run = alpha * l_run + psum;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= alpha;

    // O^T += V^T . P^T.  16-lane group q = lane / 16 reads dims
    // 32*dt + 16*(q & 1) + (lane % 16) of keys kbase + 4*h2 + e and kbase + 8 + 4*h2 + e.
    const int l16 = lane & 15, gq = lane >> 4;
    const PA_LDS char* vr = vl_ + (4 * h2 + (l16 >> 2)) * C::VRS + 32 * (gq & 1) + 8 * (l16 & 3);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kbase = 32 * kt + 16 * ks;
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pk[kt][ks][0].x, pk[kt][ks][0].y, pk[kt][ks][1].x, pk[kt][ks][1].y});
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const u32x2 a1 = lds_read_tr16(vr + kbase * C::VRS + 64 * dt);
          const u32x2 a2 = lds_read_tr16(vr + (kbase + 8) * C::VRS + 64 * dt);
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a1.x, a1.y, a2.x, a2.y});
          acc[dt] = mfma32(va, pb, acc[dt]);
        }
      }

    if (more) lstore((blk + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and write this lane's row (dims 32*dt + 8*(r/4) + 4*h2 + r%4)
  l_run += shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    __bf16* op = (__bf16*)p.out + (int64_t)(s0 + my_tok) * p.o_stride_tok + (int64_t)my_head * p.o_stride_head + 4 * h2;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& a = acc[dt];
        *(u32x2*)(op + 32 * dt + 8 * r4) = u32x2{pack_bf16x2(a[4 * r4] * inv, a[4 * r4 + 1] * inv),
                                                 pack_bf16x2(a[4 * r4 + 2] * inv, a[4 * r4 + 3] * inv)};
      }
  }
}

template <int D>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t st) {
  const int64_t total = (int64_t)p.num_qtiles * p.num_kv_heads * p.num_seqs;
  hipLaunchKernelGGL((prefill_kernel<D>), dim3((unsigned)total), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const AttnParams& p, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_prefill_t<64>(p, st);
    case 128: return launch_prefill_t<128>(p, st);
    case 256: return launch_prefill_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
