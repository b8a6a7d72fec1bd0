// Prefill-chunk attention for gfx950 (bf16 Q/K/V, MFMA 32x32x16).
//
// A workgroup of NW waves owns one tile of 32*NW query rows of one sequence
// and one KV head g.  Rows are GQA-packed like the decode tile: row r of the
// tile is token t0 + r / G and query head g*G + r % G, so a K/V block staged
// in LDS serves all G heads of the group (page "Attention kernels", Open
// questions: GQA packing in the prefill kernel; page "32. Production attention
// kernels", One kernel for the whole batch).  Each wave owns 32 rows.
//
// The tile walks the sequence's pages in 64-key blocks and ends with the
// block holding the newest key that its last token may attend to, since no
// row of the tile sees anything later (page "32. Production attention
// kernels", One kernel for the whole batch: the causal bound of a query tile).  With bf16 pools and 128-dim heads
// the blocks go from global memory straight into LDS (global_load_lds, no
// register staging, no LDS stores) through a four-stage ring, three blocks
// ahead of the one being computed; rows are 256 bytes with their 16-byte
// chunks XOR-swizzled by key so the fragment reads stay conflict free.
// Otherwise blocks pass through a two-stage ring of padded rows, and each
// thread holds up to PF further blocks in registers (quantized pools are
// dequantized on the way).  256-dim heads over bf16 pools run
// prefill16_kernel (waves of 16 rows) instead.
// Per block and wave:
//   S^T[64 keys x 32 rows] = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS);
//   mask only blocks that reach the diagonal or the context end (page
//   "Attention kernels", Walking the block table: masking is confined to the
//   pages the diagonal crosses);
//   online softmax in float32 with exp2; the scale*log2(e) factor and the
//   running max meet in one FMA per score (page "Attention kernels", One
//   kernel family).  The reference max of a row only moves when a block's max
//   exceeds it by more than 8 (log2 units): probabilities then stay below 2^8,
//   and since the row sum uses the same reference the normalised result is
//   the same softmax, while most blocks skip the accumulator rescale;
//   P rounded to bf16 (same passage), its row sum taken from the rounded
//   values, O^T[D x 32 rows] += V^T . P^T on MFMA with V^T read transposed from
//   LDS (ds_read_b64_tr_b16) and P^T taken straight from the S^T accumulator.
// Keys past the context end, and keys before the tile's first window start,
// are zero-filled in LDS and never loaded.
//
// With a sliding window (page "32. Production attention kernels", the unified
// kernel's window mask) the key loop starts at the block holding the tile's
// first window start and masks the blocks below its last one; an attention
// sink (same page, Stretch exercises) is folded into each row's state before
// the normalisation, as one more score with no value row.
//
// Quantized pools (page "Attention kernels", INT8 cache): a block's 1-byte
// codes are loaded (half the bytes), multiplied by their key's scale and
// rounded to bf16 when the block is staged in LDS, so the loop itself is the
// bf16 one; the per-channel key smoothing is moved onto the query once.
//
// Tiles with more keys run first (page "Attention kernels", Open questions:
// heaviest causal blocks first), and the flat block index is remapped so
// that the tiles of one (sequence, KV head) land on the same XCD and share
// its L2.
#include <limits.h>

#include <type_traits>

#include "pa_device.h"

namespace pa {

// s_waitcnt immediate (gfx9 layout) that waits until at most n vector-memory
// operations are in flight and does not wait on the other counters
constexpr int vm_wait(int n) { return 0x3f70 | (n & 0xf) | ((n >> 4) << 14); }

template <int D, int NW, int PF, int KB_ = 64>
struct PrefillCfg {
  static constexpr int NTH = 64 * NW;            // threads per workgroup
  static constexpr int BM = 32 * NW;             // rows per workgroup
  static constexpr int KB = KB_;                 // keys per block
  static constexpr int KT = KB / 32;             // 32-key MFMA tiles per block
  static constexpr int DS = D / 16;              // k-steps of QK^T
  static constexpr int DT = D / 32;              // 32-dim output tiles
  static constexpr int CPL = D / 8;              // 16-byte chunks per key row
  static constexpr int LOADS = KB * CPL / NTH;   // 16-byte loads per thread per tensor
  static constexpr int KRS = D * 2 + 16;         // K row stride (bytes)
  static constexpr int VRS = D * 2 + 64;         // V row stride (bytes): the 4 rows of a transpose
                                                 // read land 16 banks apart
  static constexpr int KBYTES = KB * KRS;
  static constexpr int STAGE = KBYTES + KB * VRS;
  static constexpr int NSTAGE = 2;               // LDS ring depth
  static constexpr int LDS = NSTAGE * STAGE;
  static constexpr float TAU = 8.f;              // lazy-rescale threshold (log2 units)
};

// A thread's share of one K/V block in registers: 16-byte bf16 chunks, or
// for quantized pools the same 8 elements as 8-byte codes plus their key's
// K and V scales.
template <int D, int NW, int KB, int KQ = KV_BF16>
struct PrefillRegs {
  static constexpr int N = PrefillCfg<D, NW, 1, KB>::LOADS;
  using Chunk = typename std::conditional<KQ == KV_BF16, u32x4, u32x2>::type;
  Chunk k[N], v[N];
  float ks[KQ == KV_BF16 ? 1 : N], vs[KQ == KV_BF16 ? 1 : N];
};

// WIN: the launch has a sliding window (p.window > 0); KQ: the pools' code
// type (KvCode).  The plain instantiation carries none of their code.
// CAS: the cascade's prefix pass.  The tiles then cover every query token of
// the batch as one flat, non-causal sequence over the shared prefix (keys
// [0, p.prefix_len) of block-table row 0, read once for all requests; page
// "32. Production attention kernels", Stretch exercises: cascade attention),
// each workgroup takes one key range of the prefix, and the unnormalised
// state (acc, m, l) goes to the split workspace for the combine.
template <int D, int NW, int PF, int KB, bool WIN, int KQ, bool CAS = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void prefill_kernel(const AttnParams p) {
  using C = PrefillCfg<D, NW, PF, KB>;
  // direct global -> LDS staging (see above)
  constexpr bool DMA = KQ == KV_BF16 && D == 128;   // 256-dim bf16 heads run prefill16_kernel
  constexpr int ROWB = D * 2, BLKB = KB * ROWB, DSTAGE = 2 * BLKB, DNS = 4;
  constexpr int KPI = 1024 / ROWB;               // keys per 1 KiB DMA instruction
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per key row
  constexpr int LDS_BYTES = DMA ? DNS * DSTAGE : C::LDS;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  int b, g, qt, split = 0;
  if constexpr (CAS) {
    // prefix pass: block = (key range, KV head, token tile); all tiles weigh the same
    const int id = blockIdx.x;
    split = id % p.prefix_splits;
    const int rest = id / p.prefix_splits;
    g = rest % p.num_kv_heads;
    qt = rest / p.num_kv_heads;
    b = 0;                                      // the prefix's pages come from table row 0
  } else {
    // ---- XCD-aware block order: consecutive logical tiles share an XCD
    const int total = gridDim.x;
    const int id = blockIdx.x;
    const int xcd = id & 7, per = total >> 3, rem = total & 7;
    const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (id >> 3);
    const int nqt = p.num_qtiles;
    qt = nqt - 1 - logical % nqt;               // heaviest tile of a sequence first
    const int rest = logical / nqt;
    g = rest % p.num_kv_heads;
    b = rest / p.num_kv_heads;
  }

  const int s0 = CAS ? 0 : p.query_start_loc[b];
  const int n = CAS ? p.num_tokens : p.query_start_loc[b + 1] - s0;
  if (!CAS && n <= p.dec_max_n) return;         // decode class (or empty)
  const int G = p.group;
  const int TPT = p.tok_per_tile;
  const int t0 = qt * TPT;
  if (t0 >= n) return;
  const int tcount = min(TPT, n - t0);
  const int rows_valid = tcount * G;

  const int ps = p.page_size, psh = p.page_shift;
  // prefix pass: this workgroup's key range [k_lo, L) of the prefix
  const int k_lo = CAS ? split * p.prefix_split_keys : 0;
  const int L = CAS ? min(k_lo + p.prefix_split_keys, p.prefix_len)
                    : clampi(p.context_lens[b], 0, p.table_width * ps);
  const int causal = CAS ? 0 : p.causal;
  const int diag = L - n;
  const int k_hi = causal ? clampi(diag + t0 + tcount, 0, L) : L;   // keys any row can see
  const int full_lim = causal ? clampi(diag + t0 + 1, 0, L) : L;    // keys every row sees
  const int nblk = (k_hi + C::KB - 1) / C::KB;
  // sliding window: blocks before the first row's window start are skipped,
  // and keys below the last row's window start need the window mask
  const int window = WIN ? p.window : 0;
  const int wlo_tile = WIN ? max(0, diag + t0 - window + 1) : (CAS ? k_lo : 0);   // first row's lowest key
  const int blk0 = wlo_tile / C::KB;
  const int win_all = WIN ? diag + t0 + tcount - window : INT_MIN;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int rl = 32 * wave + l32;               // row within the tile
  const bool row_ok = rl < rows_valid;
  const int my_tok = t0 + rl / G;               // token index within the sequence
  const int my_head = g * G + rl % G;

  // A negative scale is applied as a positive one on -q (negating bf16 is
  // exact), so the running max can be taken on raw scores.
  const float c = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // ---- Q^T as the B operand of S^T = K . Q^T
  bf16x8 qB[C::DS];
  if (row_ok) {
    const __bf16* qp = (const __bf16*)p.q + (int64_t)(s0 + my_tok) * p.q_stride_tok +
                       (int64_t)my_head * p.q_stride_head + 8 * h2;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      u32x4 w = *(const u32x4*)(qp + 16 * s);
      w ^= u32x4{qsign, qsign, qsign, qsign};
      qB[s] = __builtin_bit_cast(bf16x8, w);
    }
    if (KQ != KV_BF16 && p.k_smooth) {
      // scaling q per channel by the key smoothing cancels it in q . k
      const float* sm = p.k_smooth + (int64_t)g * D + 8 * h2;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        const f32x4 a = *(const f32x4*)(sm + 16 * s);
        const f32x4 c2 = *(const f32x4*)(sm + 16 * s + 4);
        const bf16x8 v = qB[s];
        qB[s] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2((float)v[0] * a[0], (float)v[1] * a[1]),
                                                 pack_bf16x2((float)v[2] * a[2], (float)v[3] * a[3]),
                                                 pack_bf16x2((float)v[4] * c2[0], (float)v[5] * c2[1]),
                                                 pack_bf16x2((float)v[6] * c2[2], (float)v[7] * c2[3])});
      }
    }
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

  // The 64 threads of a wave cover 64/CPL consecutive keys of one page, so
  // the page id is wave-uniform: it comes from a scalar load (counted by
  // lgkmcnt), and waiting for it never waits for the K/V loads in flight.
  auto gload = [&](int blk, PrefillRegs<D, NW, KB, KQ>& r) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * C::NTH + threadIdx.x;
      const int kl = idx / C::CPL, cc = idx % C::CPL;
      const int jw = __builtin_amdgcn_readfirstlane(blk * C::KB + (i * C::NTH + (threadIdx.x & ~63)) / C::CPL);
      const int j = blk * C::KB + kl;
      if constexpr (KQ == KV_BF16) {
        r.k[i] = u32x4{0u, 0u, 0u, 0u};
        r.v[i] = u32x4{0u, 0u, 0u, 0u};
      } else {
        r.k[i] = u32x2{0u, 0u};
        r.v[i] = u32x2{0u, 0u};
        r.ks[i] = 0.f;                           // keys outside the range dequantize to 0, whatever
        r.vs[i] = 0.f;                           // an unused slot's scale holds
      }
      if (jw < L) {
        const int lp = jw >> psh;
        const int pg = page_of(p, b, lp);
        const int64_t pbase = (int64_t)pg * p.kv_stride_page;
        if (j < L && ((!WIN && !CAS) || j >= wlo_tile)) {
          const int64_t off = pbase + (int64_t)(j - (lp << psh)) * p.kv_stride_slot + 8 * cc;   // elements
          if constexpr (KQ == KV_BF16) {
            r.k[i] = *(const u32x4*)(kbase + off);
            r.v[i] = *(const u32x4*)(vbase + off);
          } else {
            r.k[i] = *(const u32x2*)((const char*)p.k_pool + (int64_t)g * p.kv_stride_head + off);
            r.v[i] = *(const u32x2*)((const char*)p.v_pool + (int64_t)g * p.kv_stride_head + off);
            const int64_t so = (int64_t)pg * p.sc_stride_page + (int64_t)(j - (lp << psh)) * p.sc_stride_slot +
                               (int64_t)g * p.sc_stride_head;
            r.ks[i] = p.k_scale[so];
            r.vs[i] = p.v_scale[so];
          }
        }
      }
    }
  };
  // quantized: 8 codes times their key's scale, rounded to bf16.  An int8
  // code c is converted as c + 128 and fma(c + 128, s, -128 s) = c s exactly
  // before the one rounding, so both forms give the same bits.
  auto dequant8 = [&](u32x2 w, float sc) -> u32x4 {
    float f[8];
    if constexpr (KQ == KV_INT8) {
      const float off = -128.f * sc;
      const uint32_t u0 = w.x ^ 0x80808080u, u1 = w.y ^ 0x80808080u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = fmaf((float)((u0 >> (8 * e)) & 0xffu), sc, off);
        f[4 + e] = fmaf((float)((u1 >> (8 * e)) & 0xffu), sc, off);
      }
    } else {
      float a[4], h[4];
      codes4_to_f32<KQ == KV_BF16 ? KV_FP8 : KQ>(w.x, a);
      codes4_to_f32<KQ == KV_BF16 ? KV_FP8 : KQ>(w.y, h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = a[e] * sc;
        f[4 + e] = h[e] * sc;
      }
    }
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  };
  auto lstore = [&](int buf, const PrefillRegs<D, NW, KB, KQ>& r) {
    PA_LDS char* kl_ = lds + buf * C::STAGE;
    PA_LDS char* vl_ = kl_ + C::KBYTES;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int idx = i * C::NTH + threadIdx.x;
      const int kl = idx / C::CPL, cc = idx % C::CPL;
      if constexpr (KQ == KV_BF16) {
        *(PA_LDS u32x4*)(kl_ + kl * C::KRS + cc * 16) = r.k[i];
        *(PA_LDS u32x4*)(vl_ + kl * C::VRS + cc * 16) = r.v[i];
      } else {
        *(PA_LDS u32x4*)(kl_ + kl * C::KRS + cc * 16) = dequant8(r.k[i], r.ks[i]);
        *(PA_LDS u32x4*)(vl_ + kl * C::VRS + cc * 16) = dequant8(r.v[i], r.vs[i]);
      }
    }
  };

  const int l16 = lane & 15, gq = lane >> 4;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T = K . Q^T for the 32-key tiles of block blk (raw scores)
  auto qk = [&](int blk, f32x16 (&st)[C::KT]) {
    const PA_LDS char* kl_ = lds + (blk % C::NSTAGE) * C::STAGE;
    if constexpr (DMA) {
      // key row k holds global chunk c at position c ^ (k & 15)
      const PA_LDS char* kd = lds + (blk % DNS) * DSTAGE;
      // the first tile's fragments are requested up front; the second tile's
      // are requested one per MFMA of the first, so the first MFMA waits for
      // one read and no more than 15 reads are ever in flight (the counter's
      // range)
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ka[C::KT][C::DS];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s = 0; s < C::DS; ++s) {
          const int key = 32 * kt + l32;
          ka[kt][s] = *(const PA_LDS bf16x8*)(kd + key * ROWB + 16 * ((2 * s + h2) ^ (key & 15)));
        }
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
        f32x16 a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = 0.f;
#pragma unroll
        for (int s = 0; s < C::DS; ++s) a = mfma32(ka[kt][s], qB[s], a);
        st[kt] = a;
      }
      static_assert(C::KT == 2 && C::DS == 8, "read/MFMA interleave written for two 32-key tiles of 8 k-steps");
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);     // 8 LDS reads (tile 0)
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA (tile 0)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read (tile 1)
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);     // 8 MFMA (tile 1)
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (C::KT * C::DS <= 16) {
      // every K fragment of the block is requested before the first MFMA, so
      // the LDS latency is paid once per block rather than once per pair
      bf16x8 ka[C::KT][C::DS];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s = 0; s < C::DS; ++s)
          ka[kt][s] = *(const PA_LDS bf16x8*)(kl_ + (32 * kt + l32) * C::KRS + 16 * h2 + 32 * s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
        f32x16 a;
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = 0.f;
#pragma unroll
        for (int s = 0; s < C::DS; ++s) a = mfma32(ka[kt][s], qB[s], a);
        st[kt] = a;
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
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
    }
  };

  // Mask, online-softmax update and bf16 P^T of block blk.
  auto softmax = [&](int blk, f32x16 (&st)[C::KT], uint32_t (&pk)[C::KT][8]) {
    const int kb0 = blk * C::KB;
    if (kb0 + C::KB > full_lim || kb0 < win_all) {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb0 + 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const bool vis = j < L && (!causal || j <= diag + my_tok) && (!WIN || j > diag + my_tok - window);
          st[kt][r] = vis ? st[kt][r] : kNegInf;
        }
    }
    // one max3 per two scores, one chain per 32-key tile
    float tm[C::KT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      float m = st[kt][0];
#pragma unroll
      for (int r = 1; r < 15; r += 2) m = fmaxf(fmaxf(m, st[kt][r]), st[kt][r + 1]);
      tm[kt] = fmaxf(m, st[kt][15]);
    }
    float bmax = tm[0];
#pragma unroll
    for (int kt = 1; kt < C::KT; ++kt) bmax = fmaxf(bmax, tm[kt]);
    bmax = xor32_max(bmax);
    const float m_blk = bmax * c;               // -inf stays -inf (c > 0)
    // lazy rescale: move the reference max only when this block exceeds it by > TAU
    const bool need = m_blk > m_run + C::TAU;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // rows that keep their reference keep alpha = 1 (also while it is still
      // -inf: a row whose window starts later has seen no key yet)
      const float m_upd = need ? m_blk : m_run;
      const float alpha = need ? fast_exp2(m_run - m_blk) : 1.f;   // 0 from -inf
      l_run *= alpha;
      if constexpr (D == 256) {
        // The accumulators live in AGPRs here: each is scaled in place by an
        // AGPR -> VGPR -> AGPR round trip inside this (rare) branch, so the
        // block loop never holds VGPR copies of them.
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = acc[dt][r], t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\ts_nop 1\n\tv_mul_f32 %1, %1, %2\n\ts_nop 1\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t) : "v"(alpha));
            acc[dt][r] = x;
          }
      } else {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= alpha;
      }
      m_run = m_upd;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float p0 = fast_exp2(fmaf(st[kt][2 * w], c, -m_use));
        const float p1 = fast_exp2(fmaf(st[kt][2 * w + 1], c, -m_use));
        pk[kt][w] = pack_bf16x2(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kt][w]), ones, l_run, false);
      }
  };

  // O^T += V^T . P^T for block blk.  16-lane group gq reads dims
  // 32*dt + 16*(gq & 1) + l16 of keys kbase + 4*h2 + e and kbase + 8 + 4*h2 + e.
  auto pv = [&](int blk, const uint32_t (&pk)[C::KT][8]) {
    const PA_LDS char* vl_ = lds + (blk % C::NSTAGE) * C::STAGE + C::KBYTES;
    const PA_LDS char* vr = vl_ + (4 * h2 + (l16 >> 2)) * C::VRS + 32 * (gq & 1) + 8 * (l16 & 3);
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int kbase = 32 * kt + 16 * ks;
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pk[kt][4 * ks], pk[kt][4 * ks + 1], pk[kt][4 * ks + 2], pk[kt][4 * ks + 3]});
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          u32x2 a1, a2;
          if constexpr (DMA) {
            // value row k holds global chunk c at position c ^ 4 (k & 3): the
            // four rows of a 16-lane transpose read land on distinct banks
            const PA_LDS char* vd = lds + (blk % DNS) * DSTAGE + BLKB;
            const int vk = 4 * h2 + (l16 >> 2), cb = 2 * (gq & 1) + ((l16 & 3) >> 1), sub = 8 * (l16 & 1);
            const int k1 = kbase + vk, k2 = kbase + 8 + vk;
            a1 = lds_read_tr16(vd + k1 * ROWB + 16 * ((4 * dt + cb) ^ (4 * (k1 & 3))) + sub);
            a2 = lds_read_tr16(vd + k2 * ROWB + 16 * ((4 * dt + cb) ^ (4 * (k2 & 3))) + sub);
          } else {
            a1 = lds_read_tr16(vr + kbase * C::VRS + 64 * dt);
            a2 = lds_read_tr16(vr + (kbase + 8) * C::VRS + 64 * dt);
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a1.x, a1.y, a2.x, a2.y});
          acc[dt] = mfma32(va, pb, acc[dt]);
        }
      }
  };

  // ---- LDS holds block blk (and receives blk+1 after blk is computed);
  // registers hold blocks blk+1 .. blk+PF, issued PF blocks ahead.
  f32x16 st[C::KT];
  uint32_t pk[C::KT][8];
  if constexpr (DMA) {
    // Instruction i of wave w fills LDS bytes [(NW i + w) KiB, +1 KiB) of a
    // K or V block: keys KPI (NW i + w) .. +KPI-1, lane l writing position
    // l % CPR of key KPI (NW i + w) + l / CPR.  Every lane of every wave
    // issues every load, so all waves have the same count in flight: a key
    // outside [lo, L) (lo: the first key any row of the tile uses) loads the
    // nearest key inside, a finite copy of a live row whose score is masked
    // and whose probability is 0.
    constexpr int DL = BLKB / (C::NTH * 16);        // loads per thread per tensor
    const int lkey = lane / CPR, lpos = lane % CPR;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lo = wlo_tile;
    // the lane's part of an address: its key within a KPI-key group (which
    // never straddles a page) and its swizzled chunk; with 256-byte rows it
    // is the same for every instruction, with 512-byte rows it alternates
    const int64_t lofs = (int64_t)lkey * p.kv_stride_slot;
    auto lane_k = [&](int i) {
      return (uint32_t)((lofs + 8 * (lpos ^ ((KPI * (NW * i + wv) + lkey) & 15))) * 2);   // bytes
    };
    auto lane_v = [&](int i) {
      return (uint32_t)((lofs + 8 * (lpos ^ (4 * ((KPI * (NW * i + wv) + lkey) & 3)))) * 2);
    };
    // page ids through the constant address space: scalar loads, which wait
    // on their own counter rather than on the block loads in flight
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)b * p.table_width);
    // raw page id of a whole-page block, fetched a block-compute ahead
    auto page_raw = [&](int blk) { return bt[min((blk * C::KB) >> psh, p.table_width - 1)]; };
    auto dma = [&](int blk, int pgraw) {
      PA_LDS char* kd = lds + (blk % DNS) * DSTAGE;
      if (blk * C::KB >= lo && blk * C::KB + C::KB <= L && ps >= C::KB) {
        // the whole block lies in one page: one page id for all its loads
        const int kb = blk * C::KB;
        const int lp = kb >> psh;
        const int pg = clampi(pgraw, 0, p.num_pages - 1);
        const int64_t base = (int64_t)pg * p.kv_stride_page + (int64_t)(kb - (lp << psh)) * p.kv_stride_slot;
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const int64_t row = (base + (int64_t)(KPI * (NW * i + wv)) * p.kv_stride_slot) * 2;   // bytes
          __builtin_amdgcn_global_load_lds((const void*)((const char*)kbase + row + lane_k(i)),
                                           (PA_LDS void*)(kd + (NW * i + wv) * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)((const char*)vbase + row + lane_v(i)),
                                           (PA_LDS void*)(kd + BLKB + (NW * i + wv) * 1024), 16, 0, 0);
        }
      } else if (blk * C::KB >= lo && blk * C::KB + C::KB <= L) {
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const int kw = blk * C::KB + KPI * (NW * i + wv);
          const int lp = kw >> psh;
          const int pg = clampi(bt[lp], 0, p.num_pages - 1);
          const int64_t row = ((int64_t)pg * p.kv_stride_page + (int64_t)(kw - (lp << psh)) * p.kv_stride_slot) * 2;
          __builtin_amdgcn_global_load_lds((const void*)((const char*)kbase + row + lane_k(i)),
                                           (PA_LDS void*)(kd + (NW * i + wv) * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)((const char*)vbase + row + lane_v(i)),
                                           (PA_LDS void*)(kd + BLKB + (NW * i + wv) * 1024), 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < DL; ++i) {
          const int kw = blk * C::KB + KPI * (NW * i + wv);
          const int jw = clampi(kw, lo, L - 1);
          const int j = clampi(kw + lkey, lo, L - 1);
          const int key = KPI * (NW * i + wv) + lkey;
          // j and jw share a KPI-key group (or are equal), hence a page
          const int lp = jw >> psh;
          const int pg = clampi(bt[lp], 0, p.num_pages - 1);
          const int64_t row = (int64_t)pg * p.kv_stride_page + (int64_t)(j - (lp << psh)) * p.kv_stride_slot;
          __builtin_amdgcn_global_load_lds((const void*)(kbase + row + 8 * (lpos ^ (key & 15))),
                                           (PA_LDS void*)(kd + (NW * i + wv) * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(vbase + row + 8 * (lpos ^ (4 * (key & 3)))),
                                           (PA_LDS void*)(kd + BLKB + (NW * i + wv) * 1024), 16, 0, 0);
        }
      }
    };
    // wait until at most `more` blocks (2 DL loads per thread each) issued
    // after the one needed next are still in flight
    auto wait_more = [&](int more) {
      if (more >= 3) __builtin_amdgcn_s_waitcnt(vm_wait(6 * DL));
      else if (more == 2) __builtin_amdgcn_s_waitcnt(vm_wait(4 * DL));
      else if (more == 1) __builtin_amdgcn_s_waitcnt(vm_wait(2 * DL));
      else __builtin_amdgcn_s_waitcnt(vm_wait(0));
    };
    static_assert(DNS >= 2 && DNS <= 4 && 2 * (DNS - 1) * DL < 64, "wait_more counts up to three blocks");
#pragma unroll
    for (int x = 0; x < DNS; ++x)
      if (blk0 + x < nblk) dma(blk0 + x, page_raw(blk0 + x));
    wait_more(min(DNS - 1, nblk - 1 - blk0));       // block blk0 landed
    __syncthreads();
    for (int blk = blk0; blk < nblk; ++blk) {
      const int pnext = page_raw(blk + DNS);          // in flight while the block computes
      qk(blk, st);
      softmax(blk, st, pk);
      pv(blk, pk);
      wait_more(min(DNS - 2, nblk - 1 - (blk + 1)));   // block blk+1 landed
      __syncthreads();
      if (blk + DNS < nblk) dma(blk + DNS, pnext);     // into the stage block blk left
    }
  } else {
  PrefillRegs<D, NW, KB, KQ> rg[PF];
  if (blk0 < nblk) {
    gload(blk0, rg[0]);
    lstore(blk0 & 1, rg[0]);
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (blk0 + 1 + j < nblk) gload(blk0 + 1 + j, rg[j]);
  }
  __syncthreads();
  for (int base = blk0; base < nblk; base += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int blk = base + k;
      if (blk < nblk) {
        qk(blk, st);
        softmax(blk, st, pk);
        pv(blk, pk);
        if (blk + 1 < nblk) lstore((blk + 1) & 1, rg[k]);
        __syncthreads();
        if (blk + 1 + PF < nblk) gload(blk + 1 + PF, rg[k]);
      }
    }
  }
  }

  // ---- normalise and write this lane's row (dims 32*dt + 8*(r/4) + 4*h2 + r%4)
  l_run = xor32_sum(l_run);
  if constexpr (CAS) {
    // prefix pass: the unnormalised state of the row for the combine (m in
    // log2 units, the reference the probabilities were taken against)
    if (row_ok) {
      const int64_t NH = (int64_t)p.num_tokens * p.num_q_heads;
      const int64_t ri = (int64_t)split * NH + (int64_t)(s0 + my_tok) * p.num_q_heads + my_head;
      float* wa = p.ws_acc + ri * D + 4 * h2;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(wa + 32 * dt + 8 * r4) = f32x4{acc[dt][4 * r4], acc[dt][4 * r4 + 1], acc[dt][4 * r4 + 2],
                                                   acc[dt][4 * r4 + 3]};
      if (h2 == 0) *(f32x2*)(p.ws_ml + ri * 2) = f32x2{m_run, l_run};
    }
    return;
  }
  if (p.sinks) {
    // the row's sink is one more score with no value row
    const float s2 = row_ok ? p.sinks[my_head] * kLog2e : kNegInf;
    const float mn = fmaxf(m_run, s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float e = fast_exp2(m_run - ms);
    l_run = l_run * e + fast_exp2(s2 - ms);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= e;
  }
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

// Tile shape per head size: rows per workgroup (32 per wave) and register
// prefetch depth, chosen so the kernel fits two waves per SIMD where it can.
template <int D> struct PrefillShape;
template <> struct PrefillShape<64> { static constexpr int NW = 8, PF = 2, KB = 64; };
template <> struct PrefillShape<128> { static constexpr int NW = 8, PF = 2, KB = 64; };
template <> struct PrefillShape<256> { static constexpr int NW = 4, PF = 1, KB = 64; };

static_assert(32 * PrefillShape<64>::NW == prefill_tile_rows(64), "host and kernel tile rows differ");
static_assert(32 * PrefillShape<128>::NW == prefill_tile_rows(128), "host and kernel tile rows differ");
static_assert(32 * PrefillShape<256>::NW == prefill_tile_rows(256), "host and kernel tile rows differ");
static_assert(PrefillShape<64>::KB == prefill_block_keys() && PrefillShape<128>::KB == prefill_block_keys() &&
              PrefillShape<256>::KB == prefill_block_keys(), "host and kernel block keys differ");

hipError_t launch_prefill16(const AttnParams& p, hipStream_t st);
hipError_t launch_prefix16(const AttnParams& p, hipStream_t st);

template <int D>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t st) {
  constexpr int NW = PrefillShape<D>::NW, PF = PrefillShape<D>::PF, KB = PrefillShape<D>::KB;
  const int64_t total = (int64_t)p.num_qtiles * p.num_kv_heads * p.num_seqs;
  const dim3 grid((unsigned)total), block(64 * NW);
  const bool win = p.window > 0;
  switch (p.kv_code) {
    case KV_INT8:
      if (win) hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, true, KV_INT8>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_INT8>), grid, block, 0, st, p);
      break;
    case KV_FP8:
      if (win) hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, true, KV_FP8>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_FP8>), grid, block, 0, st, p);
      break;
    default:
      // 256-dim heads over bf16 pools: the 16-row-wave kernel
      if constexpr (D == 256) {
        return launch_prefill16(p, st);
      } else {
        if (win) hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, true, KV_BF16>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_BF16>), grid, block, 0, st, p);
      }
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefix_t(const AttnParams& p, hipStream_t st) {
  constexpr int NW = PrefillShape<D>::NW, PF = PrefillShape<D>::PF, KB = PrefillShape<D>::KB;
  const int64_t total = (int64_t)p.num_qtiles * p.num_kv_heads * p.prefix_splits;
  const dim3 grid((unsigned)total), block(64 * NW);
  switch (p.kv_code) {
    case KV_INT8: hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_INT8, true>), grid, block, 0, st, p); break;
    case KV_FP8: hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_FP8, true>), grid, block, 0, st, p); break;
    default:
      // 128- and 256-dim heads over bf16 pools: 64-row tiles of prefill16.hip
      if constexpr (D == 128 || D == 256) {
        return launch_prefix16(p, st);
      } else {
        hipLaunchKernelGGL((prefill_kernel<D, NW, PF, KB, false, KV_BF16, true>), grid, block, 0, st, p);
      }
  }
  return hipGetLastError();
}

// The cascade's prefix pass (see CAS above); p.num_qtiles counts the tiles
// of the flat token range.
hipError_t launch_prefix(const AttnParams& p, hipStream_t st) {
  switch (p.head_dim) {
    case 64: return launch_prefix_t<64>(p, st);
    case 128: return launch_prefix_t<128>(p, st);
    case 256: return launch_prefix_t<256>(p, st);
    default: return hipErrorInvalidValue;
  }
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
