// GQA-packed attention tiles over bf16 pools with waves of 16 query rows on
// v_mfma_f32_16x16x32_bf16 (gfx950), K/V blocks shared by the waves through
// LDS.  Three uses (MODE):
//   PREFILL  256-dim heads: the tile the host plans (128 rows of one sequence
//            and KV head g, row r = token t0 + r / G, query head g*G + r % G;
//            page "Attention kernels", Open questions: GQA packing in the
//            prefill kernel) in 8 waves.  A wave's accumulators (O^T: 256
//            dims x 16 rows, 64 registers), query fragments (32) and scores
//            (16) fit two waves per SIMD, so one wave's softmax and LDS waits
//            overlap the other's matrix work.
//   CASCADE  the cascade's prefix pass for 256-dim heads: every query token
//            of the batch as one flat non-causal sequence over one key range
//            of the shared prefix; the unnormalised state goes to the split
//            workspace.
//   VERIFY   verification steps (page "Attention kernels", Decode: verify
//            blocks of several tokens): the 16*NW rows of one (sequence, KV
//            head) against one key range (split) of its pages, 4 waves; the
//            tile reads each K/V block once from HBM into LDS and all row
//            groups use it (the decode tile gives every row group its own
//            copy).  One split writes the normalised rows, several write
//            partials for the combine, as the decode tiles do.
// Blocks of 64 keys go from global memory straight into LDS (global_load_lds)
// through a two-stage ring; each wave reads the whole K and V block from LDS
// for its 16 rows.
// Per block and wave:
//   S^T[64 keys x 16 rows] = K . Q^T (four 16-key tiles, eight 32-dim
//   k-steps; K row k holds global 16-byte chunk c at position c ^ (k & 15));
//   mask only blocks that reach the diagonal, the context end or a window
//   edge; online softmax in float32 with exp2 and the lazy rescale of the
//   32-row kernel (the reference max moves only when a block's max passes it
//   by more than 8, log2 units); P rounded to bf16 with its row sum taken
//   from the rounded values (page "Attention kernels", One kernel family);
//   O^T[256 dims x 16 rows] += V^T . P^T, V^T read transposed from LDS
//   (ds_read_b64_tr_b16; V row k holds chunk c at position c ^ 2 (k & 7), so
//   the 8 rows that 32 lanes of a transpose read touch use distinct banks),
//   P^T straight from the S^T accumulators: lane (q4, l16) holds the scores
//   of keys 16t + 4 q4 + r of row l16, which for the tile pair (2j, 2j+1)
//   is exactly the B operand of a 32-key k-step whose slot 8 q4 + e stands
//   for key 32j + 4 q4 + e (e < 4) or 32j + 16 + 4 q4 + e - 4; the V reads
//   use the same slot-to-key map.
// A sliding window and attention sinks behave as in the 32-row kernel (page
// "32. Production attention kernels", the unified kernel's window mask,
// Stretch exercises); in a verification tile with several splits the sink
// joins split 0's partial.
#pragma once

#include <limits.h>

#include "pa_device.h"

namespace pa {

// s_waitcnt immediate (gfx9 layout): at most n vector-memory operations in
// flight, the other counters not waited on
constexpr int vm_wait16(int n) { return 0x3f70 | (n & 0xf) | ((n >> 4) << 14); }

enum Tile16Mode { T16_PREFILL = 0, T16_CASCADE = 1, T16_VERIFY = 2 };

// LDS bytes of one tile (the ring of K/V blocks)
template <int D> constexpr int tile16_lds_bytes() { return 2 * 2 * 64 * D * 2; }

template <int D, int NW, bool WIN, int MODE>
__device__ __attribute__((always_inline)) void prefill16_tile(const AttnParams& p, PA_LDS char* smem, const int bx,
                                                              const int by, const int bz, const int gx) {
  constexpr bool CAS = MODE == T16_CASCADE, VER = MODE == T16_VERIFY;
  constexpr int NTH = 64 * NW, KB = 64;
  constexpr int ROWB = D * 2;                    // bytes per key row
  constexpr int BLKB = KB * ROWB;                // one tensor's block
  constexpr int DSTAGE = 2 * BLKB;               // K and V of a block
  constexpr int DNS = 2;                         // ring stages
  static_assert(DNS * DSTAGE == tile16_lds_bytes<D>(), "the kernel's LDS holds the ring");
  constexpr int KPI = 1024 / ROWB;               // keys per 1 KiB DMA instruction
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per key row
  constexpr int DL = BLKB / (NTH * 16);          // DMA loads per thread per tensor
  constexpr int DS = D / 32;                     // 32-dim k-steps of QK^T
  constexpr int DT = D / 16;                     // 16-dim output tiles of PV
  constexpr int KT = KB / 16;                    // 16-key tiles of S^T
  constexpr float TAU = 8.f;                     // lazy-rescale threshold (log2 units)
  static_assert(MODE != T16_PREFILL || NW == 4 || 16 * NW == prefill_tile_rows(D), "host and kernel tile rows differ");
  static_assert(prefill_block_keys() % KB == 0, "host blocks are whole kernel blocks");
  static_assert(DL >= 1 && ROWB <= 1024, "a DMA instruction covers whole key rows");

  int b, g, qt = 0, split = 0;
  if constexpr (VER) {
    split = bx;                         // split fastest, as the decode tiles
    g = by;
    b = bz;
  } else if constexpr (CAS) {
    const int id = bx;
    split = id % p.prefix_splits;
    const int rest = id / p.prefix_splits;
    g = rest % p.num_kv_heads;
    qt = rest / p.num_kv_heads;
    b = 0;
  } else if constexpr (NW == 4) {
    // 64-row tiles of short prefills, in a compact grid: p.num_qtiles tile
    // slots per KV head (a host bound on the batch's prefill tiles), slot j
    // the j-th tile of the batch's prefill sequences in sequence order,
    // heaviest first inside a sequence; consecutive slots go to different
    // XCDs (the chip's CUs rather than one XCD's L2).  Every wave finds its
    // slot's sequence by the same scan over the step lengths, 64 sequences
    // at a time; a slot past the batch's tiles has nothing to do.
    const int T = p.num_qtiles, TPTs = p.tok_per_tile;
    const int j = bx % T;
    g = bx / T;
    const int ln = threadIdx.x & 63;
    b = -1;
    int base = 0;
    for (int q0 = 0; q0 < p.num_seqs; q0 += 64) {
      const int sq = q0 + ln;
      int c = 0;
      if (sq < p.num_seqs) {
        const int nq = p.query_start_loc[sq + 1] - p.query_start_loc[sq];
        c = nq > p.dec_max_n ? (nq + TPTs - 1) / TPTs : 0;
      }
      int inc = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (ln >= o) inc += v;
      }
      const int tot = __builtin_amdgcn_readlane(inc, 63);
      if (j < base + tot) {
        const int at = __builtin_ctzll(__builtin_amdgcn_ballot_w64(base + inc > j));   // lane holding tile j
        const int cb = __builtin_amdgcn_readlane(c, at);
        const int before = base + __builtin_amdgcn_readlane(inc, at) - cb;
        b = q0 + at;
        qt = cb - 1 - (j - before);
        break;
      }
      base += tot;
    }
    if (b < 0) return;
  } else {
    // consecutive logical tiles share an XCD; the heaviest tile of a
    // sequence first
    const int total = gx;
    const int id = bx;
    const int xcd = id & 7, per = total >> 3, rem = total & 7;
    const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (id >> 3);
    const int nqt = p.num_qtiles;
    qt = nqt - 1 - logical % nqt;
    const int rest = logical / nqt;
    g = rest % p.num_kv_heads;
    b = rest / p.num_kv_heads;
  }

  const int s0 = CAS ? 0 : p.query_start_loc[b];
  const int n = CAS ? p.num_tokens : p.query_start_loc[b + 1] - s0;
  const int G = p.group;
  if constexpr (VER) {
    // the verification class of this launch; a step longer than the host
    // bound max_query_len (invalid input) would index split partials past
    // its workspace rows and is skipped
    if (n <= 0 || n > p.dec_max_n || n * G <= p.row_lo || n * G > p.row_hi) return;
    if (!p.ws_flat && n > p.ws_tok && (p.num_splits > 1 || p.force_partial)) return;
  } else if constexpr (!CAS) {
    if (n <= p.dec_max_n) return;               // decode class (or empty)
  }
  const int TPT = VER ? n : p.tok_per_tile;
  const int t0 = qt * TPT;
  if (t0 >= n) return;
  const int tcount = min(TPT, n - t0);
  const int rows_valid = tcount * G;

  // Keys [lo, KE) are this tile's range (keys outside it are masked and
  // never loaded); L is the context length the causal diagonal refers to.
  const int ps = p.page_size, psh = p.page_shift;
  const int window = WIN ? p.window : 0;
  int L, lo, KE;
  if constexpr (CAS) {
    lo = split * p.prefix_split_keys;
    L = KE = min(lo + p.prefix_split_keys, p.prefix_len);
  } else {
    L = clampi(p.context_lens[b], 0, p.table_width * ps);
    const int wlo = WIN ? max(0, L - n + t0 - window + 1) : 0;   // the first row's window start
    if constexpr (VER) {
      // the split's pages, counted from the first window start (decode tiles' split rule)
      const int npages = (L + ps - 1) / ps;
      const int pg0 = wlo / ps + split * p.pages_per_split;
      const int pg1 = min(pg0 + p.pages_per_split, npages);
      lo = max(pg0 * ps, wlo);
      KE = min(pg1 * ps, L);
    } else {
      lo = wlo;
      KE = L;
    }
  }
  const int causal = CAS ? 0 : p.causal;
  const int diag = L - n;
  const int k_hi = min(KE, causal ? clampi(diag + t0 + tcount, 0, L) : L);      // keys any row can see
  const int full_lim = min(KE, causal ? clampi(diag + t0 + 1, 0, L) : L);       // keys every row sees
  const int nblk = lo < k_hi ? (k_hi + KB - 1) / KB : 0;
  const int blk0 = lo / KB;
  const int win_all = WIN ? diag + t0 + tcount - window : INT_MIN;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int rl = 16 * wave + l16;               // the lane's row (B-operand column)
  const bool row_ok = rl < rows_valid;
  const int my_tok = t0 + rl / G;
  const int my_head = g * G + rl % G;

  const float c = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // ---- Q^T as the B operand: k-step s, lane (q4, l16): dims 32 s + 8 q4 .. +7 of row l16
  bf16x8 qB[DS];
  if (row_ok) {
    const __bf16* qp = (const __bf16*)p.q + (int64_t)(s0 + my_tok) * p.q_stride_tok +
                       (int64_t)my_head * p.q_stride_head + 8 * q4;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 w = *(const u32x4*)(qp + 32 * s);
      w ^= u32x4{qsign, qsign, qsign, qsign};
      qB[s] = __builtin_bit_cast(bf16x8, w);
    }
  } else {
#pragma unroll
    for (int s = 0; s < DS; ++s) qB[s] = bf16x8{};
  }

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const __bf16* kbase = (const __bf16*)p.k_pool + (int64_t)g * p.kv_stride_head;
  const __bf16* vbase = (const __bf16*)p.v_pool + (int64_t)g * p.kv_stride_head;
  PA_LDS char* lds = (PA_LDS char*)smem;

  // ---- DMA of block blk into stage blk % DNS.  Instruction i of wave w
  // fills LDS bytes [(NW i + w) KiB, +1 KiB) of the K or V block: keys
  // KPI (NW i + w) .. +KPI-1, lane l writing position l % CPR of key
  // KPI (NW i + w) + l / CPR with the global chunk that the swizzle puts
  // there.  A key outside [lo, KE) loads the nearest key inside: a finite copy
  // of a live row whose score is masked and whose probability is 0.
  const int lkey = lane / CPR, lpos = lane % CPR;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t lofs = (int64_t)lkey * p.kv_stride_slot;
  auto lane_k = [&](int i) {
    return (uint32_t)((lofs + 8 * (lpos ^ ((KPI * (NW * i + wv) + lkey) & 15))) * 2);   // bytes
  };
  auto lane_v = [&](int i) {
    return (uint32_t)((lofs + 8 * (lpos ^ (2 * ((KPI * (NW * i + wv) + lkey) & 7)))) * 2);
  };
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)b * p.table_width);
  auto page_raw = [&](int blk) { return bt[min((blk * KB) >> psh, p.table_width - 1)]; };
  auto dma = [&](int blk, int pgraw) {
    PA_LDS char* kd = lds + (blk % DNS) * DSTAGE;
    if (blk * KB >= lo && blk * KB + KB <= KE && ps >= KB) {
      // the whole block lies in one page
      const int kb = blk * KB;
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
    } else {
#pragma unroll
      for (int i = 0; i < DL; ++i) {
        const int kw = blk * KB + KPI * (NW * i + wv);
        const int jw = clampi(kw, lo, KE - 1);
        const int j = clampi(kw + lkey, lo, KE - 1);
        const int key = KPI * (NW * i + wv) + lkey;
        // j and jw share a KPI-key group (or are equal), hence a page
        const int lp = jw >> psh;
        const int pg = clampi(bt[lp], 0, p.num_pages - 1);
        const int64_t row = (int64_t)pg * p.kv_stride_page + (int64_t)(j - (lp << psh)) * p.kv_stride_slot;
        __builtin_amdgcn_global_load_lds((const void*)(kbase + row + 8 * (lpos ^ (key & 15))),
                                         (PA_LDS void*)(kd + (NW * i + wv) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vbase + row + 8 * (lpos ^ (2 * (key & 7)))),
                                         (PA_LDS void*)(kd + BLKB + (NW * i + wv) * 1024), 16, 0, 0);
      }
    }
  };
  static_assert(2 * (DNS - 1) * DL < 64, "the blocks in flight fit the wait count");

  // ---- S^T = K . Q^T for the 16-key tiles of block blk
  f32x4 st[KT];
  // (k-steps outer, tiles inner: consecutive MFMAs accumulate into different
  // tiles, so none waits for the one before)
  auto qk = [&](int blk) {
    const PA_LDS char* kr = lds + (blk % DNS) * DSTAGE + l16 * ROWB;
#pragma unroll
    for (int t = 0; t < KT; ++t) st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 ka = *(const PA_LDS bf16x8*)(kr + 16 * t * ROWB + 16 * ((4 * s + q4) ^ l16));
        st[t] = mfma16(ka, qB[s], st[t]);
      }
  };
  // masked maximum of block blk over the row (lanes l16, l16 + 16, + 32, + 48)
  auto block_max = [&](int blk) -> float {
    const int kb0 = blk * KB;
    if (kb0 + KB > full_lim || kb0 < win_all || kb0 < lo) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = kb0 + 16 * t + 4 * q4 + r;
          const bool vis = j >= lo && j < KE && (!causal || j <= diag + my_tok) &&
                           (!WIN || j > diag + my_tok - window);
          st[t][r] = vis ? st[t][r] : kNegInf;
        }
    }
    float m = fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3]));
#pragma unroll
    for (int t = 1; t < KT; ++t) m = fmaxf(m, fmaxf(fmaxf(st[t][0], st[t][1]), fmaxf(st[t][2], st[t][3])));
    m = xor16_max(m);
    m = xor32_max(m);
    return m * c;                               // -inf stays -inf (c > 0)
  };
  // P^T of the two 32-key k-steps: pk[j] holds keys 32j + 4 q4 + e (words 0, 1)
  // and 32j + 16 + 4 q4 + e (words 2, 3)
  uint32_t pk[KT / 2][4];
  auto probs = [&]() {
    const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const float p0 = fast_exp2(fmaf(st[t][0], c, -m_use));
      const float p1 = fast_exp2(fmaf(st[t][1], c, -m_use));
      const float p2 = fast_exp2(fmaf(st[t][2], c, -m_use));
      const float p3 = fast_exp2(fmaf(st[t][3], c, -m_use));
      pk[t >> 1][2 * (t & 1)] = pack_bf16x2(p0, p1);
      pk[t >> 1][2 * (t & 1) + 1] = pack_bf16x2(p2, p3);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[t >> 1][2 * (t & 1)]), ones, l_run, false);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[t >> 1][2 * (t & 1) + 1]), ones, l_run,
                                              false);
    }
  };
  // O^T += V^T . P^T: lane (q4, l16) reads V[32j + 4 q4 + e][16 dt + l16] and
  // V[32j + 16 + 4 q4 + e][16 dt + l16] (e = 0..3) with two transpose reads
  auto pv = [&](int blk) {
    const PA_LDS char* vd = lds + (blk % DNS) * DSTAGE + BLKB;
    const int vk = 4 * q4 + (l16 >> 2);           // key within a 16-key half
    const int cb = (l16 & 3) >> 1, sub = 8 * (l16 & 1);
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[j][0], pk[j][1], pk[j][2], pk[j][3]});
      const int k1 = 32 * j + vk, k2 = k1 + 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2 a1 = lds_read_tr16(vd + k1 * ROWB + 16 * ((2 * dt + cb) ^ (2 * (k1 & 7))) + sub);
        const u32x2 a2 = lds_read_tr16(vd + k2 * ROWB + 16 * ((2 * dt + cb) ^ (2 * (k2 & 7))) + sub);
        const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a1.x, a1.y, a2.x, a2.y});
        acc[dt] = mfma16(va, pb, acc[dt]);
      }
    }
  };

  // wait until at most `more` blocks issued after the one needed next are
  // still in flight (2 DL loads per thread each)
  auto wait_more = [&](int more) {
    if (more >= 3) __builtin_amdgcn_s_waitcnt(vm_wait16(6 * DL));
    else if (more == 2) __builtin_amdgcn_s_waitcnt(vm_wait16(4 * DL));
    else if (more == 1) __builtin_amdgcn_s_waitcnt(vm_wait16(2 * DL));
    else __builtin_amdgcn_s_waitcnt(vm_wait16(0));
  };
#pragma unroll
  for (int x = 0; x < DNS; ++x)
    if (blk0 + x < nblk) dma(blk0 + x, page_raw(blk0 + x));
  wait_more(min(DNS - 1, nblk - 1 - blk0));       // block blk0 landed
  __syncthreads();
  for (int blk = blk0; blk < nblk; ++blk) {
    const int pnext = page_raw(blk + DNS);          // in flight while the block computes
    qk(blk);
    const float m_blk = block_max(blk);
    // lazy rescale: move the reference max only when this block exceeds it by > TAU
    const bool need = m_blk > m_run + TAU;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // rows that keep their reference keep alpha = 1 (also while it is still
      // -inf: a row whose window starts later has seen no key yet)
      const float m_upd = need ? m_blk : m_run;
      const float alpha = need ? fast_exp2(m_run - m_blk) : 1.f;   // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m_run = m_upd;
    }
    probs();
    pv(blk);
    wait_more(min(DNS - 2, nblk - 1 - (blk + 1)));   // block blk+1 landed
    __syncthreads();
    if (blk + DNS < nblk) dma(blk + DNS, pnext);     // into the stage block blk left
  }

  // ---- the row's sum over its four lanes; lane (q4, l16) holds dims 16 dt + 4 q4 + r
  l_run = xor16_sum(l_run);
  l_run = xor32_sum(l_run);
  if constexpr (CAS) {
    // prefix pass: the unnormalised state of the row for the combine (m in
    // log2 units, the reference the probabilities were taken against)
    if (row_ok) {
      const int64_t NH = (int64_t)p.num_tokens * p.num_q_heads;
      const int64_t ri = (int64_t)split * NH + (int64_t)(s0 + my_tok) * p.num_q_heads + my_head;
      float* wa = p.ws_acc + ri * D + 4 * q4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(wa + 16 * dt) = acc[dt];
      if (q4 == 0) *(f32x2*)(p.ws_ml + ri * 2) = f32x2{m_run, l_run};
    }
    return;
  }
  const bool partial = VER && (p.num_splits > 1 || p.force_partial);
  if (p.sinks && (!partial || split == 0)) {
    // the row's sink is one more score with no value row (in split 0's state
    // when the splits are merged later)
    const float s2 = row_ok ? p.sinks[my_head] * kLog2e : kNegInf;
    const float mn = fmaxf(m_run, s2);
    const float ms = mn == kNegInf ? 0.f : mn;
    const float e = fast_exp2(m_run - ms);
    l_run = l_run * e + fast_exp2(s2 - ms);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= e;
    m_run = mn;
  }
  if (partial) {
    // the split's unnormalised state (m in log2 units) at the decode tiles'
    // workspace row of (sequence, step token, head), or of the flat token
    if (row_ok) {
      const int64_t NH = p.ws_flat ? (int64_t)p.num_tokens * p.num_q_heads
                                   : (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;
      const int64_t rrow = p.ws_flat ? (int64_t)(s0 + my_tok) * p.num_q_heads + my_head
                                     : ((int64_t)b * p.ws_tok + my_tok) * p.num_q_heads + my_head;
      const int64_t ri = (int64_t)(p.split_base + split) * NH + rrow;
      float* wa = p.ws_acc + ri * D + 4 * q4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4*)(wa + 16 * dt) = acc[dt];
      if (q4 == 0) *(f32x2*)(p.ws_ml + ri * 2) = f32x2{m_run, l_run};
    }
    return;
  }
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    __bf16* op = (__bf16*)p.out + (int64_t)(s0 + my_tok) * p.o_stride_tok + (int64_t)my_head * p.o_stride_head +
                 4 * q4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *(u32x2*)(op + 16 * dt) = u32x2{pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                                      pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
  }
}

}  // namespace pa
