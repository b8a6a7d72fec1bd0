// GQA-packed split-KV decode / verify attention for gfx950 (bf16 K/V, MFMA).
//
// One workgroup per (split, KV head g, sequence b); 4 waves.  The rows of the
// query tile are all n tokens of the step times the G query heads that share
// KV head g, row r = token (r / G), head g*G + r % G, padded to 16*NT rows, so
// every K/V page of the split is read from memory once for the whole group
// (page "Attention kernels", Decode: GQA packing and split-KV; page "32.
// Production attention kernels", One kernel for the whole batch).
//
// The split's keys are cut into 32-key chunks; wave w walks chunks w, w+4,
// ... with its own online-softmax state (running max m, sum l, accumulator):
// it loads a chunk's K and V into registers, then computes it.  Per chunk:
//   S^T[32 keys x rows] = K . Q^T   on v_mfma_f32_16x16x32_bf16, K loaded
//                                   from the page straight into the A operand
//                                   (8 contiguous dims per lane);
//   mask (only chunks that reach the causal diagonal or the split's end);
//   m' = max(m, rowmax), alpha = exp2(m - m'), p = exp2(s - m') in float32;
//   O^T[D x rows] += V^T . P^T      V loaded in whole rows with streaming
//                                   (nontemporal) loads, staged through the
//                                   wave's LDS tile and read back transposed
//                                   (ds_read_b64_tr_b16);
//                                   P^T is already in the B-operand layout of
//                                   S^T's accumulator registers.
// Scores use exp2 with scale*log2(e) folded in (page "Attention kernels", One
// kernel family: scores in Float32 with exp2), and p is rounded to bf16 only
// for the PV product (same passage); l sums the rounded p, so the weights
// the product uses are exactly the ones the output is normalised by.  The
// -inf guard follows page "32. Production attention kernels" (m_safe), and V
// rows past the split's end are selected to zero before the product, so a
// NaN in an unused slot cannot reach an output (page "Attention and KV
// Cache", live length: a true select, not a multiply by zero).
//
// Sliding window (page "32. Production attention kernels", the unified
// kernel's window mask): the splits cut the pages from the first token's
// window start, chunks start at that start's 16-key tile, and chunks that
// reach below the last token's window start are masked per row.  Attention
// sinks (same page, Stretch exercises): split 0 folds the head's sink logit
// into its merged state as one more score with no value row.
//
// Quantized pools (page "Attention kernels", INT8 cache; page "32.
// Production attention kernels", Quantized KV caches): K and V hold 1-byte
// int8 or float8 E4M3 codes with one float32 scale per (slot, KV head).  The
// codes are converted to bf16 in registers (exactly), each score is scaled
// by its key's scale and each probability by its value's scale ahead of the
// PV product, and the per-channel key smoothing is moved onto the query
// once, where it cancels in every score.
// A chunk's 64 scales go through a small LDS area of the wave.
//
// The four waves' states are merged in LDS in a fixed order.  With one split
// the normalised output is written directly; otherwise the unnormalised
// partial (acc, m, l) goes to the float32 workspace for the combine kernel,
// and a split without keys writes the neutral (0, -inf, 0) (page "Attention
// and KV Cache", Split-KV decode).
#pragma once

#include <limits.h>

#include <type_traits>

#include "pa_device.h"

namespace pa {

template <int D, int KQ = KV_BF16>
struct DecodeCfg {
  static constexpr int KC = 32;                  // keys per chunk: two 16-key MFMA tiles
  static constexpr int DS = D / 32;              // 32-dim k-steps of QK^T
  static constexpr int DT = D / 16;              // 16-dim output tiles of PV
  static constexpr int EB = KQ == KV_BF16 ? 2 : 1;   // bytes per cached element
  static constexpr int CPL = D * EB / 16;        // 16-byte chunks per key row
  static constexpr int EPC = 16 / EB;            // elements per 16-byte chunk
  static constexpr int VLOADS = KC * CPL / 64;   // 16-byte V loads per lane per chunk
  static constexpr int ROW_BYTES = D * 2 + 32;   // bf16 V staging row stride (32 B pad: no bank
                                                 // conflicts between the 4 rows a transpose read touches)
  static constexpr int SC_BYTES = KQ == KV_BF16 ? 0 : 64 * 4;   // the chunk's K and V scales
  static constexpr int WAVE_LDS = KC * ROW_BYTES + SC_BYTES;
  static constexpr int NBUF = KQ == KV_BF16 ? 1 : 2;   // register chunks per wave (see the main loop)
};

template <int D, int NT, int KQ>
struct DecodeLds {
  static constexpr int ROWS = 16 * NT;
  static constexpr int ORS = D + 4;              // merge buffer row stride in floats
  static constexpr int STAGE = 4 * DecodeCfg<D, KQ>::WAVE_LDS;
  static constexpr int MERGE = (128 + ROWS * ORS) * 4;
  static constexpr int MAIN = STAGE > MERGE ? STAGE : MERGE;
  // balanced launches (16-row tiles): chunk counts and prefix sums of the
  // batch's sequences and the four waves' sums, kept across pieces
  static constexpr int BAL = NT == 1 ? (2 * bal_max_seqs() + 16) * 4 : 0;
  static constexpr int BYTES = MAIN + BAL;
};

template <int D, int KQ>
struct DecodeChunk {
  // K: bf16 pools, 8 dims of one key per (tile, k-step); 1-byte codes, 16
  // dims of one key per (tile, pair of k-steps), one 16-byte load each
  static constexpr int KN = KQ == KV_BF16 ? DecodeCfg<D, KQ>::DS : DecodeCfg<D, KQ>::DS / 2;
  using KReg = typename std::conditional<KQ == KV_BF16, bf16x8, u32x4>::type;
  KReg k[2][KN];
  u32x4 v[DecodeCfg<D, KQ>::VLOADS];
  float sc;                                      // quantized: scale of key lane%32, K (lane<32) or V
};

// WIN: the launch has a sliding window (p.window > 0); KQ: the pools' code
// type (KvCode).  The plain instantiation carries none of their code.
// NB: register chunks per wave, 0 for the code type's default (see the main
// loop).  FW: the launch also writes the step's new rows (bf16 pools, 16-row
// tiles; see the main loop).
template <int D, int NT, bool WIN, int KQ, int NB = 0, bool FW = false, bool BAL = false>
__device__ __attribute__((always_inline)) void decode_tile(const AttnParams& p, PA_LDS char* smem, const int bx,
                                                           const int by, const int bz) {
  using C = DecodeCfg<D, KQ>;
  constexpr bool QUANT = KQ != KV_BF16;
  constexpr int ROWS = 16 * NT;
  constexpr int ORS = DecodeLds<D, NT, KQ>::ORS;

  // the wave index is wave-uniform: chunk positions, page lookups and tile
  // addresses derived from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int G = p.group;

  // The workgroup's work is a list of pieces: sequence b, its keys
  // [k_begin, k_end).  A split launch has one, split `split` of sequence b.
  // Grid order: the hardware deals workgroups to the 8 XCDs in turn.  With
  // the split fastest, split 0 (the longest) of every sequence lands on the
  // same XCDs; a batch of decode tiles alone therefore runs with the KV head
  // fastest, which gives each XCD the same heads of every sequence and
  // split, an equal share of the work however ragged the sequences are.
  // Batches with prefill or verification tiles beside keep the split
  // fastest, which measured faster there.
  // A balanced launch (16-row tiles, grid (KV head, bal_wgs)) lays the
  // batch's 32-key chunks end to end and gives wave w = 4 u + (wave index)
  // the R chunks from w R on, one piece per sequence they touch: every wave,
  // and with two workgroups per CU every CU, reads the same bytes however
  // ragged the batch is (a CU streams about 30 GB/s, so the CU with the most
  // bytes would set the time).  Each wave takes its pieces on its own (no
  // barrier between them) and writes each piece's partial state; a piece
  // holding all of a sequence is written normalised.
  constexpr bool bal = BAL;
  static_assert(!BAL || NT == 1, "balanced launches take 16-row tiles");
  // a balanced launch's waves take their pieces apart: no workgroup barrier
  // after the prologue (the step's new rows are written before it)
  static_assert(!(BAL && FW), "balanced launches do not write the new rows");
  int g = 0, split = 0, bnext = 0, bend = 0, bal_lo = 0, bal_hi = 0, bal_u = 0;
  const int* Cs = nullptr;                      // balanced: chunks per sequence (-1: of this launch, no keys)
  const int* Qs = nullptr;                      // balanced: chunks of the sequences before it
  if constexpr (BAL) {
    g = bx;
    bal_u = by;
    int* cs = (int*)(smem + DecodeLds<D, NT, KQ>::MAIN);
    int* qs = cs + bal_max_seqs();
    int* wsum = qs + bal_max_seqs();
    const int B = p.num_seqs;                   // at most bal_max_seqs() (host rule)
    const int tid = threadIdx.x;
    // chunks of sequences 2 tid and 2 tid + 1 (0: another launch's)
    int cnt[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int bb = 2 * tid + j;
      int c = 0;
      if (bb < B) {
        const int sb = p.query_start_loc[bb], nb = p.query_start_loc[bb + 1] - sb;
        if (nb > 0 && nb <= p.dec_max_n && nb * G > p.row_lo && nb * G <= p.row_hi && nb <= p.ws_tok) {
          const int Lb = clampi(p.context_lens[bb], 0, p.table_width * p.page_size);
          const int wl = WIN ? max(p.window > 0 ? max(0, Lb - nb - p.window + 1) : 0, p.key_lo) : 0;
          const int kb = wl & ~15;
          c = Lb > kb ? (Lb - kb + C::KC - 1) / C::KC : -1;
        }
      }
      cnt[j] = c;
    }
    // exclusive prefix sums of the chunk counts over the workgroup
    const int loc = max(cnt[0], 0) + max(cnt[1], 0);
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o);
      if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = wsum[w];
      before += w < wave ? v : 0;
      total += v;
    }
    const int ex = before + inc - loc;
    cs[2 * tid] = cnt[0];
    cs[2 * tid + 1] = cnt[1];
    qs[2 * tid] = ex;
    qs[2 * tid + 1] = ex + max(cnt[0], 0);
    __syncthreads();
    const int nw = 4 * p.bal_wgs;               // waves per KV head
    const int R = max(p.bal_min_chunks, (total + nw - 1) / nw);
    bal_u = 4 * bal_u + wave;                   // from here on: the wave's index
    bal_lo = min(bal_u * R, total);
    bal_hi = min(bal_lo + R, total);
    // for the combine: the first partial slot of each sequence and how many
    // pieces it has (0 or 1: no partials)
    if (g == 0 && by == 0)
      for (int bb = tid; bb < B; bb += 256) {
        const int c = cs[bb], q = qs[bb];
        p.bal_meta[2 * bb] = bb + q / R;
        p.bal_meta[2 * bb + 1] = c > 0 ? (q + c - 1) / R - q / R + 1 : 0;
      }
    // rows of a sequence of this launch without any key are zero
    if (by == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (cnt[j] < 0) {
          const int bb = 2 * tid + j;
          const int sb = p.query_start_loc[bb], nb = p.query_start_loc[bb + 1] - sb;
          for (int r = 0; r < nb * G; ++r) {
            __bf16* op = (__bf16*)p.out + (int64_t)(sb + r / G) * p.o_stride_tok + (int64_t)(g * G + r % G) * p.o_stride_head;
            for (int d = 0; d < D; d += 8) *(u32x4*)(op + d) = u32x4{0u, 0u, 0u, 0u};
          }
        }
    }
    // the first sequence whose chunks reach bal_lo: the last one whose
    // prefix is at most bal_lo (it has chunks: the next prefix is larger)
    bnext = bend = B;
    if (bal_lo < bal_hi) {
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qs[mid] <= bal_lo) lo = mid;
        else hi = mid - 1;
      }
      bnext = __builtin_amdgcn_readfirstlane(lo);
    }
    Cs = cs;
    Qs = qs;
  } else {
    const bool hf = NT == 1 && p.head_first;
    split = hf ? bz : bx;
    g = hf ? bx : by;
    bnext = hf ? by : bz;
    bend = bnext + 1;
  }
  for (; bnext < bend; ++bnext) {
  const int b = bnext;
  int c_lo = 0, c_hi = 0;                       // balanced: the piece's chunks of sequence b
  bool whole;                                   // the piece holds all of the row's keys
  if (bal) {
    const int cb = __builtin_amdgcn_readfirstlane(Cs[b]);
    const int qb = __builtin_amdgcn_readfirstlane(Qs[b]);
    if (qb >= bal_hi) break;
    if (cb <= 0) continue;
    c_lo = max(bal_lo, qb) - qb;
    c_hi = min(bal_hi, qb + cb) - qb;
    whole = c_lo == 0 && c_hi == cb;
  } else {
    whole = p.num_splits == 1 && !p.force_partial;
  }
  const bool first = bal ? c_lo == 0 : split == 0;   // the piece with the row's first keys (sinks)
  const int s0 = p.query_start_loc[b];
  const int n = p.query_start_loc[b + 1] - s0;
  const int rows = n * G;
  if (n <= 0 || n > p.dec_max_n || rows <= p.row_lo || rows > p.row_hi) continue;
  // a step longer than the host bound max_query_len (invalid input) would
  // index split partials past its workspace rows: such a sequence is skipped
  if (!p.ws_flat && n > p.ws_tok && (bal || p.num_splits > 1 || p.force_partial)) continue;

  // Row groups: the step's rows form groups of 16, NG of them in use (the
  // tile's NT, or for a 64-row tile whose step fills at most 32 rows, 2).
  // Wave w computes group rg = w % NG over the chunks c with c % KG == w / NG:
  // the KG = 4/NG waves of a group split its chunks, and every wave keeps the
  // state of 16 rows only (so a 32- or 64-row tile needs no more registers
  // per wave than the 16-row one, and no wave of a partly filled tile idles).
  const int NG = NT == 4 && rows <= 32 ? 2 : NT;
  const int KG = BAL ? 1 : 4 / NG;               // a balanced wave takes all of its piece's chunks
  const int rg = BAL ? 0 : wave % NG, kg = BAL ? 0 : wave / NG;

  const int ps = p.page_size;
  const int L = clampi(p.context_lens[b], 0, p.table_width * ps);
  const int npages = (L + ps - 1) / ps;
  const int window = WIN ? p.window : 0;
  const int key_lo = WIN ? p.key_lo : 0;
  // with a lower key bound (a sliding window's start, or the end of a prefix
  // handled by the cascade's prefix pass) the splits cut the pages from the
  // tile's lowest bound on, and keys below it are never loaded
  const int wlo = WIN ? max(window > 0 ? max(0, L - n - window + 1) : 0, key_lo) : 0;
  const int pg0 = wlo / ps + split * p.pages_per_split;
  const int pg1 = min(pg0 + p.pages_per_split, npages);
  // 16-key tiles stay inside pages; a balanced piece has chunks [c_lo, c_hi)
  // of the keys from the 16-key tile of wlo on
  const int k_begin = bal ? (wlo & ~15) + C::KC * c_lo : WIN ? max(pg0 * ps, wlo & ~15) : pg0 * ps;
  const int k_end = bal ? min((wlo & ~15) + C::KC * c_hi, L) : min(pg1 * ps, L);
  const int nchunks = k_end > k_begin ? (k_end - k_begin + C::KC - 1) / C::KC : 0;

  const int causal = p.causal;
  const int diag = L - n;                       // token t sees keys j <= diag + t
  // keys below mask_lim are visible to every row of this tile, and so are
  // keys at or above win_all (inside the last token's window)
  const int mask_lim = min(k_end, causal ? diag + 1 : L);
  const int win_all = WIN ? max(key_lo, window > 0 ? diag + n - window : INT_MIN) : INT_MIN;

  // ---- query tile as the B operand of S^T = K . Q^T (row = lane % 16)
  // In k-step s lane (l16, q4) holds dims kdim(s) .. kdim(s) + 7 of its key
  // (A operand) and of its query row (B operand): 32 s + 8 q4 for bf16 pools;
  // for 1-byte codes 64 (s / 2) + 16 q4 + 8 (s % 2), so that the two k-steps
  // 2j, 2j + 1 of a lane take one 16-byte piece of the key row.  Any
  // assignment of dims to k slots that K and Q share gives the same dot
  // product.
  auto kdim = [&](int s) { return QUANT ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1) : 32 * s + 8 * q4; };
  bf16x8 qB[1][C::DS];
#pragma unroll
  for (int nt = 0; nt < 1; ++nt) {
    const int r = 16 * (rg + nt) + l16;
    if (r < rows) {
      const int tok = s0 + r / G, head = g * G + r % G;
      const __bf16* qp = (const __bf16*)p.q + (int64_t)tok * p.q_stride_tok + (int64_t)head * p.q_stride_head;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) qB[nt][s] = *(const bf16x8*)(qp + kdim(s));
      if (QUANT && p.k_smooth) {
        // scaling q per channel by the key smoothing cancels it in q . k
        const float* sm = p.k_smooth + (int64_t)g * D;
#pragma unroll
        for (int s = 0; s < C::DS; ++s) {
          const f32x4 a = *(const f32x4*)(sm + kdim(s));
          const f32x4 b = *(const f32x4*)(sm + kdim(s) + 4);
          const bf16x8 v = qB[nt][s];
          qB[nt][s] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2((float)v[0] * a[0], (float)v[1] * a[1]),
                                                       pack_bf16x2((float)v[2] * a[2], (float)v[3] * a[3]),
                                                       pack_bf16x2((float)v[4] * b[0], (float)v[5] * b[1]),
                                                       pack_bf16x2((float)v[6] * b[2], (float)v[7] * b[3])});
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < C::DS; ++s) qB[nt][s] = bf16x8{};
    }
  }

  // int8 pools enter the MFMAs as c + 128 (one conversion per code); the
  // scores then lose 128 * sum_d q_d and the outputs 128 * sum_j p'_j, with
  // qsum the row sum of the bf16 query and pvsum the row sum of the
  // probabilities the PV product used (rescaled with the accumulator).
  constexpr bool BIAS = KQ == KV_INT8;
  float qsum[1], pvsum[1];
#pragma unroll
  for (int nt = 0; nt < 1; ++nt) {
    float a = 0.f;
    if constexpr (BIAS) {
#pragma unroll
      for (int s = 0; s < C::DS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) a += (float)qB[nt][s][e];
      a += shfl_xor(a, 16);
      a += shfl_xor(a, 32);
    }
    qsum[nt] = a;
    pvsum[nt] = 0.f;
  }

  f32x4 acc[1][C::DT];
  float m_run[1], l_run[1];
#pragma unroll
  for (int nt = 0; nt < 1; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  PA_LDS char* vl = (PA_LDS char*)smem + wave * C::WAVE_LDS;
  PA_LDS float* scl = (PA_LDS float*)(vl + C::KC * C::ROW_BYTES);   // quantized: [K scales 32][V scales 32]
  // element strides are byte strides times EB
  const char* kbase = (const char*)p.k_pool + (int64_t)g * p.kv_stride_head * C::EB;
  const char* vbase = (const char*)p.v_pool + (int64_t)g * p.kv_stride_head * C::EB;

  // A 16-key tile never straddles a page (ps is a multiple of 16): its
  // address is a wave-uniform base (page, first slot) plus a per-lane offset
  // that is the same for every chunk.  A tile past the sequence's last page
  // re-reads that page; its keys are masked.
  const int pshift = __builtin_ctz(ps);          // ps is a power of two
  const int64_t se = p.kv_stride_slot * C::EB;   // bytes per slot
  constexpr int KPL = 64 / C::CPL;               // keys per V load of the wave
  // K: key l16 of the tile, 16-byte piece q4 of each 64-byte step; V load i:
  // key i * KPL + lane / CPL of the chunk, 16-byte piece lane % CPL.  The host
  // keeps 16 slots of a tile below 2^31 bytes.
  const uint32_t koff = (uint32_t)(l16 * se) + 16 * q4;
  const uint32_t voff = (uint32_t)((lane / C::CPL) * se) + 16 * (lane % C::CPL);
  struct TileAt {
    int page, slot;                              // page id and first slot of the tile
  };
  auto tile_at = [&](int kt) -> TileAt {
    int lp = kt >> pshift;
    const int sl = kt - (lp << pshift);
    lp = min(lp, npages - 1);
    return TileAt{page_of(p, b, lp), sl};
  };

  auto load = [&](int c, DecodeChunk<D, KQ>& ch) __attribute__((always_inline)) {
    const int k0 = k_begin + c * C::KC;
    TileAt ta[2];
    int64_t tb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      ta[t] = tile_at(k0 + 16 * t);
      tb[t] = (int64_t)ta[t].page * p.kv_stride_page * C::EB + ta[t].slot * se;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const char* kp = kbase + tb[t] + koff;
      if constexpr (QUANT) {
#pragma unroll
        for (int j = 0; j < C::DS / 2; ++j) ch.k[t][j] = *(const u32x4*)(kp + 64 * j);
      } else {
#pragma unroll
        for (int s = 0; s < C::DS; ++s) ch.k[t][s] = *(const bf16x8*)(kp + 32 * s * C::EB);
      }
    }
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int t = (i * KPL) / 16;               // uniform per load
      const char* vp = vbase + tb[t] + (i * KPL - 16 * t) * se + voff;
      // a wave's V load covers whole rows (full cache lines) that no other
      // workgroup reads: a streaming (nontemporal) load reads them faster.
      // In a 32- or 64-row tile the waves of the other row groups read the
      // same rows, from the cache.
      if constexpr (NT == 1) ch.v[i] = __builtin_nontemporal_load((const u32x4*)vp);
      else ch.v[i] = *(const u32x4*)vp;
    }
    if constexpr (QUANT) {
      // lane l: scale of key k0 + l % 32, of K for l < 32 and of V above, in
      // K's tile (l & 16) / 16 (keys outside the split are zeroed where the
      // chunk is used, so this load is not waited for here)
      const bool hi = (lane & 16) != 0;
      const int spage = hi ? ta[1].page : ta[0].page, sslot = (hi ? ta[1].slot : ta[0].slot) + (lane & 15);
      const int64_t so = (int64_t)spage * p.sc_stride_page + (int64_t)sslot * p.sc_stride_slot +
                         (int64_t)g * p.sc_stride_head;
      // one base and a uniform byte distance, not a choice between two
      // pointers of the argument block (which would move the whole block to
      // scratch memory)
      const char* ksb = (const char*)p.k_scale;
      const int64_t vdist = (const char*)p.v_scale - ksb;
      ch.sc = *(const float*)(ksb + (lane < 32 ? 0 : vdist) + so * 4);
    }
  };

  auto process = [&](int c, const DecodeChunk<D, KQ>& ch) __attribute__((always_inline)) {
    const int k0 = k_begin + c * C::KC;
    // the chunk reaches the causal diagonal, the split's end or a window edge
    const bool need_mask = k0 + C::KC > mask_lim || k0 < win_all;
    // V chunk -> this wave's LDS tile as bf16; rows past the split's end or
    // before every row's window are selected to zero
#pragma unroll
    for (int i = 0; i < C::VLOADS; ++i) {
      const int idx = i * 64 + lane;
      const int kl = idx / C::CPL, cc = idx % C::CPL;
      u32x4 v = ch.v[i];
      if (need_mask && (k0 + kl >= k_end || (WIN && k0 + kl < wlo))) v = u32x4{0u, 0u, 0u, 0u};
      if constexpr (BIAS) {
        const u32x2 a = i8x4_to_bf16_biased(v[0]), b2 = i8x4_to_bf16_biased(v[1]);
        const u32x2 c2 = i8x4_to_bf16_biased(v[2]), d = i8x4_to_bf16_biased(v[3]);
        PA_LDS char* row = vl + kl * C::ROW_BYTES + cc * 32;
        *(PA_LDS u32x4*)row = u32x4{a.x, a.y, b2.x, b2.y};
        *(PA_LDS u32x4*)(row + 16) = u32x4{c2.x, c2.y, d.x, d.y};
      } else if constexpr (QUANT) {
        const u32x2 a = codes4_to_bf16<KQ>(v[0]), b2 = codes4_to_bf16<KQ>(v[1]);
        const u32x2 c2 = codes4_to_bf16<KQ>(v[2]), d = codes4_to_bf16<KQ>(v[3]);
        PA_LDS char* row = vl + kl * C::ROW_BYTES + cc * 32;
        *(PA_LDS u32x4*)row = u32x4{a.x, a.y, b2.x, b2.y};
        *(PA_LDS u32x4*)(row + 16) = u32x4{c2.x, c2.y, d.x, d.y};
      } else {
        *(PA_LDS u32x4*)(vl + kl * C::ROW_BYTES + cc * 16) = v;
      }
    }
    f32x4 ksc[2], vsc[2];                         // quantized: scales of keys 16t + 4*q4 + r
    if constexpr (QUANT) {
      // keys outside the split (or below every window) get scale 0, so a
      // stale scale in an unused slot never meets a probability
      float sc = ch.sc;
      if (need_mask) {
        const int kk = k0 + (lane & 31);
        if (!(kk < k_end && (!WIN || kk >= wlo))) sc = 0.f;
      }
      scl[lane] = sc;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ksc[t] = *(const PA_LDS f32x4*)(scl + 16 * t + 4 * q4);
        vsc[t] = *(const PA_LDS f32x4*)(scl + 32 + 16 * t + 4 * q4);
      }
    }
    // S^T = K . Q^T
    f32x4 st[2][1];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 kf[C::DS];
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        if constexpr (QUANT) {
          const u32x4& w = ch.k[t][s >> 1];
          const uint32_t w0 = (s & 1) ? w.z : w.x, w1 = (s & 1) ? w.w : w.y;
          const u32x2 a = BIAS ? i8x4_to_bf16_biased(w0) : codes4_to_bf16<KQ>(w0);
          const u32x2 b2 = BIAS ? i8x4_to_bf16_biased(w1) : codes4_to_bf16<KQ>(w1);
          kf[s] = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b2.x, b2.y});
        } else {
          kf[s] = ch.k[t][s];
        }
      }
#pragma unroll
      for (int nt = 0; nt < 1; ++nt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::DS; ++s) a = mfma16(kf[s], qB[nt][s], a);
        st[t][nt] = a;
      }
    }
    bf16x8 pB[1];
#pragma unroll
    for (int nt = 0; nt < 1; ++nt) {
      float x[2][4];
      const int tok = (16 * (rg + nt) + l16) / G;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = (BIAS ? st[t][nt][r] - 128.f * qsum[nt] : st[t][nt][r]) *
                    (QUANT ? p.scale_log2 * ksc[t][r] : p.scale_log2);
          if (need_mask) {
            const int j = k0 + 16 * t + 4 * q4 + r;
            const bool vis = j < k_end && (!causal || j <= diag + tok) &&
                             (!WIN || (j >= key_lo && (window <= 0 || j > diag + tok - window)));
            v = vis ? v : kNegInf;
          }
          x[t][r] = v;
        }
      float cmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                         fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      cmax = xor16_max(cmax);
      cmax = xor32_max(cmax);
      const float m_new = fmaxf(m_run[nt], cmax);
      const float m_safe = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[nt] - m_safe);
      m_run[nt] = m_new;
      uint32_t pk[4];
      float psum = 0.f;
      if constexpr (QUANT) {
        // l sums p; the PV operand is p times the value's scale
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = fast_exp2(x[t][r] - m_safe);
            psum += e[r];
          }
          pk[2 * t] = pack_bf16x2(e[0] * vsc[t][0], e[1] * vsc[t][1]);
          pk[2 * t + 1] = pack_bf16x2(e[2] * vsc[t][2], e[3] * vsc[t][3]);
        }
        if constexpr (BIAS) {
          float ps_ = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) ps_ += bf16_lo(pk[i]) + bf16_hi(pk[i]);
          pvsum[nt] = alpha * pvsum[nt] + ps_;
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pk[2 * t] = pack_bf16x2(fast_exp2(x[t][0] - m_safe), fast_exp2(x[t][1] - m_safe));
          pk[2 * t + 1] = pack_bf16x2(fast_exp2(x[t][2] - m_safe), fast_exp2(x[t][3] - m_safe));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) psum += bf16_lo(pk[i]) + bf16_hi(pk[i]);
      }
      l_run[nt] = alpha * l_run[nt] + psum;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[nt][dt] *= alpha;
      pB[nt] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
    }
    // O^T += V^T . P^T ; V^T read transposed from LDS:
    // lane (q4, l16) gets V[4*q4 + e][16*dt + l16] and V[16 + 4*q4 + e][...]
    const PA_LDS char* r1 = vl + (4 * q4 + (l16 >> 2)) * C::ROW_BYTES + 8 * (l16 & 3);
    const PA_LDS char* r2 = r1 + 16 * C::ROW_BYTES;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const u32x2 a1 = lds_read_tr16(r1 + 32 * dt);
      const u32x2 a2 = lds_read_tr16(r2 + 32 * dt);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a1.x, a1.y, a2.x, a2.y});
#pragma unroll
      for (int nt = 0; nt < 1; ++nt) acc[nt][dt] = mfma16(va, pB[nt], acc[nt][dt]);
    }
  };

  // Register pipeline of NBUF chunks per wave: chunk i + 1 of the wave is
  // loaded while chunk i is computed (NBUF = 2; the launch picks it for
  // heads of up to 128 dims and for quantized pools), or each chunk is
  // loaded, then computed (NBUF = 1).  On the 64 x 4096 decode step two
  // chunks in flight measured 1 % faster than one.
  constexpr int NBUF = NB ? NB : C::NBUF;
  DecodeChunk<D, KQ> buf[NBUF];

  if constexpr (FW) {
    // The step's new rows of KV head g whose positions fall in this piece's
    // keys (a split's pages) go to their slots before any key is read (the write of
    // kv_cache_write, done by this launch: no other workgroup reads those
    // positions).  Both rows are loaded before either is stored.  A
    // workgroup barrier orders the stores before every wave's loads: only
    // this workgroup reads the rows, so no agent-scope fence (which would
    // write back the XCD's L2) is needed.
    constexpr int CPR = D * 2 / 16;             // 16-byte chunks per row
    for (int c = threadIdx.x; c < n * CPR; c += 256) {
      const int t = c / CPR, cc = c % CPR;
      const int pos = L - n + t;
      const int slot = p.new_slots[s0 + t];
      if (pos >= 0 && pos >= (bal ? k_begin : pg0 * ps) && pos < (bal ? k_end : pg1 * ps) && slot >= 0 &&
          slot < p.num_pages * ps) {
        const int64_t src = (int64_t)(s0 + t) * p.new_stride_tok + (int64_t)g * p.new_stride_head + 8 * cc;
        const int64_t dst = (int64_t)(slot / ps) * p.kv_stride_page + (int64_t)(slot % ps) * p.kv_stride_slot +
                            (int64_t)g * p.kv_stride_head + 8 * cc;
        const u32x4 kx = *(const u32x4*)((const __bf16*)p.new_k + src);
        const u32x4 vx = *(const u32x4*)((const __bf16*)p.new_v + src);
        *(u32x4*)((__bf16*)p.k_pool + dst) = kx;
        *(u32x4*)((__bf16*)p.v_pool + dst) = vx;
      }
    }
    __syncthreads();
  }
  // a row group past the step's rows has nothing to compute (its waves
  // still take part in the merge)
  const int my_chunks = 16 * rg < rows ? nchunks : 0;
  // this wave's chunks kg, kg + KG, ...: n_w of them, chunk i in buffer i % NBUF
  const int n_w = my_chunks > kg ? (my_chunks - kg + KG - 1) / KG : 0;
  auto chunk = [&](int i) { return kg + KG * i; };
  if constexpr (NBUF == 1) {
    for (int i = 0; i < n_w; ++i) {
      load(chunk(i), buf[0]);
      process(chunk(i), buf[0]);
    }
  } else {
    static_assert(NBUF == 2, "register chunks per wave: 1 or 2");
    int i0 = 0;
    if (n_w >= 3) {
      // Steady state with every load unconditional: the compiler's memory
      // counters then know which loads each buffer waits for.  (After a
      // load that may be skipped they must assume the fewest loads in
      // flight, and processing a chunk would wait for the chunk requested
      // after it too.)
      load(chunk(0), buf[0]);
      for (; i0 + 3 <= n_w; i0 += 2) {
        load(chunk(i0 + 1), buf[1]);
        process(chunk(i0), buf[0]);
        load(chunk(i0 + 2), buf[0]);
        process(chunk(i0 + 1), buf[1]);
      }
    } else if (n_w > 0) {
      load(chunk(0), buf[0]);
    }
    // fewer than three chunks left; chunk i0 is in flight
    if (i0 + 1 < n_w) load(chunk(i0 + 1), buf[1]);
    if (i0 < n_w) process(chunk(i0), buf[0]);
    if (i0 + 1 < n_w) process(chunk(i0 + 1), buf[1]);
  }

  // ---- merge the states of the waves of each row group (fixed order:
  // bitwise repeatable)
#pragma unroll
  for (int nt = 0; nt < 1; ++nt) {
    l_run[nt] += shfl_xor(l_run[nt], 16);
    l_run[nt] += shfl_xor(l_run[nt], 32);
    if constexpr (BIAS) {
      // remove the +128 of the int8 value codes: sum_j p'_j (c_j + 128) - 128 sum_j p'_j
      float s_ = pvsum[nt];
      s_ += shfl_xor(s_, 16);
      s_ += shfl_xor(s_, 32);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) acc[nt][dt] -= 128.f * s_;
    }
  }
  if constexpr (BAL) {
    // the wave's own state of its piece: lane (q4, l16) holds dims
    // 16 dt + 4 q4 + r of row l16
    if (l16 < rows) {
      const int tok = s0 + l16 / G, head = g * G + l16 % G;
      float M = m_run[0], Lt = l_run[0], e = 1.f;
      if (p.sinks && first) {
        // the sink joins the first piece as one more score with no value row
        const float s2 = p.sinks[head] * kLog2e;
        const float Mn = fmaxf(M, s2);
        const float Ms = Mn == kNegInf ? 0.f : Mn;
        e = fast_exp2(M - Ms);
        Lt = Lt * e + fast_exp2(s2 - Ms);
        M = Mn;
      }
      if (whole) {
        const float inv = Lt > 0.f ? e / Lt : 0.f;
        __bf16* op = (__bf16*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)head * p.o_stride_head + 4 * q4;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const f32x4 o = acc[0][dt];
          *(u32x2*)(op + 16 * dt) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
        }
      } else {
        // partial slot b + w: unique, since each piece adds one to b or to w
        const int64_t ri = ((int64_t)(b + bal_u) * p.ws_tok + l16 / G) * p.num_q_heads + head;
        float* wa = p.bal_acc + ri * D + 4 * q4;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) *(f32x4*)(wa + 16 * dt) = acc[0][dt] * e;
        if (q4 == 0) *(f32x2*)(p.bal_ml + ri * 2) = f32x2{M, Lt};
      }
    }
    continue;
  } else {
  __syncthreads();                              // staging tiles are free from here on
  float* Mw = (float*)smem;                     // [4 waves][16 rows of the wave's group]
  float* Lw = Mw + 64;                          // [4 waves][16]
  float* Ob = Lw + 64;                          // [ROWS][ORS]
  if (q4 == 0) Mw[wave * 16 + l16] = m_run[0];
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < KG; ++k) M = fmaxf(M, Mw[(rg + NG * k) * 16 + l16]);
    const float Ms = M == kNegInf ? 0.f : M;
    const float e = fast_exp2(m_run[0] - Ms);
    l_run[0] *= e;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[0][dt] *= e;
    if (q4 == 0) Lw[wave * 16 + l16] = l_run[0];
  }
#pragma unroll
  for (int k = 0; k < KG; ++k) {
    if (kg == k) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        f32x4* o = (f32x4*)(Ob + (16 * rg + l16) * ORS + 16 * dt + 4 * q4);
        *o = (k == 0) ? acc[0][dt] : (*o + acc[0][dt]);
      }
    }
    __syncthreads();
  }

  const int nrows = min(rows, ROWS);
  // workspace rows per split: (sequence, step token) slots, or flat tokens
  const int64_t NH = p.ws_flat ? (int64_t)p.num_tokens * p.num_q_heads : (int64_t)p.num_seqs * p.ws_tok * p.num_q_heads;
  for (int it = threadIdx.x; it < nrows * (D / 4); it += 256) {
    const int row = it / (D / 4), c4 = it % (D / 4);
    const int tok = s0 + row / G, head = g * G + row % G;
    // the row's group and the waves that computed it
    float M = kNegInf, Lt = 0.f;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int w = (row >> 4) + NG * k;
      M = fmaxf(M, Mw[w * 16 + (row & 15)]);
      Lt += Lw[w * 16 + (row & 15)];
    }
    f32x4 o = *(const f32x4*)(Ob + row * ORS + 4 * c4);
    if (p.sinks && first) {
      // the sink joins split 0 as one more score with no value row
      const float s2 = p.sinks[head] * kLog2e;
      const float Mn = fmaxf(M, s2);
      const float Ms = Mn == kNegInf ? 0.f : Mn;
      const float e = fast_exp2(M - Ms);
      Lt = Lt * e + fast_exp2(s2 - Ms);
      o *= e;
      M = Mn;
    }
    if (p.merge_prefix > 0) {
      // cascade with a one-split suffix: merge the prefix pass's partials of
      // this row (flat workspace rows) with the suffix state and normalise
      const int64_t NHf = (int64_t)p.num_tokens * p.num_q_heads;
      const int64_t rrow = (int64_t)tok * p.num_q_heads + head;
      // All of a row's partials (up to 16) are loaded before any is used:
      // one memory latency for the fold.  More partials are read in groups
      // of 8 whose loads are issued together, one latency per group and
      // pass.  Padding entries (-inf, 0) leave every sum unchanged, so both
      // forms add the same terms in the same order.
      const int np = p.merge_prefix;
      float Ltot;
      f32x4 ot;
      if (np <= 16) {
        f32x2 ml[16];
        f32x4 pa[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < np) {
            const int64_t ri = j * NHf + rrow;
            ml[j] = *(const f32x2*)(p.ws_ml + ri * 2);
            pa[j] = *(const f32x4*)(p.ws_acc + ri * D + 4 * c4);
          } else {
            ml[j] = f32x2{kNegInf, 0.f};
            pa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        float Mx = M;
#pragma unroll
        for (int j = 0; j < 16; ++j) Mx = fmaxf(Mx, ml[j][0]);
        const float Ms = Mx == kNegInf ? 0.f : Mx;
        const float e0 = fast_exp2(M - Ms);
        Ltot = Lt * e0;
        ot = o * e0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float w = fast_exp2(ml[j][0] - Ms);
          Ltot = fmaf(w, ml[j][1], Ltot);
          ot += w * pa[j];
        }
      } else {
        float Mx = M;
        for (int g0 = 0; g0 < np; g0 += 8) {
          float m[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) m[j] = g0 + j < np ? p.ws_ml[((g0 + j) * NHf + rrow) * 2] : kNegInf;
#pragma unroll
          for (int j = 0; j < 8; ++j) Mx = fmaxf(Mx, m[j]);
        }
        const float Ms = Mx == kNegInf ? 0.f : Mx;
        const float e0 = fast_exp2(M - Ms);
        Ltot = Lt * e0;
        ot = o * e0;
        for (int g0 = 0; g0 < np; g0 += 8) {
          f32x2 ml[8];
          f32x4 pa[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (g0 + j < np) {
              const int64_t ri = (g0 + j) * NHf + rrow;
              ml[j] = *(const f32x2*)(p.ws_ml + ri * 2);
              pa[j] = *(const f32x4*)(p.ws_acc + ri * D + 4 * c4);
            } else {
              ml[j] = f32x2{kNegInf, 0.f};
              pa[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float w = fast_exp2(ml[j][0] - Ms);
            Ltot = fmaf(w, ml[j][1], Ltot);
            ot += w * pa[j];
          }
        }
      }
      const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
      __bf16* op = (__bf16*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)head * p.o_stride_head + 4 * c4;
      *(u32x2*)op = u32x2{pack_bf16x2(ot[0] * inv, ot[1] * inv), pack_bf16x2(ot[2] * inv, ot[3] * inv)};
    } else if (whole) {
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
      __bf16* op = (__bf16*)p.out + (int64_t)tok * p.o_stride_tok + (int64_t)head * p.o_stride_head + 4 * c4;
      *(u32x2*)op = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    } else {
      const int64_t rrow = p.ws_flat ? (int64_t)tok * p.num_q_heads + head
                                     : ((int64_t)b * p.ws_tok + row / G) * p.num_q_heads + head;
      const int64_t ri = (int64_t)(p.split_base + split) * NH + rrow;
      *(f32x4*)(p.ws_acc + ri * D + 4 * c4) = o;
      if (c4 == 0) *(f32x2*)(p.ws_ml + ri * 2) = f32x2{M, Lt};
    }
  }
  }
  }
}

}  // namespace pa
