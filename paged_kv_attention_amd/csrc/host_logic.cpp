// Host-only planning for paged_attention (see host_logic.h).
#include "host_logic.h"
#include "pa_params.h"

#include <limits.h>

#include <vector>

namespace pa {

static bool one_of(int v, std::initializer_list<int> set) {
  for (int x : set)
    if (v == x) return true;
  return false;
}

pa_status check_dims(const pa_dims* d, pa_dtype dtype) {
  if (!d) return PA_ERR_NULL;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs < 0 || d->num_tokens < 0 || d->max_query_len < 0 || d->num_splits < 0) return PA_ERR_SHAPE;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (d->num_pages < 0 || d->table_width < 0) return PA_ERR_SHAPE;
  if (d->num_seqs > 0 && (d->num_pages < 1 || d->table_width < 1)) return PA_ERR_SHAPE;
  if (!one_of(d->head_dim, {64, 128, 256})) return PA_ERR_UNSUPPORTED;
  if (!one_of(d->page_size, {16, 32, 64, 128})) return PA_ERR_UNSUPPORTED;
  const int64_t D = d->head_dim;
  const int64_t s[] = {d->q_stride_tok, d->q_stride_head, d->o_stride_tok, d->o_stride_head,
                       d->kv_stride_page, d->kv_stride_slot, d->kv_stride_head};
  for (int64_t x : s)
    if (x < 0) return PA_ERR_SHAPE;
  // rows of one head must not overlap: D is contiguous
  if ((d->num_q_heads > 1 && (d->q_stride_head < D || d->o_stride_head < D)) ||
      (d->num_tokens > 1 && (d->q_stride_tok < D || d->o_stride_tok < D)) ||
      (d->num_kv_heads > 1 && d->kv_stride_head < D) || d->kv_stride_slot < D ||
      (d->num_pages > 1 && d->kv_stride_page < D))
    return PA_ERR_SHAPE;
  // 16-byte vector loads: every stride a whole number of 16-byte chunks
  const int64_t vec = dtype == PA_BF16 ? 8 : 4;
  for (int64_t x : s)
    if (x % vec) return PA_ERR_UNSUPPORTED;
  // the kernels address the 16 slots of a key tile with 32-bit byte offsets
  if (d->kv_stride_slot >= ((int64_t)1 << 26)) return PA_ERR_UNSUPPORTED;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (dtype == PA_BF16 && G > 64) return PA_ERR_UNSUPPORTED;
  // grid limits (y and z dimensions are 16-bit)
  if (d->num_seqs > 65535 || d->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if ((int64_t)d->table_width * d->page_size > INT_MAX / 2) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int choose_splits(const pa_dims* d, pa_dtype dtype, int cu_count) {
  return choose_splits_over(d, dtype, cu_count, d->table_width > 0 ? d->table_width : 1);
}

int choose_splits_over(const pa_dims* d, pa_dtype dtype, int cu_count, int W) {
  if (W < 1) W = 1;
  if (d->num_splits > 0) return d->num_splits < W ? d->num_splits : W;
  if (cu_count < 1) cu_count = 1;
  // units of parallel work per split: (sequence, KV head) workgroups of 4 waves
  // for the bf16 decode kernel; (sequence, KV head, 16-row tile) workgroups of
  // 4-16 waves for float32, which spread a split's keys over all their waves.
  const int N = d->num_tokens;
  const int mql = d->max_query_len > 0 && d->max_query_len < N ? d->max_query_len : N;
  const int G = d->num_q_heads / d->num_kv_heads;
  int64_t units = dtype == PA_BF16 ? (int64_t)d->num_seqs * d->num_kv_heads
                                   : (int64_t)d->num_seqs * d->num_kv_heads * f32_row_tiles(mql, G);
  int64_t target = dtype == PA_BF16 ? 2 * (int64_t)cu_count : (int64_t)cu_count;
  if (units < 1) units = 1;
  int64_t want = (target + units - 1) / units;
  // A step of one-token decodes that cannot fill two workgroups per CU aims
  // at three: it runs alone (no other tile class beside it), and more, shorter
  // splits shorten the longest sequence's tail.  Mixed batches measured
  // faster with two.
  if (dtype == PA_BF16 && mql == 1 && units < target) want = (3 * (int64_t)cu_count + units - 1) / units;
  // at least 128 keys per bf16 split (one 32-key chunk per wave of a 4-wave
  // workgroup) and 64 per float32 split (four 16-key chunks: the 600-key
  // single-sequence decode measured 15.2 us as one split and 10.4-10.6 us
  // with 10 to 38 splits and the combine); at most 64 splits, so one
  // sequence with 8 KV heads still reaches two workgroups per CU
  const int min_keys = dtype == PA_BF16 ? 128 : 64;
  const int min_pages = (min_keys + d->page_size - 1) / d->page_size;
  const int64_t cap_pages = (W + min_pages - 1) / min_pages;
  int64_t s = want;
  if (s > 64) s = 64;
  if (s > cap_pages) s = cap_pages;
  if (s < 1) s = 1;
  return (int)s;
}

int window_pages(int window, int mql, int page_size, int W) {
  if (window <= 0) return W;
  // keys a sequence's step can see: from its first token's window start to
  // its last token, at most window + mql - 1 of them, over at most two more
  // pages than they fill
  const int64_t span = ((int64_t)window + (mql > 0 ? mql : 1) - 1) / page_size + 2;
  return span < W ? (int)span : W;
}

Plan make_plan(const pa_dims* d, pa_dtype dtype, int cu_count, int window) {
  Plan pl{};
  const int N = d->num_tokens;
  const int G = d->num_q_heads / d->num_kv_heads;
  pl.mql = d->max_query_len > 0 && d->max_query_len < N ? d->max_query_len : N;
  // with a sliding window the splits cut the window's pages, not the table
  const int W = window_pages(window, pl.mql, d->page_size, d->table_width > 0 ? d->table_width : 1);
  pl.window = window > 0 ? window : 0;
  int S = choose_splits_over(d, dtype, cu_count, W);
  pl.pages_per_split = (W + S - 1) / S;
  pl.splits = (W + pl.pages_per_split - 1) / pl.pages_per_split;
  if (dtype == PA_BF16) {
    int dm = 64 / G;
    pl.dec_max_n = dm < 16 ? dm : 16;
    const int dmax = pl.mql < pl.dec_max_n ? pl.mql : pl.dec_max_n;
    // fewest tokens any sequence can have: the others hold at most mql each
    // (a batch of equal prefill chunks has no decode-class sequence at all)
    int64_t nmin = (int64_t)N - (int64_t)(d->num_seqs - 1) * pl.mql;
    if (nmin < 1) nmin = 1;
    pl.dec_small = dmax >= 1 && G <= 16 && nmin * G <= 16;
    pl.dec_big = dmax * G > 16 && nmin <= dmax;
    pl.big_nt = dmax * G <= 32 ? 2 : 4;
    pl.prefill = pl.mql > pl.dec_max_n;
    pl.tok_per_tile = prefill_tile_rows(d->head_dim) / G;
    pl.num_qtiles = pl.prefill ? (pl.mql + pl.tok_per_tile - 1) / pl.tok_per_tile : 0;
    // The verify-tile launch (16 < n*G <= 64 rows): about two workgroups per
    // CU over the batch's (sequence, KV head) pairs, at least 256 keys per
    // split, at most 64 splits (page "Attention kernels", Decode: verify
    // steps of one sequence take several splits).
    if (d->num_splits > 0) {
      pl.splits_big = pl.splits;
      pl.pages_per_split_big = pl.pages_per_split;
    } else {
      const int64_t units = (int64_t)(d->num_seqs > 0 ? d->num_seqs : 1) * d->num_kv_heads;
      int64_t want = (2 * (int64_t)(cu_count > 0 ? cu_count : 1) + units - 1) / units;
      const int min_pages = (256 + d->page_size - 1) / d->page_size;
      const int64_t cap_pages = (W + min_pages - 1) / min_pages;
      // Beside prefill or 16-row decode tiles the verification steps are
      // likely few, and their key loops run while the other tiles hold the
      // chip: at least 16 splits keep those loops short (the mixed batch as
      // one launch: 4, 8, 16, 32 splits measured 138, 124, 119, 120 us).
      if ((pl.prefill || pl.dec_small) && want < 16) want = 16;
      if (want > 64) want = 64;
      if (want > cap_pages) want = cap_pages;
      if (want < 1) want = 1;
      pl.pages_per_split_big = (int)((W + want - 1) / want);
      pl.splits_big = (W + pl.pages_per_split_big - 1) / pl.pages_per_split_big;
    }
    if (!pl.dec_big) pl.splits_big = 1;
    // Balanced 16-row tiles: where the split launch would cut several
    // sequences into splits of 2048 keys or more (more than one split: the
    // batch's (sequence, KV head) pairs cannot fill two workgroups per CU),
    // a fixed grid of about two workgroups per CU shares the batch's 32-key
    // chunks equally among its waves instead: the longest splits of a ragged
    // batch no longer finish alone.  Shorter splits measured as fast as the
    // balanced launch with its extra partials (a ragged batch of 32 at up to
    // 4096 positions) or faster (one sequence).  An explicit split count
    // keeps the split launch.
    // (the chunk counts stay far inside int)
    const int64_t max_chunks = (int64_t)d->num_seqs * ((int64_t)W * d->page_size / 32 + 1);
    if (pl.dec_small && pl.splits > 1 && d->num_splits == 0 && d->num_seqs >= 2 &&
        d->num_seqs <= bal_max_seqs() && (int64_t)pl.pages_per_split * d->page_size >= 2048 &&
        max_chunks < ((int64_t)1 << 30)) {
      const int cu = cu_count > 0 ? cu_count : 1;
      pl.bal_wgs = (2 * cu + d->num_kv_heads - 1) / d->num_kv_heads;
      pl.bal_min_chunks = 4;
    }
    pl.combine = dmax >= 1 && ((pl.dec_small && pl.splits > 1) || (pl.dec_big && pl.splits_big > 1));
    pl.comb_tokens = dmax;
    pl.comb_max_n = pl.dec_max_n;
    pl.ws_tok = dmax;
  } else {
    pl.dec_max_n = 0;
    pl.num_qtiles = f32_row_tiles(pl.mql, G);
    pl.splits_big = pl.splits;
    pl.pages_per_split_big = pl.pages_per_split;
    pl.combine = pl.splits > 1 && pl.mql >= 1;
    pl.comb_tokens = pl.mql;
    pl.comb_max_n = INT_MAX;
    pl.ws_tok = pl.mql;
  }
  // split slots of the classes that run split launches
  pl.ws_splits = pl.bal_wgs > 0 ? pl.splits_big : (pl.splits > pl.splits_big ? pl.splits : pl.splits_big);
  // split partials are indexed by (sequence, token of the step) over the
  // split classes only, so prefill tokens take no workspace
  size_t bytes = 0;
  if (pl.ws_splits > 1 && pl.combine)
    bytes = (size_t)pl.ws_splits * (size_t)d->num_seqs * (size_t)pl.ws_tok * (size_t)d->num_q_heads *
            ((size_t)d->head_dim + 2) * 4;
  if (pl.bal_wgs > 0) {
    // balanced partials: slots b + w < B + 4 bal_wgs (w: the wave) of
    // ws_tok * Hq rows, then two ints per sequence for the combine
    bytes = (bytes + 255) & ~(size_t)255;
    pl.bal_offset = bytes;
    const size_t rows = (size_t)(d->num_seqs + 4 * pl.bal_wgs) * (size_t)pl.ws_tok * (size_t)d->num_q_heads;
    bytes += rows * ((size_t)d->head_dim + 2) * 4 + (size_t)d->num_seqs * 8;
  }
  pl.workspace_bytes = bytes;
  return pl;
}

CascadePlan make_cascade_plan(const pa_dims* d, pa_dtype dtype, int cu_count, int prefix_len, int window) {
  CascadePlan c{};
  c.status = PA_OK;
  const int ps = d->page_size, W = d->table_width, N = d->num_tokens;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (prefix_len < 0 || prefix_len % ps != 0 || (int64_t)prefix_len > (int64_t)W * ps) {
    c.status = PA_ERR_SHAPE;
    return c;
  }
  const int mql = d->max_query_len > 0 && d->max_query_len < N ? d->max_query_len : N;
  const int dm = 64 / G < 16 ? 64 / G : 16;
  // the prefix pass runs on the bf16 MFMA tiles and serves decode and
  // verification steps; a window would need per-row masks inside the prefix
  if (dtype != PA_BF16 || window > 0 || mql > dm) {
    c.status = PA_ERR_UNSUPPORTED;
    return c;
  }
  if (cu_count < 1) cu_count = 1;
  // 128- and 256-dim heads: tiles of 64 rows (4 waves of 16), otherwise
  // the prefill tile
  const bool t16 = d->head_dim == 128 || d->head_dim == 256;
  const int tpt = t16 ? 64 / G : prefill_tile_rows(d->head_dim) / G;
  c.prefix_tile_tokens = tpt;
  c.prefix_qtiles = (N + tpt - 1) / tpt;
  const int kb = prefill_block_keys();
  const int blocks = (prefix_len + kb - 1) / kb;
  // key ranges: about one 64-row tile per CU (half the CUs for the 256-row
  // tiles); more ranges add more partial-state traffic than they save
  const int64_t units = (int64_t)c.prefix_qtiles * d->num_kv_heads;
  const int64_t target = t16 ? (int64_t)cu_count : (int64_t)cu_count / 2;
  int64_t s = (target + units - 1) / units;
  if (s > blocks) s = blocks;
  if (s < 1) s = 1;
  const int per = (int)((blocks + s - 1) / s);
  c.prefix_split_keys = per * kb;
  c.prefix_splits = blocks > 0 ? (blocks + per - 1) / per : 0;
  pa_dims suf = *d;
  suf.table_width = W - prefix_len / ps > 0 ? W - prefix_len / ps : 1;
  const int S = choose_splits(&suf, PA_BF16, cu_count);
  c.suffix_pages_per_split = (suf.table_width + S - 1) / S;
  c.suffix_splits = (suf.table_width + c.suffix_pages_per_split - 1) / c.suffix_pages_per_split;
  c.workspace_bytes = (size_t)(c.prefix_splits + c.suffix_splits) * (size_t)N * (size_t)d->num_q_heads *
                      ((size_t)d->head_dim + 2) * 4;
  return c;
}

bool prefill_small_tiles(const pa_dims* d, int cu_count) {
  if (d->head_dim != 128 || d->num_kv_heads < 1) return false;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G < 1 || G > 64) return false;             // a 64-row tile holds at least one token
  const int64_t rows = (int64_t)d->num_tokens * G;
  const int64_t tiles = (rows + prefill_tile_rows(128) - 1) / prefill_tile_rows(128) * d->num_kv_heads;
  return 2 * tiles < (int64_t)cu_count;
}

int prefill_small_slots(int num_tokens, int num_seqs, int mql, int tpt, int dec_max_n) {
  if (num_tokens <= 0 || num_seqs <= 0 || tpt < 1) return 1;
  int64_t nseq = (int64_t)num_tokens / ((int64_t)dec_max_n + 1);
  if (nseq > num_seqs) nseq = num_seqs;
  if (nseq < 1) nseq = 1;
  const int64_t per_seq = ((int64_t)(mql > 0 ? mql : num_tokens) + tpt - 1) / tpt;
  int64_t slots = ((int64_t)num_tokens + tpt - 1) / tpt + nseq;
  if (slots > per_seq * nseq) slots = per_seq * nseq;
  if (slots < 1) slots = 1;
  return slots > INT_MAX / 2 ? INT_MAX / 2 : (int)slots;
}

pa_status validate_shared_prefix(const int32_t* bt, const int32_t* lens, const int32_t* qsl, int prefix_len,
                                 const pa_dims* d) {
  if (prefix_len <= 0) return PA_OK;
  const int B = d->num_seqs, W = d->table_width, ps = d->page_size;
  if (prefix_len % ps != 0 || (int64_t)prefix_len > (int64_t)W * ps) return PA_ERR_INVALID_DATA;
  const int npg = prefix_len / ps;
  for (int b = 0; b < B; ++b) {
    const int n = qsl[b + 1] - qsl[b];
    if (lens[b] - n < prefix_len) return PA_ERR_INVALID_DATA;
    for (int j = 0; j < npg; ++j)
      if (bt[(int64_t)b * W + j] != bt[j]) return PA_ERR_INVALID_DATA;
  }
  return PA_OK;
}

pa_status validate_host(const int32_t* bt, const int32_t* lens, const int32_t* qsl, const int32_t* slots,
                        int32_t num_slots, int causal, const pa_dims* d) {
  const int B = d->num_seqs, W = d->table_width, ps = d->page_size, P = d->num_pages;
  if (B > 0 && qsl[0] != 0) return PA_ERR_INVALID_DATA;
  for (int b = 0; b < B; ++b) {
    const int n = qsl[b + 1] - qsl[b];
    if (n < 0) return PA_ERR_INVALID_DATA;
    if (d->max_query_len > 0 && n > d->max_query_len) return PA_ERR_INVALID_DATA;
    const int L = lens[b];
    if (L < 0 || (int64_t)L > (int64_t)W * ps) return PA_ERR_INVALID_DATA;
    if (causal && n > L) return PA_ERR_INVALID_DATA;
    const int npg = (L + ps - 1) / ps;
    for (int j = 0; j < npg; ++j) {
      const int pg = bt[(int64_t)b * W + j];
      if (pg < 0 || pg >= P) return PA_ERR_INVALID_DATA;
    }
  }
  if (B > 0 && qsl[B] != d->num_tokens) return PA_ERR_INVALID_DATA;
  if (slots && num_slots > 0) {
    const int64_t cap = (int64_t)P * ps;
    std::vector<unsigned char> seen((size_t)cap, 0);
    for (int i = 0; i < num_slots; ++i) {
      const int s = slots[i];
      if (s == -1) continue;
      if (s < 0 || s >= cap) return PA_ERR_INVALID_DATA;
      if (seen[(size_t)s]) return PA_ERR_INVALID_DATA;
      seen[(size_t)s] = 1;
    }
  }
  return PA_OK;
}

}  // namespace pa
