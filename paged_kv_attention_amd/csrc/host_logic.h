// Host-only planning for paged_attention: argument checks, the split count
// and which kernels a call launches.  Plain C++ (no HIP), so it also builds
// with g++ for host unit tests.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

struct Plan {
  int mql;                 // effective max_query_len
  int splits;              // S after sizing (>= 1); bf16: the 16-row decode tile's launch
  int pages_per_split;     // ceil(W / S)
  int splits_big;          // bf16: splits of the 32/64-row (verify) tile's launch
  int pages_per_split_big;
  int dec_max_n;           // bf16: sequences with n <= dec_max_n use the decode kernel
  bool dec_small;          // bf16: decode launch for n*G <= 16 (16-row tile)
  bool dec_big;            // bf16: decode launch for 16 < n*G <= 16*big_nt
  int big_nt;              // 2 or 4 row tiles
  bool prefill;            // bf16: prefill launch for n > dec_max_n
  int tok_per_tile;        // prefill: tokens per tile (tile rows / G)
  int num_qtiles;          // prefill: tiles per sequence (from mql); float32: 16-row tiles
  bool combine;            // split partials need the combine launch
  int comb_tokens;         // combine: token slots per sequence
  int comb_max_n;          // combine: sequences with n <= comb_max_n
  int ws_tok;              // workspace row slots per sequence
  int ws_splits;           // split slots of the split launches' partials (1: none)
  int bal_wgs;             // bf16 16-row tiles: balanced launch, workgroups per KV head (0: split launch)
  int bal_min_chunks;      // fewest 32-key chunks a balanced workgroup takes
  size_t bal_offset;       // workspace bytes before the balanced launch's partials
  size_t workspace_bytes;  // bytes the call needs
  int window;              // sliding window (0 = none): splits cut the window's pages
};

// Checks dims and dtype; PA_OK or the error status (nothing else is touched).
pa_status check_dims(const pa_dims* d, pa_dtype dtype);

// Split count from host scalars only: bf16 aims at about two workgroups per
// CU with at least 128 keys per split, float32 at one workgroup per CU with
// at least 64 keys per split; at most 64 splits; an explicit
// dims->num_splits > 0 wins (capped at W).
int choose_splits(const pa_dims* d, pa_dtype dtype, int cu_count);
// The same rule over W pages instead of the table width.
int choose_splits_over(const pa_dims* d, pa_dtype dtype, int cu_count, int W);

// Pages a split range must cover: the table width W, or with a sliding window
// (window > 0) the pages from a step's first window start to its end.
int window_pages(int window, int mql, int page_size, int W);

// Full launch plan for valid dims (call check_dims first).  With window > 0
// the splits cut window_pages() pages starting at the page of the first
// token's window start (the kernels find that page from the device lengths).
Plan make_plan(const pa_dims* d, pa_dtype dtype, int cu_count, int window = 0);

// Cascade plan (a prefix of prefix_len positions shared by every sequence):
// the prefix pass cuts the prefix into prefix_splits key ranges of
// prefix_split_keys (a multiple of the prefill block) over prefix_qtiles tiles
// of the flat token range; the suffix pass splits the remaining table pages
// as a decode call would.  status is PA_OK or why the cascade cannot run.
struct CascadePlan {
  pa_status status;
  int prefix_splits, prefix_split_keys, prefix_qtiles;
  int prefix_tile_tokens;  // query tokens per prefix tile
  int suffix_splits, suffix_pages_per_split;
  size_t workspace_bytes;  // (prefix_splits + suffix_splits) * N * Hq * (D + 2) * 4
};
CascadePlan make_cascade_plan(const pa_dims* d, pa_dtype dtype, int cu_count, int prefix_len, int window);

// Whether a batch's prefill tiles run as 64-row tiles (bf16 pools, 128-dim
// heads): when even the bound N*G on its prefill rows fills fewer 256-row
// tiles than half the CUs, the smaller tiles spread the work over the chip.
bool prefill_small_tiles(const pa_dims* d, int cu_count);

// Tile slots per KV head of the compact grid of 64-row prefill tiles
// (tpt tokens each): a bound from host scalars on the batch's prefill tiles.
// A prefill sequence has more than dec_max_n tokens, so there are at most
// min(B, N / (dec_max_n + 1)) of them, and their tiles number at most
// ceil(N / tpt) plus one per sequence, and at most ceil(mql / tpt) each.
int prefill_small_slots(int num_tokens, int num_seqs, int mql, int tpt, int dec_max_n);

// Shared-prefix contract on copied metadata: table rows agree with row 0 on
// the prefix's pages and every query token sits after the prefix.
pa_status validate_shared_prefix(const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start_loc, int prefix_len, const pa_dims* d);

// Host-side check of copied metadata (the body of pa_validate).
pa_status validate_host(const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                        const int32_t* slot_mapping, int32_t num_slots, int causal, const pa_dims* d);

}  // namespace pa
