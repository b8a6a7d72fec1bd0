// Kernel argument blocks.  Each kernel takes one of these by value, so a
// launch carries a single packed argument however many sizes and strides it
// needs (page "cuTile design choices", Keep launches under 32 kernel
// parameters: wide argument lists made every launch slow there).
#pragma once

#include <stdint.h>

namespace pa {

// Query rows per prefill workgroup tile (32 per wave): 8 waves for head_dim
// <= 128, 4 waves for 256 (its accumulator does not fit two waves per SIMD).
constexpr int prefill_tile_rows(int head_dim) { return head_dim <= 128 ? 256 : 128; }
// Keys per K/V block of the prefill kernel (also the granule of the
// cascade's prefix key ranges).
constexpr int prefill_block_keys() { return 64; }
// Float32 kernel: 16-row tiles (step tokens x group heads) per sequence.
constexpr int f32_row_tiles(int max_query_len, int group) {
  return max_query_len > 0 ? (max_query_len * group + 15) / 16 : 1;
}

struct AttnParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  void* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  float* ws_acc;            // [S][B*ws_tok*Hq][D] float32 split accumulators
  float* ws_ml;             // [S][B*ws_tok*Hq][2] float32 (running max in log2 units, sum)
  int32_t ws_tok;           // workspace row slots per sequence (tokens of the split classes)
  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t kv_stride_page, kv_stride_slot, kv_stride_head;
  float scale_log2;         // scale * log2(e): scores go straight into exp2
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, group;
  int32_t head_dim, page_size, page_shift, num_pages, table_width;
  int32_t num_splits;       // S (>= 1)
  int32_t pages_per_split;  // ceil(W / S)
  int32_t causal;
  int32_t dec_max_n;        // sequences with n <= dec_max_n are the decode class
  int32_t row_lo, row_hi;   // decode kernel: takes sequences with row_lo < n*G <= row_hi
  int32_t tok_per_tile;     // prefill: query tokens per tile
  int32_t num_qtiles;       // prefill: tiles per (sequence, KV head); float32: 16-row tiles per sequence
  int32_t comb_max_n;       // combine: sequences with n <= comb_max_n
  int32_t comb_tokens;      // combine: token slots per sequence in the grid
  int32_t comb_splits_small;  // combine: splits of rows with n*G <= 16 (1 = written by the decode kernel)
  int32_t comb_splits_big;    // combine: splits of rows with n*G > 16
  int32_t window;           // sliding window: key j visible to position pos only if j > pos - window (0 = none)
  const float* sinks;       // [Hq] sink logits in scaled-score units, or null
  // quantized pools (kv_code != 0): 1-byte codes, one float32 scale per
  // (page, slot, KV head) and optional per-channel key smoothing [Hkv, D]
  int32_t kv_code;          // 0 = pools in the q dtype, 1 = int8, 2 = fp8 E4M3
  const float* k_scale;
  const float* v_scale;
  int64_t sc_stride_page, sc_stride_slot, sc_stride_head;
  const float* k_smooth;
  // cascade (a prefix shared by every sequence of the batch):
  int32_t key_lo;           // decode: keys below key_lo are left to the prefix pass (0 = none)
  int32_t split_base;       // decode: its partials take split slots split_base + split
  int32_t force_partial;    // decode: write partials even with one split
  int32_t ws_flat;          // workspace rows indexed by flat token (N * Hq per split)
  int32_t prefix_len;       // prefix pass: keys [0, prefix_len) of block-table row 0
  int32_t prefix_splits;    // prefix pass: key ranges, each prefix_split_keys long
  int32_t prefix_split_keys;
  int32_t merge_prefix;     // decode with one split: fold this many prefix partials (slots 0..) into
                            // the output instead of writing a partial
  int32_t head_first;       // 16-row decode tiles: grid (KV head, sequence, split) instead of
                            // (split, KV head, sequence)
  // 16-row decode tiles, bf16 pools: the step's new K/V rows, written by the
  // workgroup whose pages hold each token's position before it attends
  // (NULL = none); element strides of the [N, Hkv, D] rows
  const void* new_k;
  const void* new_v;
  const int32_t* new_slots;
  int64_t new_stride_tok, new_stride_head;
  // balanced 16-row decode tiles (bal_wgs > 0): a grid of (KV head,
  // bal_wgs) workgroups; wave w = 4 u + (wave index) takes chunks
  // [w R, (w + 1) R) of the batch's 32-key chunks laid end to end (R =
  // max(bal_min_chunks, ceil(total / (4 bal_wgs)))); its piece of sequence
  // b keeps partial slot b + w
  int32_t bal_wgs, bal_min_chunks;
  float* bal_acc;           // [(B + 4 bal_wgs) * ws_tok * Hq][D] float32
  float* bal_ml;            // [(B + 4 bal_wgs) * ws_tok * Hq][2] float32
  int32_t* bal_meta;        // [B][2]: first partial slot of sequence b, slots (0 or 1: no combine)
};

// Most sequences a balanced decode launch takes (its prefix sums live in LDS).
constexpr int bal_max_seqs() { return 512; }

// First page of the split ranges of a sequence with context L and n step
// tokens: the page of its first token's window start (0 without a window).
constexpr int split_page_base(int L, int n, int window, int page_size) {
  if (window <= 0) return 0;
  const int lo = L - n - window + 1;
  return lo > 0 ? lo / page_size : 0;
}

struct KvWriteParams {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* slot_mapping;
  int64_t new_stride_tok, new_stride_head;
  int64_t kv_stride_page, kv_stride_slot, kv_stride_head;
  int32_t num_tokens, num_kv_heads, head_dim, page_size, num_pages;
  int32_t elem_bytes;       // bytes per element of the new rows
  // quantizing write (kv_code != 0): pools hold 1-byte codes
  int32_t kv_code;
  float* k_scale;
  float* v_scale;
  int64_t sc_stride_page, sc_stride_slot, sc_stride_head;
  const float* k_smooth;
};

}  // namespace pa
