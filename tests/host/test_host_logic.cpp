// Host unit test of the planning and validation code (built with g++ and
// AddressSanitizer by tests/test_host_logic.py; no GPU involved).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "host_logic.h"
#include "pa_params.h"

static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static pa_dims dims(int B, int N, int mql, int Hq, int Hkv, int D, int ps, int P, int W) {
  pa_dims d{};
  d.num_seqs = B; d.num_tokens = N; d.max_query_len = mql; d.num_q_heads = Hq; d.num_kv_heads = Hkv;
  d.head_dim = D; d.page_size = ps; d.num_pages = P; d.table_width = W;
  d.q_stride_tok = (int64_t)Hq * D; d.q_stride_head = D; d.o_stride_tok = (int64_t)Hq * D; d.o_stride_head = D;
  d.kv_stride_page = (int64_t)ps * Hkv * D; d.kv_stride_slot = (int64_t)Hkv * D; d.kv_stride_head = D;
  return d;
}

int main() {
  // decode 64 x 4096: one split fills 256 CUs twice over
  pa_dims c3 = dims(64, 64, 1, 32, 8, 128, 64, 4096, 64);
  CHECK(pa::check_dims(&c3, PA_BF16) == PA_OK);
  pa::Plan p3 = pa::make_plan(&c3, PA_BF16, 256);
  CHECK(p3.splits == 1 && p3.workspace_bytes == 0 && p3.dec_small && !p3.dec_big && !p3.prefill && !p3.combine);
  // ragged 32 one-token decodes: 256 (sequence, KV head) pairs do not fill
  // two workgroups per CU, so three splits; workspace for every row
  pa_dims c2 = dims(32, 32, 1, 32, 8, 128, 64, 2000, 64);
  pa::Plan p2 = pa::make_plan(&c2, PA_BF16, 256);
  CHECK(p2.splits == 3 && p2.pages_per_split == 22 && p2.combine && p2.comb_tokens == 1);
  // splits of 1408 keys: the split launch
  CHECK(p2.bal_wgs == 0 && p2.ws_splits == 3);
  CHECK(p2.workspace_bytes == (size_t)3 * 32 * 32 * 130 * 4);
  // the same batch over a table of 16384 positions cuts splits of 5504 keys:
  // the balanced launch, whose 256 waves of 64 workgroups per KV head share
  // the batch's chunks; partial slots b + w < 32 + 256 of 32 rows, and two
  // ints per sequence for the combine
  pa_dims c2l = dims(32, 32, 1, 32, 8, 128, 64, 8192, 256);
  pa::Plan p2l = pa::make_plan(&c2l, PA_BF16, 256);
  CHECK(p2l.splits == 3 && p2l.bal_wgs == 64 && p2l.bal_min_chunks == 4 && p2l.ws_splits == 1 && p2l.bal_offset == 0);
  CHECK(p2l.workspace_bytes == (size_t)(32 + 256) * 32 * 130 * 4 + 32 * 8);
  // one sequence keeps the split launch
  pa_dims c1l = dims(1, 1, 1, 32, 8, 128, 64, 512, 512);
  CHECK(pa::make_plan(&c1l, PA_BF16, 256).bal_wgs == 0);
  // an explicit split count keeps the split launch
  pa_dims c2s = c2;
  c2s.num_splits = 3;
  pa::Plan p2s = pa::make_plan(&c2s, PA_BF16, 256);
  CHECK(p2s.bal_wgs == 0 && p2s.ws_splits == 3 && p2s.workspace_bytes == (size_t)3 * 32 * 32 * 130 * 4);
  // more sequences than a balanced launch takes (a chip of 1024 CUs would
  // still split them): split launch
  pa_dims c2b = dims(513, 513, 1, 32, 1, 128, 64, 2000, 256);
  pa::Plan p2b = pa::make_plan(&c2b, PA_BF16, 1024);
  CHECK(p2b.splits > 1 && p2b.bal_wgs == 0);
  // the float32 path never balances
  CHECK(pa::make_plan(&c2l, PA_F32, 256).bal_wgs == 0);
  // the same sequences with 2-token steps aim at two workgroups per CU
  pa_dims c2v = dims(32, 64, 2, 32, 8, 128, 64, 2000, 64);
  CHECK(pa::make_plan(&c2v, PA_BF16, 256).splits == 2);
  // sliding window: the splits cut the window's pages, never more than the table's
  CHECK(pa::window_pages(0, 1, 64, 64) == 64);
  CHECK(pa::window_pages(1024, 1, 64, 64) == 18);          // 1024 keys over at most 18 pages
  CHECK(pa::window_pages(100000, 1, 64, 64) == 64);
  CHECK(pa::window_pages(1, 16, 16, 64) == 3);          // 16 keys straddle at most 2 pages; one spare
  pa::Plan pw = pa::make_plan(&c2, PA_BF16, 256, 1024);
  CHECK(pw.window == 1024 && pw.splits == 3 && pw.pages_per_split == 6);
  CHECK(pw.workspace_bytes <= p2.workspace_bytes);
  // split ranges start at the page of the first token's window start
  CHECK(pa::split_page_base(4096, 1, 1024, 64) == 48 && pa::split_page_base(4096, 1, 0, 64) == 0);
  CHECK(pa::split_page_base(100, 1, 1024, 64) == 0 && pa::split_page_base(1025, 1, 1024, 64) == 0);
  CHECK(pa::split_page_base(1089, 1, 1024, 64) == 1);
  // cascade: 64 decodes over a 4096-position shared prefix, suffixes up to 8 pages
  pa_dims cc = dims(64, 64, 1, 32, 8, 128, 64, 362, 72);
  pa::CascadePlan cpl = pa::make_cascade_plan(&cc, PA_BF16, 256, 4096, 0);
  // 64-row prefix tiles: 16 tokens of 4 heads, 4 tiles x 8 KV heads, 8 key ranges (one tile per CU)
  CHECK(cpl.status == PA_OK && cpl.prefix_tile_tokens == 16 && cpl.prefix_qtiles == 4 && cpl.prefix_splits == 8 &&
        cpl.prefix_split_keys == 512);
  CHECK(cpl.suffix_splits == 1 && cpl.suffix_pages_per_split == 8);
  CHECK(cpl.workspace_bytes == (size_t)9 * 64 * 32 * 130 * 4);
  // short prefills (their N*G rows fill fewer 256-row tiles than half the CUs) take 64-row tiles
  pa_dims mx = dims(32, 547, 512, 32, 8, 128, 64, 4096, 128);
  CHECK(pa::prefill_small_tiles(&mx, 256));                                   // 9 x 8 = 72 tiles < 128
  pa_dims pf = dims(4, 32768, 8192, 32, 8, 128, 64, 4096, 128);
  CHECK(!pa::prefill_small_tiles(&pf, 256));
  pa_dims m256 = dims(32, 547, 512, 16, 4, 256, 64, 4096, 128);
  CHECK(!pa::prefill_small_tiles(&m256, 256));                                // 128-dim heads only
  // compact grid of 64-row prefill tiles (16 tokens at group 4): the mixed
  // batch's 547 tokens over 32 sequences (at most 32 prefill sequences of
  // more than 16 tokens) give ceil(547 / 16) + 32 = 67 slots per KV head;
  // one 8192-token prompt 512 + 1; a bound never above B * ceil(mql / 16)
  CHECK(pa::prefill_small_slots(547, 32, 512, 16, 16) == 67);
  CHECK(pa::prefill_small_slots(8192, 1, 8192, 16, 16) == 512);
  CHECK(pa::prefill_small_slots(40, 2, 20, 16, 16) == 4);        // two 20-token steps: 2 tiles each
  CHECK(pa::prefill_small_slots(17, 1, 17, 16, 16) == 2);
  CHECK(pa::prefill_small_slots(0, 4, 8, 16, 16) == 1);
  pa_dims p2k = dims(1, 2048, 2048, 32, 8, 128, 64, 64, 64);
  CHECK(!pa::prefill_small_tiles(&p2k, 256));                                 // 32 x 8 = 256 tiles
  // 64-dim heads keep the 256-row prefill tiles, about half the CUs busy
  pa_dims c64 = dims(64, 64, 1, 32, 8, 64, 64, 362, 72);
  pa::CascadePlan cp64 = pa::make_cascade_plan(&c64, PA_BF16, 256, 4096, 0);
  CHECK(cp64.status == PA_OK && cp64.prefix_tile_tokens == 64 && cp64.prefix_qtiles == 1 && cp64.prefix_splits == 16);
  CHECK(pa::make_cascade_plan(&cc, PA_BF16, 256, 4000, 0).status == PA_ERR_SHAPE);       // not whole pages
  CHECK(pa::make_cascade_plan(&cc, PA_BF16, 256, 4096, 512).status == PA_ERR_UNSUPPORTED);   // with a window
  CHECK(pa::make_cascade_plan(&cc, PA_F32, 256, 4096, 0).status == PA_ERR_UNSUPPORTED);
  pa_dims cpf = dims(2, 100, 50, 32, 8, 128, 64, 362, 72);                              // prefill-class steps
  CHECK(pa::make_cascade_plan(&cpf, PA_BF16, 256, 4096, 0).status == PA_ERR_UNSUPPORTED);
  {
    // contract: rows share the prefix pages and every token sits after the prefix
    const int32_t bt[6] = {5, 6, 1, 5, 6, 2}, lens[2] = {9, 10}, qsl[3] = {0, 1, 3};
    pa_dims dv = dims(2, 3, 2, 4, 2, 64, 4, 8, 3);
    CHECK(pa::validate_shared_prefix(bt, lens, qsl, 8, &dv) == PA_OK);
    const int32_t bt2[6] = {5, 6, 1, 5, 7, 2};
    CHECK(pa::validate_shared_prefix(bt2, lens, qsl, 8, &dv) == PA_ERR_INVALID_DATA);
    const int32_t lens2[2] = {9, 9};                                                     // token inside the prefix
    CHECK(pa::validate_shared_prefix(bt, lens2, qsl, 8, &dv) == PA_ERR_INVALID_DATA);
  }
  // mixed batch: prefill + small and large decode tiles
  pa_dims c4 = dims(32, 547, 512, 32, 8, 128, 64, 2000, 128);
  pa::Plan p4 = pa::make_plan(&c4, PA_BF16, 256);
  CHECK(p4.prefill && p4.tok_per_tile == 64 && p4.num_qtiles == 8 && p4.dec_small && p4.dec_big && p4.big_nt == 4);
  CHECK(p4.dec_max_n == 16 && p4.comb_max_n == 16);
  // the verify-tile launch would aim at two workgroups per CU over the 32 x 8
  // (sequence, KV head) pairs (2 splits), but beside the prefill and 16-row
  // decode tiles it takes at least 16 (8 pages each); partials only for the
  // 16 decode-class token slots
  CHECK(p4.splits == 2 && p4.splits_big == 16 && p4.pages_per_split_big == 8 && p4.ws_tok == 16);
  // the 16-row tiles run balanced: their partials follow the verify tiles'
  const size_t w4 = (size_t)16 * 32 * 16 * 32 * 130 * 4;
  CHECK(p4.bal_wgs == 64 && p4.ws_splits == 16 && p4.bal_offset == w4);
  CHECK(p4.workspace_bytes == w4 + (size_t)(32 + 256) * 16 * 32 * 130 * 4 + 32 * 8);
  // one sequence's 16-token verify block over 2048 positions: 8 splits of
  // 256 keys (the fewest keys a verify split takes)
  pa_dims v1 = dims(1, 16, 16, 32, 8, 128, 64, 32, 32);
  pa::Plan pv1 = pa::make_plan(&v1, PA_BF16, 256);
  CHECK(pv1.dec_big && pv1.splits_big == 8 && pv1.pages_per_split_big == 4);
  // four equal 8192-token chunks: every sequence is prefill, so no decode
  // launch, no combine and no workspace
  pa_dims c5 = dims(4, 32768, 8192, 32, 8, 128, 64, 512, 128);
  pa::Plan p5 = pa::make_plan(&c5, PA_BF16, 256);
  CHECK(p5.prefill && p5.num_qtiles == 128 && !p5.dec_small && !p5.dec_big && !p5.combine);
  CHECK(p5.workspace_bytes == 0);
  // one token short of equal chunks: some sequence may have 8191 tokens, still no decode class
  c5.num_tokens = 32767;
  CHECK(!pa::make_plan(&c5, PA_BF16, 256).dec_small);
  // 3 x 8192 + 1: the last sequence may be a decode token
  c5.num_tokens = 3 * 8192 + 1;
  pa::Plan p5b = pa::make_plan(&c5, PA_BF16, 256);
  CHECK(p5b.prefill && p5b.dec_small && p5b.dec_big && p5b.combine);
  CHECK(p5b.bal_wgs == 0);                       // splits of 512 keys
  CHECK(p5b.workspace_bytes == (size_t)p5b.splits * 4 * 16 * 32 * 130 * 4 && p5b.splits >= p5b.splits_big);
  // two verify blocks of 15 and 15 (bound 16): at least 14 tokens each -> only the big tile
  pa_dims v2 = dims(2, 30, 16, 32, 8, 128, 64, 100, 16);
  pa::Plan pv2 = pa::make_plan(&v2, PA_BF16, 256);
  CHECK(!pv2.prefill && !pv2.dec_small && pv2.dec_big && pv2.big_nt == 4);
  // a 5-token verify bound: 20 rows -> 32-row tile; 17 tokens over 4
  // sequences leave room for one of 2 tokens (16-row tile)
  pa_dims v5 = dims(4, 17, 5, 32, 8, 128, 64, 100, 16);
  pa::Plan pv = pa::make_plan(&v5, PA_BF16, 256);
  CHECK(!pv.prefill && pv.dec_small && pv.dec_big && pv.big_nt == 2);
  v5.num_tokens = 20;                                      // four blocks of exactly 5
  pv = pa::make_plan(&v5, PA_BF16, 256);
  CHECK(!pv.prefill && !pv.dec_small && pv.dec_big && pv.big_nt == 2);
  // group 32: even one token needs 32 rows; decode class stops at 2 tokens
  pa_dims g32 = dims(2, 2, 1, 64, 2, 128, 64, 100, 16);
  pa::Plan pg = pa::make_plan(&g32, PA_BF16, 256);
  CHECK(pg.dec_max_n == 2 && !pg.dec_small && pg.dec_big && pg.big_nt == 2);
  // float32: a 600-key context (38 pages of 16) is cut into splits of at
  // least 64 keys, 4 pages: 10 splits of one 16-row tile and the combine;
  // a long one into at most 64 splits
  pa_dims c1 = dims(1, 1, 1, 8, 2, 64, 16, 64, 38);
  pa::Plan p1 = pa::make_plan(&c1, PA_F32, 256);
  CHECK(p1.splits == 10 && p1.pages_per_split == 4 && p1.combine && p1.num_qtiles == 1);
  CHECK(p1.workspace_bytes == (size_t)10 * 1 * 1 * 8 * 66 * 4);
  pa_dims l1 = dims(1, 1, 1, 8, 2, 64, 16, 2048, 2048);   // 32768 keys
  pa::Plan pl1 = pa::make_plan(&l1, PA_F32, 256);
  CHECK(pl1.splits == 64 && pl1.pages_per_split == 32 && pl1.combine && pl1.comb_tokens == 1);
  // a context of 64 keys or fewer stays one split with no combine
  pa_dims s1 = dims(1, 1, 1, 8, 2, 64, 16, 64, 4);
  pa::Plan ps1 = pa::make_plan(&s1, PA_F32, 256);
  CHECK(ps1.splits == 1 && !ps1.combine && ps1.workspace_bytes == 0);
  pa_dims f5 = dims(2, 10, 5, 8, 2, 64, 16, 64, 38);      // 5 tokens x group 4: two 16-row tiles
  CHECK(pa::make_plan(&f5, PA_F32, 256).num_qtiles == 2);
  c1.num_splits = 38;
  CHECK(pa::make_plan(&c1, PA_F32, 256).splits == 38);
  c1.num_splits = 100;
  CHECK(pa::choose_splits(&c1, PA_F32, 256) == 38);
  // argument checks
  pa_dims bad = c3; bad.num_kv_heads = 3;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_ERR_SHAPE);
  bad = c3; bad.head_dim = 96;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_ERR_UNSUPPORTED);
  bad = c3; bad.kv_stride_slot = 1028;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_ERR_UNSUPPORTED);
  CHECK(pa::check_dims(&bad, PA_F32) == PA_OK);     // 4-element multiple suffices for float32
  bad = c3; bad.q_stride_head = 64;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_ERR_SHAPE);
  bad = c3; bad.kv_stride_slot = (int64_t)1 << 26;   // tile offsets past 32 bits
  bad.kv_stride_page = bad.kv_stride_slot * bad.page_size;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_ERR_UNSUPPORTED);
  bad.kv_stride_slot = ((int64_t)1 << 26) - 8;
  CHECK(pa::check_dims(&bad, PA_BF16) == PA_OK);
  CHECK(pa::check_dims(nullptr, PA_BF16) == PA_ERR_NULL);

  // validate_host
  pa_dims v = dims(2, 3, 0, 4, 2, 64, 16, 4, 2);
  std::vector<int32_t> bt = {0, 1, 2, 3}, lens = {20, 5}, qsl = {0, 2, 3}, slots = {5, -1, 63};
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), slots.data(), 3, 1, &v) == PA_OK);
  lens[0] = 33;   // beyond W * ps
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 1, &v) == PA_ERR_INVALID_DATA);
  lens[0] = 20; bt[1] = 4;  // page outside the pool
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 1, &v) == PA_ERR_INVALID_DATA);
  bt[1] = 1; bt[3] = 77;    // unused entry: not checked
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 1, &v) == PA_OK);
  qsl = {0, 3, 2};
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 1, &v) == PA_ERR_INVALID_DATA);
  qsl = {0, 2, 3}; lens[1] = 0;   // one token over an empty context under causal
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 1, &v) == PA_ERR_INVALID_DATA);
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 0, &v) == PA_OK);
  v.max_query_len = 1;      // sequence 0 has 2 tokens
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), nullptr, 0, 0, &v) == PA_ERR_INVALID_DATA);
  v.max_query_len = 0;
  lens[1] = 5; slots = {5, 5, -1};
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), slots.data(), 3, 1, &v) == PA_ERR_INVALID_DATA);
  slots = {64, -1, 0};
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), slots.data(), 3, 1, &v) == PA_ERR_INVALID_DATA);
  slots = {-2, -1, 0};
  CHECK(pa::validate_host(bt.data(), lens.data(), qsl.data(), slots.data(), 3, 1, &v) == PA_ERR_INVALID_DATA);

  if (failures) { std::printf("%d failures\n", failures); return 1; }
  std::printf("host logic: all checks passed\n");
  return 0;
}
