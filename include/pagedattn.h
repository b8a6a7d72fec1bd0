/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged KV attention library.
 *
 * The library computes causal scaled-dot-product attention of a step's new
 * query tokens over a block-paged KV cache with grouped-query heads, for a
 * flattened ragged batch that may mix decode tokens, short verification
 * blocks and prefill chunks (page "32. Production attention kernels", One
 * kernel for the whole batch; page "Attention kernels", One kernel family,
 * three uses).  It also writes new K/V rows into the pools through a slot map.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All buffers are device memory owned by the caller.  The library
 *   allocates no memory, keeps no per-call state and never reads device
 *   memory back in paged_attention / kv_cache_write, so both can be captured
 *   in a hipGraph.  Its one device buffer of its own is the static scratch
 *   array of paged_attention_noalloc (PA_STATIC_SCRATCH_BYTES per device,
 *   loaded with the library's code).  Cached per device: the CU count, the
 *   address of that array, and two side streams
 *   with three events (default priority), created by the first bf16
 *   paged_attention call made outside graph capture and kept until the
 *   process ends.  They serve calls that launch more than one tile class
 *   (16-row decode tiles, verification tiles, prefill tiles: decided on the
 *   host from max_query_len and the group size).  HIP deals streams to the
 *   process's hardware queues in creation order, so making the first call
 *   before creating other streams keeps the side streams on queues of their
 *   own; side streams that share a queue with `stream` run their launches
 *   one after another.  A graph captured before they exist gets serial
 *   launches.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *   void*; NULL = the default stream).  Nothing is synchronised.  A mixed
 *   call forks into the side streams through an event recorded on `stream`
 *   and joins them back into `stream` before returning, so all of its work is
 *   ordered before anything enqueued on `stream` afterwards.  Calls from
 *   several host threads are serialised while they enqueue.
 * - Element types: PA_F32 or PA_BF16 for q, out, pools and new rows.  All
 *   metadata is int32.
 * - Strides are in elements.  The head dimension must be contiguous.
 * - On any error nothing is launched and no output is touched.  Device
 *   data (lengths, page ids, slots) is not validated on the hot path: kernels
 *   clamp lengths to the table, and pa_validate() checks the data on request.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,          /* a required pointer is NULL                        */
  PA_ERR_SHAPE = 2,         /* sizes/strides inconsistent (Hq % Hkv, D stride..)  */
  PA_ERR_UNSUPPORTED = 3,   /* dtype, head_dim or page_size not built            */
  PA_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required       */
  PA_ERR_LAUNCH = 5,        /* the HIP runtime refused a launch                  */
  PA_ERR_INVALID_DATA = 6,  /* pa_validate only: device metadata out of range   */
  PA_ERR_SCRATCH_LIMIT = 7  /* paged_attention_noalloc: the call's split partials
                               need more than PA_STATIC_SCRATCH_BYTES             */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * Host-side description of one call.  Only host scalars live here; every
 * per-step quantity (lengths, positions, page ids) is read from device
 * buffers, so a launch captured in a graph stays valid as sequences grow
 * (page "Attention kernels", Walking the block table).
 */
typedef struct pa_dims {
  int32_t num_seqs;        /* B: sequences in the flattened batch                 */
  int32_t num_tokens;      /* N: query tokens (rows of q and out)                  */
  int32_t max_query_len;   /* host upper bound on any sequence's tokens; 0 = N     */
  int32_t num_q_heads;     /* Hq                                                   */
  int32_t num_kv_heads;    /* Hkv; Hq % Hkv == 0, group G = Hq / Hkv               */
  int32_t head_dim;        /* D in {64, 128, 256}                                  */
  int32_t page_size;       /* ps in {16, 32, 64, 128}                              */
  int32_t num_pages;       /* P: pages in each pool                                */
  int32_t table_width;     /* W: entries per block-table row                       */
  int32_t num_splits;      /* split-KV count for decode rows; 0 = automatic        */
  int64_t q_stride_tok;    /* q  [N, Hq, D]: element stride between tokens         */
  int64_t q_stride_head;   /*                element stride between heads          */
  int64_t o_stride_tok;    /* out[N, Hq, D]                                        */
  int64_t o_stride_head;
  int64_t kv_stride_page;  /* pools: element strides of page, slot and head;       */
  int64_t kv_stride_slot;  /* the default layout [P, ps, Hkv, D] has               */
  int64_t kv_stride_head;  /* (ps*Hkv*D, Hkv*D, D).  K and V share the strides;   */
                           /* kv_stride_slot < 2^26 (16 slots of a tile stay      */
                           /* within 32-bit byte offsets), else UNSUPPORTED.      */
} pa_dims;

/*
 * paged_attention -- out = attention(q, K, V) for every query row.
 *
 * Definition (page "32. Production attention kernels", One kernel for the
 * whole batch and its first point; page "Attention and KV Cache", Attention as
 * primitive ops; page "paged-attn-xpu", Validation):
 *   sequence b owns flat rows [qsl[b], qsl[b+1]) with n = qsl[b+1]-qsl[b];
 *   L = clamp(context_lens[b], 0, W*ps) counts every cached position
 *   including the step's own tokens; token t sits at pos = L - n + t;
 *   query head h reads KV head h / G; key j (0 <= j < L) is stored at page
 *   block_tables[b*W + j/ps], slot j%ps; it is visible to token t iff
 *   causal == 0 or j <= pos;  out = softmax(scale * q.K^T over visible keys) V,
 *   and a row with no visible key is exactly zero.
 *
 * Arguments
 *   q             [N, Hq, D] (strides in dims), element type `dtype`.
 *   k_pool/v_pool [P, ps, Hkv, D] by the strides in dims.
 *   block_tables  int32 [B, W], row-major; entries past a sequence's
 *                 ceil(L/ps) pages are never read.
 *   context_lens  int32 [B].
 *   query_start_loc int32 [B+1], qsl[0] = 0, non-decreasing, qsl[B] = N.
 *   scale         finite float; scores are scale * q.k.
 *   causal        nonzero applies the position rule above.
 *   out           [N, Hq, D], same element type as q.  Rows not covered by
 *                 [qsl[0], qsl[B]) are not written.
 *   workspace     device scratch of at least pa_workspace_size(dims, dtype)
 *                 bytes (may be NULL when that size is 0).  Needs no
 *                 initialisation; contents are undefined afterwards.
 * Returns PA_OK, or an error status with nothing launched.
 */
pa_status paged_attention(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* query_start_loc, float scale, int causal,
                          void* out, void* workspace, size_t workspace_bytes,
                          const pa_dims* dims, pa_dtype dtype, void* stream);

/*
 * paged_attention_noalloc -- paged_attention for callers that cannot allocate
 * device memory (code under hipGraph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation, arguments, layouts, kernels
 * and results as paged_attention with the same dims, but no workspace
 * argument.  The split partials go to the library's own static device buffer
 * of PA_STATIC_SCRATCH_BYTES per device (a file-scope array loaded with the
 * library, held until the process ends); its device address is looked up
 * once per device, on the first call made on that device.  The call
 * allocates nothing: no hipMalloc / hipFree, no stream or event creation (all
 * launches go to `stream`, one after another, even for mixed batches).
 *
 * Limit: a call whose split partials need more than PA_STATIC_SCRATCH_BYTES
 * (pa_workspace_size(dims, dtype) > PA_STATIC_SCRATCH_BYTES) returns
 * PA_ERR_SCRATCH_LIMIT with nothing launched.
 * Sharing: every call on one device uses the same buffer and it keeps the
 * last call's contents.  Calls that overlap in time on one device (on
 * different streams without ordering between them, or from several threads)
 * race on it and their results are undefined; calls ordered on one stream
 * are safe.  Nothing in the buffer needs to start at zero: every partial a
 * call reads was written earlier in the same call.
 */
#define PA_STATIC_SCRATCH_BYTES (32u << 20)
pa_status paged_attention_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start_loc, float scale, int causal, void* out,
                                  const pa_dims* dims, pa_dtype dtype, void* stream);

/*
 * Quantized KV cache (page "32. Production attention kernels", Quantized KV
 * caches; page "Attention kernels", INT8 cache).  The pools hold 1-byte codes
 * ([P, ps, Hkv, D] by the kv strides of pa_dims, which count bytes here) and
 * one float32 scale per (page, slot, KV head) in two scale pools addressed by
 * the strides below (in floats).  A cached value is code * scale; a cached
 * key is code * scale * k_smooth[g][d] when smoothing factors are given.
 *
 * kv_cache_write_quant writes them: for each new head vector x (float32;
 * keys first divided by k_smooth), amax = max(max |x|, 1e-8),
 * scale = amax / q_max (127 int8, 448 fp8), codes = round-half-even(x / scale)
 * clamped to [-127, 127] (int8) or x / scale converted to float8 E4M3 with
 * round-to-nearest-even (fp8).  Every step is one float32 operation, so the
 * codes and scales are reproducible bit for bit.
 */
typedef enum pa_kv_dtype { PA_KV_SAME = 0, PA_KV_INT8 = 1, PA_KV_FP8_E4M3 = 2 } pa_kv_dtype;

typedef struct pa_kv_quant {
  int32_t kv_dtype;            /* PA_KV_INT8 or PA_KV_FP8_E4M3                      */
  int32_t reserved0;           /* must be 0                                          */
  float* k_scale;              /* scale pools: one float32 per (page, slot, KV head) */
  float* v_scale;
  int64_t scale_stride_page;   /* float strides of both scale pools                  */
  int64_t scale_stride_slot;
  int64_t scale_stride_head;
  const float* k_smooth;       /* [Hkv, D] float32 key smoothing factors, or NULL    */
} pa_kv_quant;

/*
 * Options of paged_attention_opts.  Zero-initialise the struct and set the
 * fields you use; a NULL options pointer means all defaults.
 *
 *   window  Sliding window (page "32. Production attention kernels", One
 *           kernel for the whole batch: the window mask and the point on
 *           sliding windows): when > 0, key j is visible to the query at
 *           position pos only if also j > pos - window, so a row sees at most
 *           its last `window` positions.  The condition applies with and
 *           without `causal`.  0 = no window; negative is PA_ERR_SHAPE.
 *   sinks   Attention sinks (same page, Stretch exercises: one learned logit
 *           per head joins every softmax denominator and contributes no
 *           value): device float32 [Hq], sink_h in the units of the scaled
 *           scores scale * q.k.  Row (i, h) becomes
 *           sum_J exp(x_j - M) v_j / (exp(sink_h - M) + sum_J exp(x_j - M)),
 *           M = max(sink_h, max_J x_j); a row with no visible key stays zero.
 *           NULL = no sinks.  Must be 4-byte aligned.
 *   kv_quant  Quantized pools (see pa_kv_quant), or NULL for pools in q's
 *           element type.  Needs dtype PA_BF16 (PA_ERR_UNSUPPORTED
 *           otherwise); the pools and kv strides must be 16-byte aligned in
 *           bytes and the scale pools 4-byte aligned.  The codes are
 *           converted to bf16 in registers, each score is scaled by its
 *           key's scale and each probability by its value's scale ahead of
 *           the PV product (decode and verification tiles); prefill tiles
 *           dequantize into bf16 when a block is staged.
 *   shared_prefix_len  Cascade attention (page "32. Production attention
 *           kernels", Stretch exercises: cascade attention): when > 0, every
 *           sequence's first shared_prefix_len positions are the same cached
 *           keys on the same pages (block_tables[b][0 .. len/ps) equal for
 *           all b; len a multiple of ps), and every query token sits after
 *           them (L_b - n_b >= len; pa_validate_opts checks both).  The
 *           prefix's K/V is then read once for the whole batch by MFMA
 *           tiles over all query tokens, each sequence attends its own
 *           suffix, and the two partial results are merged by their
 *           log-sum-exp.  The result equals the plain call's.  Needs dtype
 *           PA_BF16, no window, and max_query_len within the decode /
 *           verification class (n*G <= 64, n <= 16); PA_ERR_UNSUPPORTED
 *           otherwise.  Its workspace is pa_workspace_size_opts().
 */
typedef struct pa_attn_opts {
  int32_t window;
  int32_t reserved0;       /* must be 0 */
  const float* sinks;
  const pa_kv_quant* kv_quant;
  int32_t shared_prefix_len;
  int32_t reserved1;       /* must be 0 */
  /* The step's new K/V rows: with k_new set, the call first writes them as
   * kv_cache_write(k_new, v_new, k_pool, v_pool, slot_mapping,
   * dims->num_tokens, new_stride_tok, new_stride_head, dims, dtype) would,
   * then attends; so the pools are written (plain pools only: with kv_quant,
   * PA_ERR_UNSUPPORTED).  A batch of decode tokens alone (no prefill or
   * verification tiles) does the write inside its decode launch: the
   * workgroup whose pages hold a token's position writes that token's rows
   * of its KV head before it reads a key, which requires every new token's
   * slot to be the one its own sequence's table gives for its position (the
   * contract of a decode step; pa_validate checks slots, not this).  Other
   * batches launch the write first.  k_new == NULL: no write. */
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int64_t new_stride_tok, new_stride_head;   /* element strides of [N, Hkv, D] k_new / v_new */
} pa_attn_opts;

/*
 * paged_attention_opts -- paged_attention with the options above.  Every
 * other argument, the layouts and the error behaviour are those of
 * paged_attention, which is this call with opts == NULL.  The workspace
 * needed is pa_workspace_size_opts(dims, dtype, opts); without a shared
 * prefix it never exceeds pa_workspace_size(dims, dtype) (a window only
 * lowers the split count).
 */
pa_status paged_attention_opts(const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* query_start_loc, float scale, int causal,
                               void* out, void* workspace, size_t workspace_bytes,
                               const pa_dims* dims, pa_dtype dtype, const pa_attn_opts* opts,
                               void* stream);

/*
 * kv_cache_write -- scatter new K/V rows into the pools.
 *
 * Token i's rows k_new[i, :, :] and v_new[i, :, :] ([num_tokens, Hkv, D] with
 * the given token and head strides, D contiguous) go to flat slot
 * s = slot_mapping[i] = page * ps + offset of both pools; s < 0 writes
 * nothing (page "Attention and KV Cache", Paged KV: the write map; page
 * "32. Production attention kernels", write through slot_mapping).  Slots
 * >= P*ps are skipped as a guard; duplicate slots are a caller error that
 * only pa_validate reports.  Uses dims->num_kv_heads, head_dim, page_size,
 * num_pages and the kv strides.
 */
pa_status kv_cache_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         const int32_t* slot_mapping, int32_t num_tokens,
                         int64_t new_stride_tok, int64_t new_stride_head,
                         const pa_dims* dims, pa_dtype dtype, void* stream);

/*
 * kv_cache_write_quant -- kv_cache_write into quantized pools: token i's K and
 * V head vectors (new_dtype PA_BF16 or PA_F32, [num_tokens, Hkv, D] with the
 * given element strides, D contiguous) are quantized as described above and
 * their codes and scales go to flat slot slot_mapping[i]; -1 writes nothing
 * and slots >= P*ps are skipped.  k_codes / v_codes are the code pools (kv
 * strides of dims in bytes, 16-byte aligned), `quant` gives the scale pools
 * and the optional key smoothing factors.
 */
pa_status kv_cache_write_quant(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                               const int32_t* slot_mapping, int32_t num_tokens, int64_t new_stride_tok,
                               int64_t new_stride_head, const pa_dims* dims, pa_dtype new_dtype,
                               const pa_kv_quant* quant, void* stream);

/*
 * pa_workspace_size -- bytes of workspace paged_attention needs for these
 * dims: S * B * T * Hq * (D + 2) * 4 when split-KV partials are used, else 0.
 * S is the largest split count of the call's launches, T the query tokens per
 * sequence the split launches can take (min(max_query_len, 16, 64/G) for
 * bf16, max_query_len for float32).  Each partial is a float32 accumulator
 * with its running max and sum (page "Attention kernels", Decode: GQA packing
 * and split-KV).  Prefill tokens take no workspace.  Returns 0 for invalid
 * dims as well; paged_attention reports those.
 */
size_t pa_workspace_size(const pa_dims* dims, pa_dtype dtype);

/*
 * pa_workspace_size_opts -- the same for paged_attention_opts: with a shared
 * prefix, (Sp + Ss) * N * Hq * (D + 2) * 4 bytes, Sp the prefix key ranges
 * and Ss the suffix splits; otherwise pa_workspace_size.  0 for invalid
 * arguments.
 */
size_t pa_workspace_size_opts(const pa_dims* dims, pa_dtype dtype, const pa_attn_opts* opts);

/*
 * pa_choose_splits -- the split count paged_attention will use for decode
 * rows (one token, or n*G <= 16 rows): dims->num_splits when > 0, else enough
 * workgroups for two per CU of the current device (three when every sequence
 * has one token, max_query_len == 1, and two are not reached), with at least
 * 128 keys per split and at most 64 splits (page "32. Production attention
 * kernels", How many splits?); this is the count for bf16 pools (float32
 * calls aim at one workgroup per CU with at least 64 keys per split, at most
 * 64 splits).  Verification blocks (16 < n*G <= 64 rows)
 * take a count of their own: about two workgroups per CU over the batch's
 * (sequence, KV head) pairs, at least 16 when prefill or decode-row tiles
 * share the batch (the few verification steps of a mixed batch then run
 * short key loops), with at least 256 keys per split and at most 64;
 * dims->num_splits, when > 0, sets both counts.  Returns 1 for invalid dims.
 */
int32_t pa_choose_splits(const pa_dims* dims);

/*
 * pa_validate -- SYNCHRONOUS debug/test check of device metadata.
 * Copies the metadata to the host and checks: 0 <= qsl[b] <= qsl[b+1],
 * qsl[0] == 0, qsl[B] == N; n <= max_query_len when that bound is set;
 * 0 <= context_lens[b] <= W*ps; n <= L when
 * causal (a token with pos < 0 sees nothing); every block-table entry a
 * sequence uses lies in [0, P); and, when slot_mapping is not NULL, every
 * slot is -1 or in [0, P*ps) and no slot repeats (page "Attention and KV
 * Cache": its checked write map rejects out-of-pool and repeated slots).  Returns PA_OK, PA_ERR_INVALID_DATA, or an argument error.
 */
pa_status pa_validate(const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* query_start_loc, const int32_t* slot_mapping,
                      int32_t num_slots, int causal, const pa_dims* dims, void* stream);

/*
 * pa_validate_opts -- pa_validate plus the contract of the options: with a
 * shared prefix of len positions, every sequence's first len/ps table entries
 * equal sequence 0's and L_b - n_b >= len.  SYNCHRONOUS, debug and test only.
 */
pa_status pa_validate_opts(const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* query_start_loc, const int32_t* slot_mapping,
                           int32_t num_slots, int causal, const pa_dims* dims, const pa_attn_opts* opts,
                           void* stream);

/* pa_status_string -- static human-readable text for a status code. */
const char* pa_status_string(pa_status status);

/* pa_device_cu_count -- compute units of the current device (cached). */
int32_t pa_device_cu_count(void);

/*
 * pa_read_probe -- measurement aid, not part of the attention path: reads the
 * device buffer `buf` of `bytes` bytes once with 16-byte streaming loads
 * (16384 workgroups of 256 threads) and writes one folded word per workgroup
 * to the device buffer `sink`, so the reads cannot be elided.  The time it
 * takes gives the HBM read rate a streaming kernel reaches on this device,
 * the practical ceiling the decode kernel's read rate is compared with.
 * `buf` must be 16-byte aligned and `bytes` a multiple of 16
 * (PA_ERR_SHAPE otherwise); `sink` needs 65536 bytes (PA_ERR_WORKSPACE);
 * NULL pointers give PA_ERR_NULL.  Asynchronous on `stream`; the caller owns
 * both buffers.
 */
pa_status pa_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
