// C-ABI entry points of libpagedattn.so (declared in include/pagedattn.h).
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "host_logic.h"
#include "pa_device.h"

namespace pa {
hipError_t launch_decode(const AttnParams& p, int nt, hipStream_t st);
hipError_t launch_prefill(const AttnParams& p, hipStream_t st);
hipError_t launch_prefix(const AttnParams& p, hipStream_t st);
hipError_t launch_verify16(const AttnParams& p, hipStream_t st);
hipError_t launch_prefill16_small(const AttnParams& p, hipStream_t st);
bool verify16_supported(int head_dim);

// Verification tiles (16 < n*G <= 64 rows): over bf16 pools with 128- or
// 256-dim heads the shared-block tile of prefill16.hip, otherwise the decode
// kernel's 32- and 64-row tiles.
static hipError_t launch_verify(const AttnParams& p, int big_nt, hipStream_t st) {
  if (p.kv_code == KV_BF16 && verify16_supported(p.head_dim)) return launch_verify16(p, st);
  return launch_decode(p, big_nt, st);
}
hipError_t launch_f32(const AttnParams& p, hipStream_t st);
hipError_t launch_combine(const AttnParams& p, bool bf16, hipStream_t st);
bool mixed_supported(int head_dim);
hipError_t launch_mixed(const AttnParams& pp, bool have_pre, const AttnParams& pv, bool have_ver,
                        const AttnParams& pd, bool have_dec, hipStream_t st);
hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t st);
hipError_t launch_kv_write_quant(const KvWriteParams& p, hipStream_t st);

static std::atomic<int> g_cu_cache[64];

static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (dev < 64) g_cu_cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Argument checks of a quantized-pool description (nothing is read from the
// device): a known code type, non-negative scale strides, 16-byte kv strides
// (1-byte codes), 4-byte aligned scale and smoothing pointers.
static pa_status check_kv_quant(const pa_kv_quant* q, const pa_dims* d) {
  if (q->kv_dtype != PA_KV_INT8 && q->kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
  if (q->reserved0 != 0) return PA_ERR_SHAPE;
  if (q->scale_stride_page < 0 || q->scale_stride_slot < 0 || q->scale_stride_head < 0) return PA_ERR_SHAPE;
  if (d->kv_stride_page % 16 || d->kv_stride_slot % 16 || d->kv_stride_head % 16) return PA_ERR_UNSUPPORTED;
  if (!aligned4(q->k_scale) || !aligned4(q->v_scale) || !aligned4(q->k_smooth)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Two side streams and their events per device, so the launches of a mixed
// batch (prefill tiles, 16-row decode tiles, verification tiles) run side by
// side instead of one after another: a prefill launch alone fills few CUs
// (page "Attention kernels", Open questions: a chunk's tiles versus the
// chip's CUs).  They are created once, on the first bf16 call made outside
// graph capture, at the default priority, and live until the process ends.
// The caller's stream forks into them through an event and joins them again
// before paged_attention returns, so the call stays stream-ordered and
// capturable.
struct SideStreams {
  std::mutex mu;
  bool ready = false, failed = false;
  hipStream_t side[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr, join[2] = {nullptr, nullptr};
};
static SideStreams g_side[64];

// Returns the device's side streams with their mutex held, or nullptr.
static SideStreams* lock_side_streams(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStreams& ss = g_side[dev];
  ss.mu.lock();
  if (!ss.ready && !ss.failed) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
      ss.mu.unlock();
      return nullptr;                      // nothing is created while a graph is being captured
    }
    bool ok = hipStreamCreateWithFlags(&ss.side[0], hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&ss.side[1], hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&ss.join[0], hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&ss.join[1], hipEventDisableTiming) == hipSuccess;
    if (ok) {
      ss.ready = true;
    } else {
      ss.failed = true;                    // serial launches from now on
      (void)hipGetLastError();
    }
  }
  if (!ss.ready) {
    ss.mu.unlock();
    return nullptr;
  }
  return &ss;
}

// Device memory of paged_attention_noalloc: the split partials of a call go
// here instead of a caller's workspace.  One copy per device, at its own
// address, loaded with the library's code and held until the process ends.
// Host code never uses the name itself for device memory (on the host it is
// only a stand-in): the device address comes from hipGetSymbolAddress, once
// per device, and is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// Device address of `scratch` on the current device, or nullptr.
static void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace pa

using namespace pa;

extern "C" {
static pa_status attention_impl(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start_loc, float scale, int causal,
                                void* out, void* workspace, size_t workspace_bytes, const pa_dims* dims,
                                pa_dtype dtype, const pa_attn_opts* opts, hipStream_t stream, bool side_ok);
static pa_status kv_write_setup(const void* k_new, const void* v_new, const void* k_pool, const void* v_pool,
                                const int32_t* slot_mapping, int32_t num_tokens, int64_t new_stride_tok,
                                int64_t new_stride_head, const pa_dims* dims, pa_dtype dtype, KvWriteParams& p);


const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent sizes or strides";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, page_size, group or alignment";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_INVALID_DATA: return "device metadata out of range";
    case PA_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

int32_t pa_device_cu_count(void) { return cu_count(); }

int32_t pa_choose_splits(const pa_dims* dims) {
  if (check_dims(dims, PA_BF16) != PA_OK && check_dims(dims, PA_F32) != PA_OK) return 1;
  const Plan pl = make_plan(dims, PA_BF16, cu_count());
  return pl.splits;
}

size_t pa_workspace_size(const pa_dims* dims, pa_dtype dtype) {
  if (check_dims(dims, dtype) != PA_OK) return 0;
  return make_plan(dims, dtype, cu_count()).workspace_bytes;
}

size_t pa_workspace_size_opts(const pa_dims* dims, pa_dtype dtype, const pa_attn_opts* opts) {
  if (check_dims(dims, dtype) != PA_OK) return 0;
  const int window = opts && opts->window > 0 ? opts->window : 0;
  if (opts && opts->shared_prefix_len > 0) {
    const CascadePlan cp = make_cascade_plan(dims, dtype, cu_count(), opts->shared_prefix_len, window);
    return cp.status == PA_OK ? cp.workspace_bytes : 0;
  }
  return make_plan(dims, dtype, cu_count(), window).workspace_bytes;
}

pa_status paged_attention(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* query_start_loc, float scale, int causal,
                          void* out, void* workspace, size_t workspace_bytes, const pa_dims* dims, pa_dtype dtype,
                          void* stream) {
  return paged_attention_opts(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, causal, out,
                              workspace, workspace_bytes, dims, dtype, nullptr, stream);
}

pa_status paged_attention_opts(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                               const int32_t* context_lens, const int32_t* query_start_loc, float scale, int causal,
                               void* out, void* workspace, size_t workspace_bytes, const pa_dims* dims,
                               pa_dtype dtype, const pa_attn_opts* opts, void* stream) {
  return attention_impl(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, causal, out, workspace,
                        workspace_bytes, dims, dtype, opts, (hipStream_t)stream, true);
}

pa_status paged_attention_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start_loc, float scale, int causal, void* out,
                                  const pa_dims* dims, pa_dtype dtype, void* stream) {
  pa_status st = check_dims(dims, dtype);
  if (st != PA_OK) return st;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  // the split partials this call needs must fit the static buffer
  const size_t need = make_plan(dims, dtype, cu_count()).workspace_bytes;
  if (need > (size_t)PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_address())) return PA_ERR_LAUNCH;
  return attention_impl(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale, causal, out, ws,
                        ws ? (size_t)PA_STATIC_SCRATCH_BYTES : 0, dims, dtype, nullptr, (hipStream_t)stream, false);
}

// The body of paged_attention_opts.  side_ok = false keeps every launch on
// `stream`: the side streams are neither created nor used.
static pa_status attention_impl(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start_loc, float scale, int causal,
                                void* out, void* workspace, size_t workspace_bytes, const pa_dims* dims,
                                pa_dtype dtype, const pa_attn_opts* opts, hipStream_t stream, bool side_ok) {
  pa_status st = check_dims(dims, dtype);
  if (st != PA_OK) return st;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  const int window = opts ? opts->window : 0;
  const float* sinks = opts ? opts->sinks : nullptr;
  const int prefix_len = opts ? opts->shared_prefix_len : 0;
  if (window < 0 || prefix_len < 0 || (opts && (opts->reserved0 != 0 || opts->reserved1 != 0))) return PA_ERR_SHAPE;
  if (sinks && ((uintptr_t)sinks & 3u)) return PA_ERR_UNSUPPORTED;
  const pa_kv_quant* kq = opts ? opts->kv_quant : nullptr;
  if (kq) {
    if ((st = check_kv_quant(kq, dims)) != PA_OK) return st;
    if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  }
  // the step's new rows, written before the call attends
  KvWriteParams wp{};
  if (opts && opts->k_new) {
    if (kq) return PA_ERR_UNSUPPORTED;       // a quantizing write is kv_cache_write_quant's
    if ((st = kv_write_setup(opts->k_new, opts->v_new, k_pool, v_pool, opts->slot_mapping, dims->num_tokens,
                             opts->new_stride_tok, opts->new_stride_head, dims, dtype, wp)) != PA_OK)
      return st;
  }
  if (dims->num_seqs == 0 || dims->num_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start_loc || !out) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_UNSUPPORTED;
  if (kq && (!kq->k_scale || !kq->v_scale)) return PA_ERR_NULL;
  const Plan pl = make_plan(dims, dtype, cu_count(), window);
  CascadePlan cp{};
  if (prefix_len > 0) {
    cp = make_cascade_plan(dims, dtype, cu_count(), prefix_len, window);
    if (cp.status != PA_OK) return cp.status;
  }
  const size_t need = prefix_len > 0 ? cp.workspace_bytes : pl.workspace_bytes;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PA_ERR_WORKSPACE;

  AttnParams p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.out = out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start_loc = query_start_loc;
  const int N = dims->num_tokens, Hq = dims->num_q_heads;
  if (pl.ws_splits > 1) {
    p.ws_acc = (float*)workspace;
    p.ws_ml = (float*)workspace + (size_t)pl.ws_splits * dims->num_seqs * pl.ws_tok * Hq * dims->head_dim;
  }
  p.q_stride_tok = dims->q_stride_tok;
  p.q_stride_head = dims->q_stride_head;
  p.o_stride_tok = dims->o_stride_tok;
  p.o_stride_head = dims->o_stride_head;
  p.kv_stride_page = dims->kv_stride_page;
  p.kv_stride_slot = dims->kv_stride_slot;
  p.kv_stride_head = dims->kv_stride_head;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.num_seqs = dims->num_seqs;
  p.num_tokens = N;
  p.num_q_heads = Hq;
  p.num_kv_heads = dims->num_kv_heads;
  p.group = Hq / dims->num_kv_heads;
  p.head_dim = dims->head_dim;
  p.page_size = dims->page_size;
  p.page_shift = __builtin_ctz((unsigned)dims->page_size);
  p.num_pages = dims->num_pages;
  p.table_width = dims->table_width;
  p.num_splits = pl.splits;
  p.pages_per_split = pl.pages_per_split;
  p.causal = causal ? 1 : 0;
  p.dec_max_n = pl.dec_max_n;
  p.tok_per_tile = pl.tok_per_tile;
  p.num_qtiles = pl.num_qtiles;
  p.comb_max_n = pl.comb_max_n;
  p.comb_tokens = pl.comb_tokens;
  p.ws_tok = pl.ws_tok;
  p.comb_splits_small = pl.dec_small || dtype == PA_F32 ? pl.splits : 1;
  p.comb_splits_big = pl.dec_big || dtype == PA_F32 ? pl.splits_big : 1;
  p.window = pl.window;
  p.sinks = sinks;
  if (kq) {
    p.kv_code = kq->kv_dtype == PA_KV_INT8 ? KV_INT8 : KV_FP8;
    p.k_scale = kq->k_scale;
    p.v_scale = kq->v_scale;
    p.sc_stride_page = kq->scale_stride_page;
    p.sc_stride_slot = kq->scale_stride_slot;
    p.sc_stride_head = kq->scale_stride_head;
    p.k_smooth = kq->k_smooth;
  }

  hipStream_t s = stream;
  hipError_t e = hipSuccess;
  if (prefix_len > 0) {
    // cascade: prefix pass over all query tokens (split slots 0..Sp-1), the
    // sequences' own suffixes (slots Sp..Sp+Ss-1), then one combine of all
    // partials per row; workspace rows are flat tokens
    const int slots = cp.prefix_splits + cp.suffix_splits;
    p.ws_acc = (float*)workspace;
    p.ws_ml = (float*)workspace + (size_t)slots * N * Hq * dims->head_dim;
    p.ws_flat = 1;
    p.comb_splits_small = p.comb_splits_big = slots;
    p.comb_max_n = pl.dec_max_n;
    p.comb_tokens = pl.mql < pl.dec_max_n ? pl.mql : pl.dec_max_n;
    AttnParams pre = p;
    pre.prefix_len = prefix_len;
    pre.prefix_splits = cp.prefix_splits;
    pre.prefix_split_keys = cp.prefix_split_keys;
    pre.num_qtiles = cp.prefix_qtiles;
    pre.tok_per_tile = cp.prefix_tile_tokens;
    pre.sinks = nullptr;                       // folded once, by the suffix pass
    AttnParams suf = p;
    suf.key_lo = prefix_len;
    suf.force_partial = 1;
    suf.split_base = cp.prefix_splits;
    suf.num_splits = cp.suffix_splits;
    suf.pages_per_split = cp.suffix_pages_per_split;
    AttnParams q1 = suf, q2 = suf;
    q1.row_lo = 0;
    q1.row_hi = 16;
    q2.row_lo = 16;
    q2.row_hi = 16 * pl.big_nt;
    // Launched in order on the caller's stream: the passes are short, and a
    // fork onto a side stream cost more than their overlap gained.  With a
    // one-split suffix the decode kernel folds the prefix partials into its
    // output itself and no combine is launched.
    const bool fold = cp.suffix_splits == 1;
    if (fold) {
      q1.merge_prefix = q2.merge_prefix = cp.prefix_splits;
      q1.force_partial = q2.force_partial = 0;
    }
    if (wp.num_tokens > 0) e = launch_kv_write(wp, s);
    if (e == hipSuccess && cp.prefix_splits > 0) e = launch_prefix(pre, s);
    if (e == hipSuccess && pl.dec_small) e = launch_decode(q1, 1, s);
    if (e == hipSuccess && pl.dec_big) e = launch_decode(q2, pl.big_nt, s);
    if (e == hipSuccess && !fold) e = launch_combine(p, true, s);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
  }
  if (dtype == PA_F32) {
    if (wp.num_tokens > 0) e = launch_kv_write(wp, s);
    if (e == hipSuccess) e = launch_f32(p, s);
    if (e == hipSuccess && pl.combine) e = launch_combine(p, false, s);
  } else {
    if (pl.bal_wgs > 0) {
      // balanced 16-row tiles: partial slots b + w (w: the wave), then the
      // combine's map
      const size_t rows = (size_t)(dims->num_seqs + 4 * pl.bal_wgs) * pl.ws_tok * Hq;
      p.bal_wgs = pl.bal_wgs;
      p.bal_min_chunks = pl.bal_min_chunks;
      p.bal_acc = (float*)((char*)workspace + pl.bal_offset);
      p.bal_ml = p.bal_acc + rows * dims->head_dim;
      p.bal_meta = (int32_t*)(p.bal_ml + rows * 2);
    }
    AttnParams q1 = p;                       // 16-row decode tiles
    q1.row_lo = 0;
    q1.row_hi = 16;
    AttnParams q2 = p;                       // verification tiles
    q2.row_lo = 16;
    q2.row_hi = 16 * pl.big_nt;
    q2.num_splits = pl.splits_big;
    q2.pages_per_split = pl.pages_per_split_big;
    const int classes = (int)pl.prefill + (int)pl.dec_small + (int)pl.dec_big;
    // prefill tiles: 64-row tiles spread over the chip for a short prefill
    // over bf16 pools, the planned tiles otherwise
    auto run_prefill = [&](hipStream_t st) -> hipError_t {
      if (!kq && prefill_small_tiles(dims, cu_count())) {
        AttnParams pp = p;
        pp.tok_per_tile = 64 / p.group;
        pp.num_qtiles = prefill_small_slots(dims->num_tokens, dims->num_seqs, pl.mql, pp.tok_per_tile, pl.dec_max_n);
        return launch_prefill16_small(pp, st);
      }
      return launch_prefill(p, st);
    };
    // New rows: a batch of 16-row decode tiles alone on a split launch writes
    // them inside its decode launch (each workgroup the rows of its own KV
    // head and pages, before it reads a key); otherwise they are written
    // first.
    const bool fuse = wp.num_tokens > 0 && classes == 1 && pl.dec_small && pl.bal_wgs == 0;
    if (wp.num_tokens > 0 && !fuse && launch_kv_write(wp, s) != hipSuccess) return PA_ERR_LAUNCH;
#ifndef PA_MIXED
#define PA_MIXED 1
#endif
    // A batch of several classes over bf16 pools with 128-dim heads whose
    // prefill (if any) takes 64-row tiles runs as one launch of all its
    // tiles, then the combine, on the caller's stream.  Beside a prefill
    // class a balanced decode class takes about one workgroup per CU (its
    // partial slots stay within the planned ones).  The mixed batch measured
    // 150 us with the three launches on forked streams, 148 us as one launch
    // with the prefill tiles first and two decode workgroups per CU, 144 us
    // with the decode tiles first, 130-135 us with the decode tiles first at
    // 0.75-1.25 workgroups per CU, and 122-125 us with the prefill tiles in a
    // compact grid (67 slots per KV head instead of 1,024).
    if (PA_MIXED && classes >= 2 && !kq && mixed_supported(dims->head_dim) &&
        (!pl.prefill || prefill_small_tiles(dims, cu_count()))) {
      AttnParams pp = p;
      pp.tok_per_tile = 64 / p.group;
      pp.num_qtiles = prefill_small_slots(dims->num_tokens, dims->num_seqs, pl.mql, pp.tok_per_tile, pl.dec_max_n);
      AttnParams qd = q1;
      if (qd.bal_wgs > 0 && pl.prefill) qd.bal_wgs = (cu_count() + p.num_kv_heads - 1) / p.num_kv_heads;
      e = launch_mixed(pp, pl.prefill, q2, pl.dec_big, qd, pl.dec_small, s);
      if (e == hipSuccess && pl.combine) e = launch_combine(p, true, s);
      return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    // The side streams are made on the first bf16 call of any kind: HIP deals
    // streams to the process's few hardware queues in the order they are
    // created, and side streams that share a queue with the caller's stream
    // run their launches one after the other (the mixed batch measured 270
    // instead of 171 us with side streams made after two other streams).
    SideStreams* ss = side_ok ? lock_side_streams(s) : nullptr;
    if (ss && classes < 2) {
      ss->mu.unlock();
      ss = nullptr;
    }
    if (ss) {
      // prefill on side 0, verification on side 1 (when 16-row tiles are
      // launched too), 16-row tiles and the combine on the caller's stream;
      // the combine waits for side 1, the return for side 0
      const bool p_side = pl.prefill, v_side = pl.dec_big && pl.dec_small;
      e = hipEventRecord(ss->fork, s);
      bool p_fork = false, v_fork = false;   // side streams that joined this call
      if (e == hipSuccess && p_side) p_fork = (e = hipStreamWaitEvent(ss->side[0], ss->fork, 0)) == hipSuccess;
      if (e == hipSuccess && v_side) v_fork = (e = hipStreamWaitEvent(ss->side[1], ss->fork, 0)) == hipSuccess;
      if (e == hipSuccess && p_side) e = run_prefill(ss->side[0]);
      if (e == hipSuccess && pl.dec_big) e = launch_verify(q2, pl.big_nt, v_side ? ss->side[1] : s);
      if (e == hipSuccess && pl.dec_small) e = launch_decode(q1, 1, s);
      if (v_fork) {                          // joined even after a failed launch
        hipError_t j = hipEventRecord(ss->join[1], ss->side[1]);
        if (j == hipSuccess) j = hipStreamWaitEvent(s, ss->join[1], 0);
        if (e == hipSuccess) e = j;
      }
      if (e == hipSuccess && pl.combine) e = launch_combine(p, true, s);
      if (p_fork) {
        hipError_t j = hipEventRecord(ss->join[0], ss->side[0]);
        if (j == hipSuccess) j = hipStreamWaitEvent(s, ss->join[0], 0);
        if (e == hipSuccess) e = j;
      }
      ss->mu.unlock();
      return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    if (pl.prefill) e = run_prefill(s);
    q1.head_first = classes == 1;            // decode tiles have the chip to themselves
    if (fuse) {
      q1.new_k = wp.k_new;
      q1.new_v = wp.v_new;
      q1.new_slots = wp.slot_mapping;
      q1.new_stride_tok = wp.new_stride_tok;
      q1.new_stride_head = wp.new_stride_head;
    }
    if (e == hipSuccess && pl.dec_small) e = launch_decode(q1, 1, s);
    if (e == hipSuccess && pl.dec_big) e = launch_verify(q2, pl.big_nt, s);
    if (e == hipSuccess && pl.combine) e = launch_combine(p, true, s);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// Checks and launch parameters of a slot-mapped write of num_tokens new rows
// (kv_cache_write; also the new rows of paged_attention_opts).  PA_OK with
// p.num_tokens == 0 means there is nothing to write.
static pa_status kv_write_setup(const void* k_new, const void* v_new, const void* k_pool, const void* v_pool,
                                const int32_t* slot_mapping, int32_t num_tokens, int64_t new_stride_tok,
                                int64_t new_stride_head, const pa_dims* dims, pa_dtype dtype, KvWriteParams& p) {
  p = KvWriteParams{};
  if (!dims) return PA_ERR_NULL;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || new_stride_tok < 0 || new_stride_head < 0) return PA_ERR_SHAPE;
  if (dims->num_kv_heads < 1 || dims->num_pages < 0) return PA_ERR_SHAPE;
  if (dims->head_dim != 64 && dims->head_dim != 128 && dims->head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (dims->page_size != 16 && dims->page_size != 32 && dims->page_size != 64 && dims->page_size != 128)
    return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL;
  const int64_t vec = dtype == PA_BF16 ? 8 : 4;
  const int64_t s[] = {new_stride_tok, new_stride_head, dims->kv_stride_page, dims->kv_stride_slot,
                       dims->kv_stride_head};
  for (int64_t x : s)
    if (x % vec) return PA_ERR_UNSUPPORTED;
  if ((dims->num_kv_heads > 1 && (new_stride_head < dims->head_dim || dims->kv_stride_head < dims->head_dim)))
    return PA_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return PA_ERR_UNSUPPORTED;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = const_cast<void*>(k_pool);
  p.v_pool = const_cast<void*>(v_pool);
  p.slot_mapping = slot_mapping;
  p.new_stride_tok = new_stride_tok;
  p.new_stride_head = new_stride_head;
  p.kv_stride_page = dims->kv_stride_page;
  p.kv_stride_slot = dims->kv_stride_slot;
  p.kv_stride_head = dims->kv_stride_head;
  p.num_tokens = num_tokens;
  p.num_kv_heads = dims->num_kv_heads;
  p.head_dim = dims->head_dim;
  p.page_size = dims->page_size;
  p.num_pages = dims->num_pages;
  p.elem_bytes = dtype == PA_BF16 ? 2 : 4;
  return PA_OK;
}

pa_status kv_cache_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                         const int32_t* slot_mapping, int32_t num_tokens, int64_t new_stride_tok,
                         int64_t new_stride_head, const pa_dims* dims, pa_dtype dtype, void* stream) {
  KvWriteParams p;
  const pa_status st = kv_write_setup(k_new, v_new, k_pool, v_pool, slot_mapping, num_tokens, new_stride_tok,
                                      new_stride_head, dims, dtype, p);
  if (st != PA_OK || p.num_tokens == 0) return st;
  return launch_kv_write(p, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status kv_cache_write_quant(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                               const int32_t* slot_mapping, int32_t num_tokens, int64_t new_stride_tok,
                               int64_t new_stride_head, const pa_dims* dims, pa_dtype new_dtype,
                               const pa_kv_quant* quant, void* stream) {
  if (!dims || !quant) return PA_ERR_NULL;
  if (new_dtype != PA_F32 && new_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || new_stride_tok < 0 || new_stride_head < 0) return PA_ERR_SHAPE;
  if (dims->num_kv_heads < 1 || dims->num_pages < 0) return PA_ERR_SHAPE;
  if (dims->head_dim != 64 && dims->head_dim != 128 && dims->head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (dims->page_size != 16 && dims->page_size != 32 && dims->page_size != 64 && dims->page_size != 128)
    return PA_ERR_UNSUPPORTED;
  if (dims->kv_stride_page < 0 || dims->kv_stride_slot < 0 || dims->kv_stride_head < 0) return PA_ERR_SHAPE;
  pa_status st = check_kv_quant(quant, dims);
  if (st != PA_OK) return st;
  if (dims->num_kv_heads > 1 && (new_stride_head < dims->head_dim || dims->kv_stride_head < dims->head_dim))
    return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_codes || !v_codes || !slot_mapping || !quant->k_scale || !quant->v_scale)
    return PA_ERR_NULL;
  const int64_t vec = new_dtype == PA_BF16 ? 8 : 4;
  if (new_stride_tok % vec || new_stride_head % vec) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_codes) || !aligned16(v_codes))
    return PA_ERR_UNSUPPORTED;
  KvWriteParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_pool = k_codes;
  p.v_pool = v_codes;
  p.slot_mapping = slot_mapping;
  p.new_stride_tok = new_stride_tok;
  p.new_stride_head = new_stride_head;
  p.kv_stride_page = dims->kv_stride_page;
  p.kv_stride_slot = dims->kv_stride_slot;
  p.kv_stride_head = dims->kv_stride_head;
  p.num_tokens = num_tokens;
  p.num_kv_heads = dims->num_kv_heads;
  p.head_dim = dims->head_dim;
  p.page_size = dims->page_size;
  p.num_pages = dims->num_pages;
  p.elem_bytes = new_dtype == PA_BF16 ? 2 : 4;
  p.kv_code = quant->kv_dtype == PA_KV_INT8 ? KV_INT8 : KV_FP8;
  p.k_scale = quant->k_scale;
  p.v_scale = quant->v_scale;
  p.sc_stride_page = quant->scale_stride_page;
  p.sc_stride_slot = quant->scale_stride_slot;
  p.sc_stride_head = quant->scale_stride_head;
  p.k_smooth = quant->k_smooth;
  return launch_kv_write_quant(p, (hipStream_t)stream) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_validate(const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                      const int32_t* slot_mapping, int32_t num_slots, int causal, const pa_dims* dims,
                      void* stream) {
  return pa_validate_opts(block_tables, context_lens, query_start_loc, slot_mapping, num_slots, causal, dims,
                          nullptr, stream);
}

pa_status pa_validate_opts(const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* query_start_loc, const int32_t* slot_mapping, int32_t num_slots,
                           int causal, const pa_dims* dims, const pa_attn_opts* opts, void* stream) {
  if (!dims) return PA_ERR_NULL;
  if (dims->num_seqs < 0 || dims->table_width < 0 || dims->num_pages < 0 || num_slots < 0) return PA_ERR_SHAPE;
  if (dims->page_size < 1) return PA_ERR_UNSUPPORTED;
  const int B = dims->num_seqs, W = dims->table_width;
  if (B > 0 && (!block_tables || !context_lens || !query_start_loc)) return PA_ERR_NULL;
  if (num_slots > 0 && !slot_mapping) return PA_ERR_NULL;
  std::vector<int32_t> bt((size_t)B * W), lens(B), qsl(B + 1), sl(num_slots > 0 ? num_slots : 0);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (B > 0) {
    if (W > 0) e = hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(lens.data(), context_lens, lens.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(qsl.data(), query_start_loc, qsl.size() * 4, hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess && num_slots > 0) e = hipMemcpyAsync(sl.data(), slot_mapping, sl.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return PA_ERR_LAUNCH;
  const pa_status st = validate_host(bt.data(), lens.data(), qsl.data(), num_slots > 0 ? sl.data() : nullptr,
                                     num_slots, causal, dims);
  if (st != PA_OK || !opts) return st;
  if (opts->window < 0 || opts->shared_prefix_len < 0) return PA_ERR_SHAPE;
  return validate_shared_prefix(bt.data(), lens.data(), qsl.data(), opts->shared_prefix_len, dims);
}

}  // extern "C"
