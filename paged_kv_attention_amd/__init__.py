"""Paged KV attention for MI355X (gfx950): hand-written HIP kernels behind a C ABI.

The public functions marshal torch tensors into ``libpagedattn.so``:

* ``paged_attention`` -- causal GQA attention of a flattened ragged batch of
  query tokens (decode, verify blocks and prefill chunks) over block-paged K/V;
* ``paged_attention_noalloc`` -- the same call with the split partials in the
  library's static device buffer, for callers that cannot allocate;
* ``kv_cache_write`` -- scatter new K/V rows into the pools through a slot map;
* ``workspace_size`` / ``choose_splits`` / ``validate`` -- planning and checks;
* ``read_probe`` -- a streaming read of a device buffer (the HBM read ceiling
  the benchmark compares the decode kernel with).
"""
from ._lib import (PaDims, PagedAttnError, LIB_PATH, EXPORTED, load_library, paged_attention, kv_cache_write,
                   paged_attention_noalloc, STATIC_SCRATCH_BYTES, PA_ERR_SCRATCH_LIMIT,
                   kv_cache_write_quant, KvQuant, empty_code_pool, empty_scale_pool,
                   workspace_size, choose_splits, validate, make_dims, status_string, device_cu_count, empty_pool, pool_like,
                   read_probe, READ_PROBE_SINK_BYTES,
                   PA_F32, PA_BF16, PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH,
                   PA_ERR_INVALID_DATA)

__all__ = ["PaDims", "PagedAttnError", "LIB_PATH", "EXPORTED", "load_library", "paged_attention", "kv_cache_write",
           "paged_attention_noalloc", "STATIC_SCRATCH_BYTES",
           "kv_cache_write_quant", "KvQuant", "empty_code_pool", "empty_scale_pool",
           "workspace_size", "choose_splits", "validate", "make_dims", "status_string", "device_cu_count",
           "empty_pool", "pool_like", "read_probe", "READ_PROBE_SINK_BYTES"]
