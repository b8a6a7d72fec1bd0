"""CPU float64 oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Nothing in the product path may import, call or link this package.  Only the
tests (``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library: it reads the same
seeded inputs (``workloads``) and computes the plain definition of causal
grouped-query attention over a block-paged cache, in float64.

Functions (each cites the passage it follows in ``oracle/attention.py``):

* ``attention_f64``     -- gather each sequence's pages, then dense softmax
                           attention in float64 (the gather-then-dense reference
                           of page "paged-attn-xpu" and of the reference backend of
                           page "32. Production attention kernels").
* ``brute_force``       -- pure-Python scalar loops with ``math.exp`` and
                           ``math.fsum``; every pool address is computed from
                           strides.  Tiny inputs only.
* ``split_combine_f64`` -- split-KV: per-split normalised output and
                           log-sum-exp, merged with weights exp(lse_s - lse).
* ``kv_write_ref``      -- the slot-mapped scatter of new K/V rows into the pools.
* ``quantize_head_vectors``, ``kv_write_quant_ref``, ``dequantize`` (``oracle/kv_quant.py``)
                        -- the quantized cache: one float32 scale per (token,
                           KV head), int8 or fp8 E4M3 codes, optional key
                           smoothing, and the exact float64 read-back.

What pins each function (checks against something other than itself):

* ``attention_f64``: brute force on tiny batches; torch's
  ``scaled_dot_product_attention`` with an explicit bottom-right causal mask;
  two-key closed forms (both signs, causal and not); one visible key returns
  its value row; constant values; empty rows; causal independence; chunk
  positions equal shorter decodes; page permutation; GQA equals MHA with
  repeated heads; clamped lengths (``tests/test_oracle.py``); window and sink
  closed forms and reductions (``tests/test_oracle_window_sinks.py``).
* ``brute_force``: the same two-key closed forms, and agreement with the
  library special case through ``attention_f64``.
* ``split_combine_f64``: equals the unsplit result for several split counts
  and arbitrary cut points, with and without window and sinks, and at a
  shared prefix boundary (``tests/test_oracle_cascade.py``).
* ``kv_write_ref``: a hand-checked scatter with a skipped slot.
* ``quantize_head_vectors`` / ``kv_write_quant_ref`` / ``dequantize``: reconstruction
  error bounds and range edges, hand-worked E4M3 conversions, unchanged
  scores under smoothing, the printed cache sizes, and the write map
  (``tests/test_oracle_kv_quant.py``).

No function here is "parity unpinned".
"""
from .attention import attention_f64, brute_force, split_combine_f64, kv_write_ref
from .kv_quant import KV_QMAX, KV_CODE_DTYPE, quantize_head_vectors, kv_write_quant_ref, dequantize

__all__ = ["attention_f64", "brute_force", "split_combine_f64", "kv_write_ref", "KV_QMAX",
           "KV_CODE_DTYPE", "quantize_head_vectors", "kv_write_quant_ref", "dequantize"]
