"""The C-ABI library loads on a CPU-only host, exports every symbol the
header declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import paged_kv_attention_amd as pa
from paged_kv_attention_amd._lib import PaDims, PaAttnOpts

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pagedattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w ]*?[\s\*]+)?([A-Za-z_]\w*)\s*\(", text, flags=re.M))
                  - {"if", "defined"})


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    declared = _declared_functions()
    assert set(pa.EXPORTED) == set(declared), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    assert pa.status_string(pa.PA_OK) == "ok"
    for s in range(1, 8):
        assert pa.status_string(s) and pa.status_string(s) != "unknown status"
    assert pa.status_string(99) == "unknown status"


def _dims(**kw):
    d = PaDims()
    base = dict(num_seqs=2, num_tokens=2, max_query_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                page_size=64, num_pages=128, table_width=64, num_splits=0, q_stride_tok=32 * 128,
                q_stride_head=128, o_stride_tok=32 * 128, o_stride_head=128, kv_stride_page=64 * 8 * 128,
                kv_stride_slot=8 * 128, kv_stride_head=128)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def _call(d, dtype=1, scale=0.088, ptr=None, ws=None, ws_bytes=0):
    lib = pa.load_library()
    p = ptr
    return lib.paged_attention(p, p, p, p, p, p, ctypes.c_float(scale), 1, p, ws, ws_bytes, ctypes.byref(d), dtype,
                               None)


def test_argument_errors_return_status_without_launch():
    lib = pa.load_library()
    assert lib.paged_attention(None, None, None, None, None, None, 1.0, 1, None, None, 0, None, 1, None) == pa.PA_ERR_NULL
    assert _call(_dims(num_kv_heads=3)) == pa.PA_ERR_SHAPE                 # 32 % 3 != 0
    assert _call(_dims(head_dim=96)) == pa.PA_ERR_UNSUPPORTED
    assert _call(_dims(page_size=8)) == pa.PA_ERR_UNSUPPORTED
    assert _call(_dims(), dtype=7) == pa.PA_ERR_UNSUPPORTED
    assert _call(_dims(q_stride_head=100)) == pa.PA_ERR_SHAPE              # rows overlap: D not contiguous
    assert _call(_dims(kv_stride_slot=8 * 128 + 3)) == pa.PA_ERR_UNSUPPORTED   # breaks 16-byte loads
    assert _call(_dims(num_seqs=-1)) == pa.PA_ERR_SHAPE
    assert _call(_dims(), scale=float("nan")) == pa.PA_ERR_SHAPE
    assert _call(_dims()) == pa.PA_ERR_NULL                                 # valid dims, NULL buffers
    assert _call(_dims(num_seqs=0, num_tokens=0)) == pa.PA_OK              # nothing to do
    assert _call(_dims(num_q_heads=65 * 2, num_kv_heads=2, q_stride_tok=130 * 128, o_stride_tok=130 * 128)) \
        == pa.PA_ERR_UNSUPPORTED                                            # bf16 group > 64


def test_option_errors_return_status_without_launch():
    lib = pa.load_library()
    p = ctypes.c_void_p(16)

    def call(opts, d=None):
        d = d or _dims()
        return lib.paged_attention_opts(p, p, p, p, p, p, ctypes.c_float(0.088), 1, p, None, 0, ctypes.byref(d), 1,
                                        None if opts is None else ctypes.byref(opts), None)
    assert call(PaAttnOpts(-1, 0, None)) == pa.PA_ERR_SHAPE                 # negative window
    assert call(PaAttnOpts(0, 5, None)) == pa.PA_ERR_SHAPE                  # reserved field set
    assert call(PaAttnOpts(0, 0, 18)) == pa.PA_ERR_UNSUPPORTED              # sinks not 4-byte aligned
    assert call(PaAttnOpts(0, 0, None), _dims(head_dim=96)) == pa.PA_ERR_UNSUPPORTED
    assert call(PaAttnOpts(16, 0, None), _dims(num_seqs=0, num_tokens=0)) == pa.PA_OK
    # the step's new rows: all three pointers, 16-byte alignment, whole-vector strides
    o = PaAttnOpts(0, 0, None)
    o.k_new, o.v_new, o.slot_mapping, o.new_stride_tok, o.new_stride_head = 16, None, 16, 8 * 128, 128
    assert call(o) == pa.PA_ERR_NULL                                        # v_new missing
    o.v_new, o.slot_mapping = 16, None
    assert call(o) == pa.PA_ERR_NULL                                        # slot_mapping missing
    o.slot_mapping, o.k_new = 16, 24
    assert call(o) == pa.PA_ERR_UNSUPPORTED                                 # k_new not 16-byte aligned
    o.k_new, o.new_stride_head = 16, 100
    assert call(o) == pa.PA_ERR_UNSUPPORTED                                 # stride not whole 16-byte chunks
    o.new_stride_head = 64
    assert call(o) == pa.PA_ERR_SHAPE                                       # head rows overlap (stride < D)


def test_workspace_and_split_rules():
    lib = pa.load_library()
    # 64 x 8 (sequence, KV head) units already fill 2 workgroups per CU: one split, no workspace
    d = _dims(num_seqs=64, num_tokens=64)
    assert lib.pa_choose_splits(ctypes.byref(d)) == 1
    assert lib.pa_workspace_size(ctypes.byref(d), 1) == 0
    # 32 one-token decodes: three workgroups per CU when two are not filled
    d = _dims(num_seqs=32, num_tokens=32)
    cus = lib.pa_device_cu_count()
    S = lib.pa_choose_splits(ctypes.byref(d))
    assert S == (1 if 32 * 8 >= 2 * cus else min(32, -(-3 * cus // (32 * 8)), 64 // 4))
    assert lib.pa_workspace_size(ctypes.byref(d), 1) == (S * 32 * 32 * 130 * 4 if S > 1 else 0)
    # over a table of 16384 positions the splits reach 2048 keys and more:
    # the balanced launch instead, whose partials take slots b + w < 32 +
    # 4 ceil(2 CUs / 8) (w: a wave) of 32 rows each, plus two ints per sequence
    d = _dims(num_seqs=32, num_tokens=32, table_width=256, num_pages=8192)
    U = -(-2 * cus // 8)
    assert lib.pa_workspace_size(ctypes.byref(d), 1) == (32 + 4 * U) * 32 * 130 * 4 + 32 * 8
    # an explicit count wins (capped at the table width)
    d = _dims(num_splits=3)
    assert lib.pa_choose_splits(ctypes.byref(d)) == 3
    assert lib.pa_workspace_size(ctypes.byref(d), 1) == 3 * 2 * 32 * 130 * 4
    d = _dims(num_splits=500)
    assert lib.pa_choose_splits(ctypes.byref(d)) == 64


def test_kv_write_argument_errors():
    lib = pa.load_library()
    d = _dims()
    assert lib.kv_cache_write(None, None, None, None, None, 4, 1024, 128, ctypes.byref(d), 1, None) == pa.PA_ERR_NULL
    assert lib.kv_cache_write(None, None, None, None, None, 0, 1024, 128, ctypes.byref(d), 1, None) == pa.PA_OK
    assert lib.kv_cache_write(None, None, None, None, None, 4, 1024, 128, None, 1, None) == pa.PA_ERR_NULL
    assert lib.kv_cache_write(None, None, None, None, None, 4, 1024, 128, ctypes.byref(_dims(head_dim=80)), 1,
                              None) == pa.PA_ERR_UNSUPPORTED


def test_read_probe_rejects_bad_arguments_without_launch():
    lib = pa.load_library()
    sink = ctypes.c_void_p(4096)
    assert lib.pa_read_probe(None, 16, sink, 65536, None) == pa.PA_ERR_NULL
    assert lib.pa_read_probe(ctypes.c_void_p(4096), 16, None, 65536, None) == pa.PA_ERR_NULL
    assert lib.pa_read_probe(ctypes.c_void_p(4096), 20, sink, 65536, None) == pa.PA_ERR_SHAPE      # not 16-byte sized
    assert lib.pa_read_probe(ctypes.c_void_p(4104), 16, sink, 65536, None) == pa.PA_ERR_SHAPE      # not 16-byte aligned
    assert lib.pa_read_probe(ctypes.c_void_p(4096), 16, sink, 1024, None) == pa.PA_ERR_WORKSPACE   # sink too small
    assert lib.pa_read_probe(ctypes.c_void_p(4096), 0, sink, 65536, None) == pa.PA_OK              # nothing to read
