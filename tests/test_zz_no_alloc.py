"""paged_attention_noalloc: the same results as paged_attention, with the split
partials in the library's static device buffer instead of a workspace.

Two calls in a row go through the C ABI (the second with a smaller batch, so
it runs over what the first left in the buffer), each compared bit for bit
with paged_attention on the same inputs and split count, and within the
parity tolerance with the float64 oracle.  A call whose partials exceed the
buffer is refused with PA_ERR_SCRATCH_LIMIT and leaves out untouched.
"""
import ctypes

import pytest
import torch

import paged_kv_attention_amd as pa
from tests.gpu_util import TOL, check, to_dev
from workloads import make_custom, poison_unused

pytestmark = pytest.mark.gpu


def _pair(w, splits, mql):
    t = to_dev(w)
    ref = pa.paged_attention(t["q"], t["k_pool"], t["v_pool"], t["block_tables"], t["context_lens"],
                             t["query_start_loc"], w.scale, w.causal, max_query_len=mql, num_splits=splits)
    dims = pa.make_dims(t["q"], t["k_pool"], t["block_tables"], max_query_len=mql, num_splits=splits)
    code = pa.PA_BF16 if w.dtype == torch.bfloat16 else pa.PA_F32
    need = pa.workspace_size(dims, w.dtype)
    assert 0 < need <= pa.STATIC_SCRATCH_BYTES, need          # the call really uses the buffer
    out = torch.full_like(t["q"], float("nan"))
    lib = pa.load_library()
    st = lib.paged_attention_noalloc(t["q"].data_ptr(), t["k_pool"].data_ptr(), t["v_pool"].data_ptr(),
                                     t["block_tables"].data_ptr(), t["context_lens"].data_ptr(),
                                     t["query_start_loc"].data_ptr(), ctypes.c_float(w.scale), 1 if w.causal else 0,
                                     out.data_ptr(), ctypes.byref(dims), code,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == pa.PA_OK, pa.status_string(st)
    return ref.cpu(), out.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_paged_attention_twice(dtype):
    Hq, Hkv, D, ps = (32, 8, 128, 64) if dtype == torch.bfloat16 else (8, 2, 64, 16)
    # first call: ragged decodes and verification blocks, split 5 ways
    w1 = poison_unused(make_custom(seed=501, context_lens=[4000, 17, 900, 2500, 64, 1],
                                   query_lens=[1, 1, 4, 1, 3, 1], num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                   page_size=ps, dtype=dtype))
    ref1, got1 = _pair(w1, splits=5, mql=4)
    assert torch.equal(ref1, got1), "first call differs from paged_attention"
    check(w1, got1, label=f"noalloc call 1 {dtype}")
    # second call: a smaller batch with another split count, over the first call's leftovers
    w2 = poison_unused(make_custom(seed=502, context_lens=[300, 1200], query_lens=[1, 2], num_q_heads=Hq,
                                   num_kv_heads=Hkv, head_dim=D, page_size=ps, dtype=dtype))
    ref2, got2 = _pair(w2, splits=2, mql=2)
    assert torch.equal(ref2, got2), "second call differs from paged_attention"
    check(w2, got2, label=f"noalloc call 2 {dtype}")


def test_noalloc_mixed_batch_runs_in_order():
    # prefill, verification and decode tiles in one call: all launches on one stream
    w = poison_unused(make_custom(seed=503, context_lens=[700, 90, 2000, 33], query_lens=[200, 5, 1, 33],
                                  num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                                  dtype=torch.bfloat16))
    ref, got = _pair(w, splits=3, mql=200)
    assert torch.equal(ref, got)
    check(w, got, label="noalloc mixed")


def test_noalloc_refuses_calls_beyond_the_buffer():
    # 1024 sequences of 16-token steps with 32 heads and 8 splits: far beyond 32 MiB of partials
    dev = torch.device("cuda", 0)
    B, n, Hq, Hkv, D, ps = 1024, 16, 32, 8, 128, 64
    q = torch.zeros(B * n, Hq, D, dtype=torch.bfloat16, device=dev)
    k = pa.empty_pool(4, ps, Hkv, D, device=dev)
    bt = torch.zeros(B, 4, dtype=torch.int32, device=dev)
    cl = torch.full((B,), 200, dtype=torch.int32, device=dev)
    qsl = torch.arange(0, B * n + 1, n, dtype=torch.int32, device=dev)
    dims = pa.make_dims(q, k, bt, max_query_len=n, num_splits=8)
    assert pa.workspace_size(dims, torch.bfloat16) > pa.STATIC_SCRATCH_BYTES
    out = torch.full_like(q, 3.0)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attention_noalloc(q, k, k, bt, cl, qsl, out=out, max_query_len=n, num_splits=8)
    assert e.value.status == pa.PA_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
