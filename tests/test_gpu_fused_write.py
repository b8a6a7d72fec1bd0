"""The step's new rows passed to paged_attention (k_new, v_new, slot_mapping)
give the pools and the output of kv_cache_write followed by paged_attention,
bit for bit (the same attention kernels read the same values), and match the
oracle over the written pools.  Covered: decode batches, where the decode
launch writes the rows itself (several splits, a sequence's new tokens cut
apart by a split boundary, padding tokens with slot -1, a sliding window);
and a mixed batch and the float32 path, where the rows are written first."""
import dataclasses

import pytest
import torch

import paged_kv_attention_amd as pa
from oracle import kv_write_ref
from workloads import make, make_custom
from tests.gpu_util import check, to_dev

pytestmark = pytest.mark.gpu


def _case(w, seed, pad_tokens=()):
    """New rows for every query token and slots at their own positions
    (-1 for the tokens in pad_tokens)."""
    g = torch.Generator().manual_seed(seed)
    N = w.q.shape[0]
    Hkv, D = w.k_pool.shape[2], w.k_pool.shape[3]
    k_new = torch.randn(N, Hkv, D, generator=g).to(w.dtype)
    v_new = torch.randn(N, Hkv, D, generator=g).to(w.dtype)
    ps = w.k_pool.shape[1]
    qsl, lens = w.query_start_loc.tolist(), w.context_lens.tolist()
    slots = []
    for b in range(len(lens)):
        n = qsl[b + 1] - qsl[b]
        for t in range(n):
            pos = lens[b] - n + t
            slots.append(int(w.block_tables[b, pos // ps]) * ps + pos % ps)
    for i in pad_tokens:
        slots[i] = -1
    return k_new, v_new, torch.tensor(slots, dtype=torch.int32)


def _both(w, k_new, v_new, slots, **kw):
    dev = torch.device("cuda", 0)
    a, b = to_dev(w), to_dev(w)
    args = dict(max_query_len=w.max_query_len, **kw)
    pa.kv_cache_write(k_new.to(dev), v_new.to(dev), a["k_pool"], a["v_pool"], slots.to(dev))
    out_a = pa.paged_attention(a["q"], a["k_pool"], a["v_pool"], a["block_tables"], a["context_lens"],
                               a["query_start_loc"], w.scale, w.causal, **args)
    out_b = pa.paged_attention(b["q"], b["k_pool"], b["v_pool"], b["block_tables"], b["context_lens"],
                               b["query_start_loc"], w.scale, w.causal, k_new=k_new.to(dev), v_new=v_new.to(dev),
                               slot_mapping=slots.to(dev), **args)
    torch.cuda.synchronize()
    assert torch.equal(a["k_pool"].cpu(), b["k_pool"].cpu()) and torch.equal(a["v_pool"].cpu(), b["v_pool"].cpu())
    assert torch.equal(out_a.cpu(), out_b.cpu())
    ek, ev = kv_write_ref(k_new, v_new, w.k_pool, w.v_pool, slots)
    assert torch.equal(b["k_pool"].cpu(), ek) and torch.equal(b["v_pool"].cpu(), ev)
    return dataclasses.replace(w, k_pool=ek, v_pool=ev), out_b.cpu()


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_decode_batch_writes_inside_the_decode_launch(splits):
    w = make_custom(seed=31, context_lens=[1, 63, 64, 65, 700, 2049, 3000, 4096], query_lens=[1] * 8,
                    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, dtype=torch.bfloat16)
    k_new, v_new, slots = _case(w, 1)
    w2, out = _both(w, k_new, v_new, slots, num_splits=splits)
    check(w2, out, label=f"fused write decode S={splits}")


def test_new_tokens_cut_apart_by_a_split_boundary_and_padding():
    # 16-key pages, 2 pages per split: positions 126..129 of the 130-token
    # sequence fall in two splits; token 1 of the first sequence is padding
    w = make_custom(seed=32, context_lens=[40, 130, 97], query_lens=[3, 4, 2], num_q_heads=16, num_kv_heads=4,
                    head_dim=128, page_size=16, dtype=torch.bfloat16, table_width=16)
    k_new, v_new, slots = _case(w, 2, pad_tokens=(1,))
    w2, out = _both(w, k_new, v_new, slots, num_splits=8)
    check(w2, out, label="fused write across splits")


def test_decode_batch_with_window():
    w = make_custom(seed=33, context_lens=[300, 1000, 77], query_lens=[1, 1, 1], num_q_heads=32, num_kv_heads=8,
                    head_dim=64, page_size=32, dtype=torch.bfloat16)
    k_new, v_new, slots = _case(w, 3)
    w2, out = _both(w, k_new, v_new, slots, window=64)
    check(w2, out, label="fused write with window", window=64)


def test_mixed_batch_writes_first():
    w = make(4)
    k_new, v_new, slots = _case(w, 4)
    w2, out = _both(w, k_new, v_new, slots)
    check(w2, out, tokens=list(range(0, 547, 7)), label="mixed batch with new rows")


def test_float32_path_writes_first():
    w = make(1)
    k_new, v_new, slots = _case(w, 5)
    w2, out = _both(w, k_new, v_new, slots, num_splits=3)
    check(w2, out, label="fp32 with new rows")
