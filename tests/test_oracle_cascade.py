"""Cascade attention needs no new oracle arithmetic: attending a shared
prefix and each request's own suffix separately and merging the two partial
results by their log-sum-exp is an exact rearrangement of attention over the
whole context (page "32. Production attention kernels", Long contexts: split
the keys, and Stretch exercises: cascade attention).  These CPU checks pin
that on shared-prefix batches: the split-and-merge oracle cut at the prefix
boundary equals the plain definition, which equals brute force."""
import torch

from oracle import attention_f64, brute_force, split_combine_f64
from workloads import make_shared_prefix


def _args(w):
    return (w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)


def test_shared_prefix_tables():
    w = make_shared_prefix(seed=1, prefix_len=8, suffix_lens=[3, 1, 6], query_lens=[1, 1, 2], num_q_heads=4,
                           num_kv_heads=2, head_dim=8, page_size=4, dtype=torch.float32)
    assert torch.equal(w.block_tables[:, :2], w.block_tables[0, :2].expand(3, 2))
    own = [set(w.block_tables[b, 2:2 + (s + 3) // 4].tolist()) for b, s in enumerate([3, 1, 6])]
    assert not (own[0] & own[1]) and not (own[0] & own[2]) and not (own[1] & own[2])
    assert w.context_lens.tolist() == [11, 9, 14]


def test_cascade_merge_equals_plain_and_brute_force():
    w = make_shared_prefix(seed=2, prefix_len=12, suffix_lens=[5, 1, 9, 3], query_lens=[1, 1, 4, 3],
                           num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=4, dtype=torch.float32)
    plain = attention_f64(*_args(w))
    brute = torch.tensor(brute_force(*_args(w)), dtype=torch.float64)
    assert torch.max(torch.abs(plain - brute)).item() <= 1e-12
    cascade = split_combine_f64(*_args(w), boundaries=[12])
    assert torch.max(torch.abs(cascade - plain)).item() <= 1e-13
    # with the prefix also cut into several ranges, as the kernels do
    cascade3 = split_combine_f64(*_args(w), boundaries=[4, 8, 12])
    assert torch.max(torch.abs(cascade3 - plain)).item() <= 1e-13


def test_cascade_with_sinks():
    w = make_shared_prefix(seed=3, prefix_len=8, suffix_lens=[4, 7], query_lens=[1, 2], num_q_heads=4,
                           num_kv_heads=1, head_dim=8, page_size=4, dtype=torch.float32)
    sk = torch.tensor([0.3, -1.0, 2.0, 0.0], dtype=torch.float64)
    plain = attention_f64(*_args(w), sinks=sk)
    cascade = split_combine_f64(*_args(w), boundaries=[8], sinks=sk)
    assert torch.max(torch.abs(cascade - plain)).item() <= 1e-13
