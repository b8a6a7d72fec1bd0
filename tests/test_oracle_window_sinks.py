"""Pins of the oracle's two variants: sliding windows and attention sinks
(page "32. Production attention kernels": the window mask of the unified
kernel and its point on sliding windows; Stretch exercises, attention sinks).

Independent checks, each aimed at a plausible mistake:

* brute force with the window condition and the sink term written out
  (off-by-one in the window edge, sink missing from the maximum or the sum);
* a windowed decode equals plain attention over a copy of the sequence that
  only holds its last ``window`` keys (window measured from the wrong end);
* window 1 returns the row's own value row; a window covering the context
  changes nothing;
* one key with a sink has the closed form ``v0 * sigmoid(x0 - sink)``; a
  sink far below the scores changes nothing, one far above drives the row to
  zero (sign of the sink);
* the split-and-merge form with the sink as one more range equals the
  unsplit result.
"""
import math

import pytest
import torch

from oracle import attention_f64, brute_force, split_combine_f64
from workloads import make_custom, Workload


def _args(w: Workload):
    return (w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)


CASES = [
    # (lens, qlens, Hq, Hkv, D, ps, causal, window)
    ([9, 13, 1, 0, 7], [5, 1, 1, 0, 3], 4, 2, 8, 4, True, 3),
    ([11, 6], [4, 6], 6, 2, 4, 2, True, 4),
    ([10, 7], [3, 2], 4, 1, 8, 4, False, 5),
    ([16, 5], [16, 1], 2, 2, 4, 4, True, 1),
    ([20], [6], 4, 2, 4, 4, True, 25),
]


def _sinks(Hq, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(Hq, generator=g, dtype=torch.float64) * 2.0


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("with_sinks", [False, True])
def test_window_and_sinks_match_brute_force(case, with_sinks):
    lens, qlens, Hq, Hkv, D, ps, causal, window = CASES[case]
    w = make_custom(seed=300 + case, context_lens=lens, query_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, page_size=ps, scale=0.41, causal=causal)
    sk = _sinks(Hq, case) if with_sinks else None
    ref = torch.tensor(brute_force(*_args(w), causal=causal, window=window,
                                   sinks=None if sk is None else sk.tolist()), dtype=torch.float64)
    got = attention_f64(*_args(w), causal=causal, window=window, sinks=sk)
    assert torch.max(torch.abs(got - ref)).item() <= 1e-12


def test_windowed_decode_equals_truncated_sequence():
    """Decode rows with window w see exactly the last w keys: copy those keys
    into a fresh pool as a sequence of length w and attend without a window."""
    lens, w_ = [37, 20, 5, 64], 12
    Hq, Hkv, D, ps = 4, 2, 8, 4
    w = make_custom(seed=11, context_lens=lens, query_lens=[1] * len(lens), num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, page_size=ps, scale=0.3)
    got = attention_f64(*_args(w), window=w_)
    B = len(lens)
    newlens = [min(L, w_) for L in lens]
    npg = [(L + ps - 1) // ps for L in newlens]
    P = sum(npg)
    kp = torch.zeros(P, ps, Hkv, D, dtype=w.k_pool.dtype)
    vp = torch.zeros_like(kp)
    bt = torch.zeros(B, max(npg), dtype=torch.int32)
    page = 0
    for b, L in enumerate(lens):
        for i in range(newlens[b]):
            j = L - newlens[b] + i                          # old key position
            src_pg, src_sl = int(w.block_tables[b, j // ps]), j % ps
            kp[page + i // ps, i % ps] = w.k_pool[src_pg, src_sl]
            vp[page + i // ps, i % ps] = w.v_pool[src_pg, src_sl]
        bt[b, :npg[b]] = torch.arange(page, page + npg[b], dtype=torch.int32)
        page += npg[b]
    ref = attention_f64(w.q, kp, vp, bt, torch.tensor(newlens, dtype=torch.int32), w.query_start_loc, w.scale)
    assert torch.max(torch.abs(got - ref)).item() <= 1e-12


def test_window_one_returns_own_value_row():
    w = make_custom(seed=12, context_lens=[9, 6], query_lens=[4, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=4, scale=0.5)
    got = attention_f64(*_args(w), window=1)
    G, ps = 2, 4
    for b, (L, n) in enumerate([(9, 4), (6, 1)]):
        s0 = int(w.query_start_loc[b])
        for t in range(n):
            pos = L - n + t
            pg, sl = int(w.block_tables[b, pos // ps]), pos % ps
            for h in range(4):
                assert torch.equal(got[s0 + t, h], w.v_pool[pg, sl, h // G].to(torch.float64))


def test_window_covering_the_context_changes_nothing():
    w = make_custom(seed=13, context_lens=[9, 30], query_lens=[9, 2], num_q_heads=4, num_kv_heads=1,
                    head_dim=8, page_size=4)
    assert torch.equal(attention_f64(*_args(w), window=30), attention_f64(*_args(w)))


def test_single_key_with_sink_closed_form():
    w = make_custom(seed=14, context_lens=[1], query_lens=[1], num_q_heads=2, num_kv_heads=1, head_dim=8,
                    page_size=4, scale=0.25)
    sk = torch.tensor([0.7, -1.3], dtype=torch.float64)
    got = attention_f64(*_args(w), sinks=sk)
    k0 = w.k_pool[int(w.block_tables[0, 0]), 0, 0].to(torch.float64)
    v0 = w.v_pool[int(w.block_tables[0, 0]), 0, 0].to(torch.float64)
    for h in range(2):
        x0 = 0.25 * float(torch.dot(w.q[0, h].to(torch.float64), k0))
        expect = v0 / (1.0 + math.exp(float(sk[h]) - x0))
        assert torch.max(torch.abs(got[0, h] - expect)).item() <= 1e-14


def test_sink_sign_and_limits():
    w = make_custom(seed=15, context_lens=[12, 7], query_lens=[3, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=4, scale=0.3)
    base = attention_f64(*_args(w))
    low = attention_f64(*_args(w), sinks=torch.full((4,), -math.inf, dtype=torch.float64))
    assert torch.equal(low, base)
    far_low = attention_f64(*_args(w), sinks=torch.full((4,), -80.0, dtype=torch.float64))
    assert torch.max(torch.abs(far_low - base)).item() <= 1e-15
    high = attention_f64(*_args(w), sinks=torch.full((4,), 80.0, dtype=torch.float64))
    assert torch.max(torch.abs(high)).item() <= 1e-25


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_split_merge_with_window_and_sinks(splits):
    w = make_custom(seed=16, context_lens=[40, 9, 0, 25], query_lens=[6, 1, 0, 25], num_q_heads=4,
                    num_kv_heads=2, head_dim=8, page_size=4, scale=0.35)
    sk = _sinks(4, 99)
    ref = attention_f64(*_args(w), window=7, sinks=sk)
    got = split_combine_f64(*_args(w), num_splits=splits, window=7, sinks=sk)
    assert torch.max(torch.abs(got - ref)).item() <= 1e-13
