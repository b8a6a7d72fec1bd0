"""Pins of the float64 oracle against things other than itself.

Every test here runs on the CPU.  Each pin is chosen so that a plausible
mistake in the oracle (a dropped scale, a wrong sign, the wrong KV head, an
off-by-one in the causal position, a wrong page index, a transposed operand)
fails at least one of them:

* brute force (pure-Python scalar loops, every address from strides);
* a library special case (torch's scaled_dot_product_attention in float64 on
  the gathered, head-repeated K/V with an explicit bottom-right causal mask);
* closed forms (two keys with known softmax weights; one key returns its V);
* invariants (constant V, empty context, split invariance, causal
  independence of later keys, page permutation, GQA = repeated-head MHA,
  positions of a chunk = decodes at shorter lengths).
"""
import math
import random

import pytest
import torch

from oracle import attention_f64, brute_force, split_combine_f64, kv_write_ref
from workloads import make_custom, poison_unused, Workload
import dataclasses


def _args(w: Workload):
    return (w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)


TINY = [
    # (lens, qlens, Hq, Hkv, D, ps, causal)
    ([5, 9, 1, 0, 7], [5, 1, 1, 0, 3], 4, 2, 8, 4, True),     # prefill, decode, L=1, empty, verify
    ([6, 11, 3], [2, 4, 3], 6, 2, 4, 2, True),                 # group 3, page size 2
    ([4, 13], [4, 1], 2, 2, 8, 4, True),                      # MHA
    ([7, 10], [3, 2], 4, 1, 8, 4, False),                     # MQA, not causal
    ([12], [12], 4, 2, 8, 4, True),                           # whole prompt as one chunk
    ([20, 3], [1, 3], 8, 2, 4, 4, True),                      # 20 keys over 5 pages
]


@pytest.mark.parametrize("case", range(len(TINY)))
def test_matches_brute_force(case):
    lens, qlens, Hq, Hkv, D, ps, causal = TINY[case]
    w = make_custom(seed=100 + case, context_lens=lens, query_lens=qlens, num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, page_size=ps, num_pages=sum((L + ps - 1) // ps for L in lens) + 3,
                    scale=0.37, causal=causal)
    ref = torch.tensor(brute_force(*_args(w), causal=causal), dtype=torch.float64)
    got = attention_f64(*_args(w), causal=causal)
    assert got.shape == ref.shape
    assert torch.max(torch.abs(got - ref)).item() <= 1e-12


def test_matches_brute_force_bf16_values():
    """bf16 inputs are used at their bf16 values, exactly upcast."""
    w = make_custom(seed=7, context_lens=[9, 4], query_lens=[2, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=4, dtype=torch.bfloat16)
    ref = torch.tensor(brute_force(*_args(w)), dtype=torch.float64)
    got = attention_f64(*_args(w))
    assert torch.max(torch.abs(got - ref)).item() <= 1e-12


def test_matches_sdpa_with_bottom_right_mask():
    """Library special case: gather, repeat KV heads, SDPA in float64."""
    lens, qlens = [40, 17, 64, 5], [40, 3, 1, 5]
    Hq, Hkv, D, ps = 8, 2, 16, 8
    w = make_custom(seed=11, context_lens=lens, query_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, page_size=ps, scale=0.21)
    got = attention_f64(*_args(w))
    qsl = w.query_start_loc.tolist()
    G = Hq // Hkv
    for b, (L, n) in enumerate(zip(lens, qlens)):
        npg = (L + ps - 1) // ps
        pages = w.block_tables[b, :npg].long()
        K = w.k_pool[pages].reshape(npg * ps, Hkv, D)[:L].double()
        V = w.v_pool[pages].reshape(npg * ps, Hkv, D)[:L].double()
        Kr = K.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        Vr = V.repeat_interleave(G, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        Q = w.q[qsl[b]:qsl[b + 1]].double().permute(1, 0, 2).unsqueeze(0).contiguous()
        t = torch.arange(n)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - n + t)                 # bottom-right aligned causal mask
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, attn_mask=mask, scale=w.scale)
        assert torch.max(torch.abs(got[qsl[b]:qsl[b + 1]] - ref[0].permute(1, 0, 2))).item() <= 1e-12


def test_closed_form_two_keys():
    """Two keys with scores 0 and 1: weights 1/(1+e) and e/(1+e)."""
    # D=2, one head, page size 2, a 2-token prompt (n = L = 2), scale 1/2.
    q = torch.tensor([[[7.0, -3.0]], [[2.0, 0.0]]], dtype=torch.float32)
    k = torch.zeros(1, 2, 1, 2)
    v = torch.zeros(1, 2, 1, 2)
    k[0, 0, 0] = torch.tensor([0.0, 0.0])
    k[0, 1, 0] = torch.tensor([1.0, 0.0])
    v[0, 0, 0] = torch.tensor([4.0, 0.0])
    v[0, 1, 0] = torch.tensor([0.0, 8.0])
    bt = torch.zeros(1, 1, dtype=torch.int32)
    lens = torch.tensor([2], dtype=torch.int32)
    qsl = torch.tensor([0, 2], dtype=torch.int32)
    out = attention_f64(q, k, v, bt, lens, qsl, 0.5)
    e = math.e
    # token 0 sits at position 0 and sees key 0 only: its V row exactly
    assert out[0, 0].tolist() == [4.0, 0.0]
    # token 1 sees both keys; score of key 1 is 0.5 * (2*1 + 0*0) = 1
    assert abs(out[1, 0, 0].item() - 4.0 / (1.0 + e)) <= 1e-15
    assert abs(out[1, 0, 1].item() - 8.0 * e / (1.0 + e)) <= 1e-14
    # a negative score flips the weights: q = [-2, 0] gives e^-1
    q2 = q.clone()
    q2[1, 0] = torch.tensor([-2.0, 0.0])
    out2 = attention_f64(q2, k, v, bt, lens, qsl, 0.5)
    assert abs(out2[1, 0, 0].item() - 4.0 * e / (1.0 + e)) <= 1e-14
    # not causal: token 0 also sees key 1 (score 0.5 * 7 * 1 = 3.5 vs 0)
    out3 = attention_f64(q, k, v, bt, lens, qsl, 0.5, causal=False)
    w1 = math.exp(3.5) / (1.0 + math.exp(3.5))
    assert abs(out3[0, 0, 1].item() - 8.0 * w1) <= 1e-13
    # the scalar-loop oracle meets the same closed forms
    bf = brute_force(q, k, v, bt, lens, qsl, 0.5)
    assert bf[0][0] == [4.0, 0.0]
    assert abs(bf[1][0][0] - 4.0 / (1.0 + e)) <= 1e-15 and abs(bf[1][0][1] - 8.0 * e / (1.0 + e)) <= 1e-14
    assert abs(brute_force(q2, k, v, bt, lens, qsl, 0.5)[1][0][0] - 4.0 * e / (1.0 + e)) <= 1e-14
    assert abs(brute_force(q, k, v, bt, lens, qsl, 0.5, causal=False)[0][0][1] - 8.0 * w1) <= 1e-13


def test_single_key_returns_its_value_row():
    w = make_custom(seed=3, context_lens=[1, 1, 17], query_lens=[1, 1, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=16, page_size=16)
    out = attention_f64(*_args(w))
    for b in range(2):
        page = int(w.block_tables[b, 0])
        for h in range(4):
            assert torch.equal(out[b, h], w.v_pool[page, 0, h // 2].double())


def test_constant_values_return_the_constant():
    w = make_custom(seed=4, context_lens=[33, 70], query_lens=[5, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=16)
    c = torch.randn(2, 8, generator=torch.Generator().manual_seed(0))
    v = w.v_pool.clone()
    v[:] = c                                         # every slot of KV head g holds c[g]
    w = dataclasses.replace(w, v_pool=v)
    out = attention_f64(*_args(w))
    for h in range(4):
        assert torch.max(torch.abs(out[:, h] - c[h // 2].double())).item() <= 1e-14


def test_empty_rows_are_exact_zeros():
    # L = 0, and a 3-token step over L = 1 (tokens 0, 1 sit at negative positions)
    w = make_custom(seed=5, context_lens=[0, 1, 6], query_lens=[2, 3, 1], num_q_heads=2, num_kv_heads=1,
                    head_dim=4, page_size=4)
    w = poison_unused(w)
    out = attention_f64(*_args(w))
    assert not torch.isnan(out).any()
    assert torch.equal(out[0:2], torch.zeros_like(out[0:2]))
    assert torch.equal(out[2:4], torch.zeros_like(out[2:4]))
    assert not torch.equal(out[4], torch.zeros_like(out[4]))


@pytest.mark.parametrize("splits", [1, 3, 8, 0])
def test_split_combine_matches_unsplit(splits):
    lens, qlens, ps = [600, 1500, 37, 0, 64], [1, 4, 37, 0, 1], 16
    w = make_custom(seed=12, context_lens=lens, query_lens=qlens, num_q_heads=8, num_kv_heads=2, head_dim=16,
                    page_size=ps)
    ref = attention_f64(*_args(w))
    S = splits if splits else max((L + ps - 1) // ps for L in lens)     # 0: one page per split
    got = split_combine_f64(*_args(w), num_splits=S)
    assert torch.max(torch.abs(got - ref)).item() <= 1e-13


def test_split_points_anywhere():
    w = make_custom(seed=13, context_lens=[300, 45], query_lens=[3, 45], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=16)
    ref = attention_f64(*_args(w))
    rng = random.Random(0)
    for _ in range(4):
        cuts = sorted(rng.sample(range(1, 300), 7))
        got = split_combine_f64(*_args(w), boundaries=cuts)
        assert torch.max(torch.abs(got - ref)).item() <= 1e-13


def test_causal_rows_ignore_later_keys_and_unused_slots():
    lens, qlens, ps = [50, 23], [20, 1], 8
    w = make_custom(seed=14, context_lens=lens, query_lens=qlens, num_q_heads=4, num_kv_heads=2, head_dim=8,
                    page_size=ps, num_pages=16)
    base = attention_f64(*_args(w))
    # NaN in every slot no sequence may read changes nothing, bit for bit
    wp = poison_unused(w)
    assert torch.equal(attention_f64(*_args(wp)), base)
    # perturb keys/values at positions 40..49 of sequence 0: tokens at pos < 40 are untouched
    k, v = w.k_pool.clone(), w.v_pool.clone()
    for j in range(40, 50):
        page = int(w.block_tables[0, j // ps])
        k[page, j % ps] += 5.0
        v[page, j % ps] -= 3.0
    out = attention_f64(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    n, L = 20, 50
    for t in range(n):
        pos = L - n + t
        if pos < 40:
            assert torch.equal(out[t], base[t])
        else:
            assert not torch.equal(out[t], base[t])
    assert torch.equal(out[20], base[20])            # the other sequence


def test_positions_of_a_chunk_equal_shorter_decodes():
    L, n, ps = 45, 6, 8
    w = make_custom(seed=15, context_lens=[L], query_lens=[n], num_q_heads=4, num_kv_heads=2, head_dim=8,
                    page_size=ps)
    chunk = attention_f64(*_args(w))
    for t in range(n):
        dec = attention_f64(w.q[t:t + 1], w.k_pool, w.v_pool, w.block_tables,
                            torch.tensor([L - n + t + 1], dtype=torch.int32),
                            torch.tensor([0, 1], dtype=torch.int32), w.scale)
        assert torch.max(torch.abs(dec[0] - chunk[t])).item() <= 1e-14


def test_page_permutation_is_invisible():
    w = make_custom(seed=16, context_lens=[70, 33], query_lens=[4, 1], num_q_heads=4, num_kv_heads=2,
                    head_dim=8, page_size=16, num_pages=12)
    base = attention_f64(*_args(w))
    perm = torch.randperm(12, generator=torch.Generator().manual_seed(1))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(12)
    k2 = w.k_pool[perm]                  # new page p holds old page perm[p]
    v2 = w.v_pool[perm]
    bt2 = inv[w.block_tables.long()].to(torch.int32)
    out = attention_f64(w.q, k2, v2, bt2, w.context_lens, w.query_start_loc, w.scale)
    assert torch.equal(out, base)


def test_gqa_equals_mha_with_repeated_heads():
    w = make_custom(seed=17, context_lens=[29, 64], query_lens=[3, 1], num_q_heads=6, num_kv_heads=2,
                    head_dim=8, page_size=16)
    gqa = attention_f64(*_args(w))
    k = w.k_pool.repeat_interleave(3, dim=2)
    v = w.v_pool.repeat_interleave(3, dim=2)
    mha = attention_f64(w.q, k, v, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    assert torch.equal(gqa, mha)
    # and the mapping is the contiguous group h // G, not h % Hkv
    k_bad = torch.cat([w.k_pool] * 3, dim=2)
    v_bad = torch.cat([w.v_pool] * 3, dim=2)
    bad = attention_f64(w.q, k_bad, v_bad, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    assert not torch.equal(gqa, bad)


def test_length_beyond_table_is_clamped():
    w = make_custom(seed=18, context_lens=[32], query_lens=[1], num_q_heads=2, num_kv_heads=1, head_dim=4,
                    page_size=16, table_width=2)
    base = attention_f64(*_args(w))
    over = attention_f64(w.q, w.k_pool, w.v_pool, w.block_tables, torch.tensor([999], dtype=torch.int32),
                         w.query_start_loc, w.scale)
    assert torch.equal(base, over)


def test_kv_write_reference():
    P, ps, Hkv, D = 3, 4, 2, 4
    k_pool = torch.zeros(P, ps, Hkv, D)
    v_pool = torch.zeros(P, ps, Hkv, D)
    k_new = torch.arange(3 * Hkv * D, dtype=torch.float32).reshape(3, Hkv, D) + 1
    v_new = -k_new
    kp, vp = kv_write_ref(k_new, v_new, k_pool, v_pool, torch.tensor([9, -1, 0], dtype=torch.int32))
    assert torch.equal(kp[2, 1], k_new[0]) and torch.equal(vp[2, 1], v_new[0])
    assert torch.equal(kp[0, 0], k_new[2]) and torch.equal(vp[0, 0], v_new[2])
    assert int((kp != 0).sum()) == 2 * Hkv * D
    assert torch.equal(k_pool, torch.zeros_like(k_pool))      # inputs untouched
