"""The seeded generators: determinism and the shapes of the measured workloads."""
import torch

from workloads import make, make_custom, poison_unused


def test_same_seed_same_tensors():
    a = make(1)
    b = make(1)
    for x, y in [(a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.block_tables, b.block_tables)]:
        assert torch.equal(x, y)
    c = make(1, seed=99)
    assert not torch.equal(a.q, c.q)


def test_config1_shape():
    w = make(1)
    assert w.dtype == torch.float32
    assert tuple(w.q.shape) == (1, 8, 64)
    assert tuple(w.k_pool.shape) == (64, 16, 2, 64)
    assert w.block_tables.shape == (1, 38) and w.context_lens.tolist() == [600]
    assert len(set(w.block_tables[0].tolist())) == 38          # distinct pages of a permutation
    assert w.scale == 0.125
    wp = make(1, padded_width=True)
    assert wp.block_tables.shape == (1, 48)
    assert torch.equal(wp.block_tables[0, :38], w.block_tables[0])
    assert int(wp.block_tables[0, 38:].abs().sum()) == 0


def test_config2_ragged_pool_is_exact():
    w = make(2)
    lens = w.context_lens.tolist()
    assert len(lens) == 32 and all(1 <= L <= 4096 for L in lens)
    pages = sum((L + 63) // 64 for L in lens)
    assert w.num_pages == pages
    used = []
    for b, L in enumerate(lens):
        used += w.block_tables[b, :(L + 63) // 64].tolist()
    assert sorted(used) == list(range(pages))


def test_config4_mixed_batch_layout():
    w = make(4)
    assert w.query_lens[0] == 512 and w.context_lens[0] == 1536
    assert w.query_lens[1:31] == [1] * 30
    assert all(256 <= L <= 8192 for L in w.context_lens[1:31].tolist())
    assert w.query_lens[31] == 5 and w.context_lens[31] == 2048
    assert w.num_tokens == 547 and w.table_width == 128


def test_poison_marks_exactly_the_unread_slots():
    w = make_custom(seed=1, context_lens=[5, 0, 9], query_lens=[1, 0, 2], num_q_heads=2, num_kv_heads=1,
                    head_dim=4, page_size=4, num_pages=7)
    p = poison_unused(w)
    nan = torch.isnan(p.k_pool[..., 0, 0])                  # [P, ps]
    readable = 0
    for b, L in enumerate([5, 0, 9]):
        for j in range(L):
            assert not nan[int(w.block_tables[b, j // 4]), j % 4]
            readable += 1
    assert int((~nan).sum()) == readable
