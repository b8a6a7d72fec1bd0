"""The balanced 16-row decode launch against the float64 oracle.

A batch of one-to-a-few-token steps whose (sequence, KV head) pairs cannot
fill two workgroups per CU, over a table long enough that its splits would
hold 2048 keys or more, runs as a fixed grid of about two workgroups per
CU.  The batch's 32-key chunks are laid end to end and each wave takes
an equal run of them, cut into one piece per sequence it touches.  A piece
holding all of a sequence is written directly; the others are partials that
the combine merges (page "Attention and KV Cache", Split-KV decode; page "32.
Production attention kernels", One kernel for the whole batch and Long
contexts: split the keys).  These cases aim at the seams:
- runs much longer than the sequences, so a wave holds many pieces;
- one sequence cut into dozens of pieces;
- contexts with no key;
- sinks and a window, which only a sequence's first piece may apply;
- steps of several tokens;
- agreement with the split launch;
- repeatability.
"""
import pytest
import torch

import paged_kv_attention_amd as pa
from workloads import make_custom, poison_unused
from tests.gpu_util import run_lib, check, to_dev

pytestmark = pytest.mark.gpu


def _custom(seed, lens, qlens, Hq=32, Hkv=8, D=128, ps=64, **kw):
    return make_custom(seed=seed, context_lens=lens, query_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, page_size=ps, dtype=torch.bfloat16, **kw)


def _balanced(w):
    """Whether the call takes the balanced launch: its workspace holds slots
    b + w < B + 4 ceil(2 CUs / Hkv) (w: a wave) of partial rows plus the
    combine's map."""
    t = to_dev(w)
    d = pa.make_dims(t["q"], t["k_pool"], t["block_tables"], max_query_len=w.max_query_len)
    B, Hq, D = len(w.context_lens), w.q.shape[1], w.q.shape[2]
    Hkv = w.k_pool.shape[2]
    U = -(-2 * pa.device_cu_count() // Hkv)
    ws_tok = min(w.max_query_len, 16)
    return pa.workspace_size(d, w.dtype) == (B + 4 * U) * ws_tok * Hq * (D + 2) * 4 + B * 8


def test_many_short_sequences_per_wave():
    # one KV head: 300 pairs; a table of 128 pages gives the split rule
    # splits of 2752 keys, so the launch balances, and a wave's run of 4
    # chunks crosses several of these short sequences
    g = torch.Generator().manual_seed(5)
    lens = torch.randint(1, 100, (300,), generator=g).tolist()
    w = poison_unused(_custom(700, lens, [1] * 300, Hq=4, Hkv=1, table_width=128))
    assert _balanced(w)
    check(w, run_lib(w), label="balanced 300 short sequences")


def test_one_sequence_in_many_pieces():
    # one long sequence among short ones: it spans about a hundred waves' runs
    lens = [16000] + [5, 70, 300, 1, 900, 64, 65] * 4
    w = poison_unused(_custom(701, lens, [1] * len(lens), table_width=256))
    assert _balanced(w)
    check(w, run_lib(w), label="balanced 16000-key sequence among short ones")


def test_contexts_without_keys_are_zero():
    lens = [0, 5, 0, 700, 0, 2000, 1, 0]
    w = poison_unused(_custom(702, lens, [1] * len(lens), causal=False, table_width=512))
    assert _balanced(w)
    got = run_lib(w, out_fill=7.0)
    check(w, got, label="balanced empty contexts")
    qsl = w.query_start_loc.tolist()
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(got[qsl[b]:qsl[b + 1]]) == 0


@pytest.mark.parametrize("window", [0, 300])
def test_sinks_and_window_on_the_first_piece(window):
    lens = [1, 63, 64, 65, 700, 2048, 4096, 3000, 129, 5000]
    w = poison_unused(_custom(703, lens, [1] * len(lens), table_width=512))
    assert _balanced(w)
    sinks = (torch.randn(32, generator=torch.Generator().manual_seed(7)) * 2).to(torch.float32)
    check(w, run_lib(w, window=window, sinks=sinks), label=f"balanced window {window} sinks", window=window,
          sinks=sinks)


def test_multi_token_steps():
    # steps of 1-4 tokens at group 4: every step still fits a 16-row tile
    lens = [10, 300, 2048, 4000, 77, 1500]
    qlens = [1, 2, 4, 3, 4, 1]
    w = poison_unused(_custom(704, lens, qlens, table_width=512))
    assert _balanced(w)
    check(w, run_lib(w), label="balanced multi-token steps")


def test_agrees_with_the_split_launch_and_repeats():
    g = torch.Generator().manual_seed(9)
    lens = torch.randint(1, 16385, (32,), generator=g).tolist()
    w = poison_unused(_custom(705, lens, [1] * 32, table_width=256))
    assert _balanced(w)
    a = run_lib(w)
    b = run_lib(w)
    assert torch.equal(a, b)                       # bitwise repeatable
    check(w, a, label="balanced ragged 32")
    check(w, run_lib(w, num_splits=3), label="split launch ragged 32")
