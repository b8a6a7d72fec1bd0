"""GPU parity of the HIP kernels with the float64 oracle, through the C ABI.

Bar: max abs error <= 1e-5 for float32 inputs and <= 2e-2 for bf16 inputs
(fp32 accumulation), no NaN or Inf in any written row.  The cases follow the
pages' own test lists: a mixed batch covering every request state, GQA at
group 4, group 3 and MHA, and several split counts (page "32. Production
attention kernels", The tests and the measurements); head sizes 64/128/256, ragged contexts spanning many pages,
split and unsplit runs of a few-hundred and a thousand-plus key context, empty contexts giving zeros and a
constant V returning the constant (page "paged-attn-xpu", Validation).
"""
import dataclasses
import sys

import pytest
import torch

import paged_kv_attention_amd as pa
from oracle import kv_write_ref
from workloads import make, make_custom, poison_unused
from tests.gpu_util import run_lib, check, check_every_row, to_dev

pytestmark = pytest.mark.gpu


def _custom(seed, lens, qlens, Hq=32, Hkv=8, D=128, ps=64, dtype=torch.bfloat16, **kw):
    return make_custom(seed=seed, context_lens=lens, query_lens=qlens, num_q_heads=Hq, num_kv_heads=Hkv,
                       head_dim=D, page_size=ps, dtype=dtype, **kw)


# ---------------------------------------------------------------- float32
@pytest.mark.parametrize("splits", [0, 1, 3, 8, 38])
def test_config1_fp32_splits(splits):
    w = poison_unused(make(1))
    check(w, run_lib(w, num_splits=splits), label=f"C1 fp32 S={splits}")


def test_config1_fp32_padded_table():
    w = poison_unused(make(1, padded_width=True))
    check(w, run_lib(w), label="C1 fp32 W=48")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_fp32_mixed_batch_head_sizes(D):
    lens = [37, 600, 1500, 1, 0, 130]
    qlens = [37, 1, 1, 1, 0, 5]
    w = poison_unused(_custom(20 + D, lens, qlens, Hq=8, Hkv=2, D=D, ps=16, dtype=torch.float32))
    check(w, run_lib(w), label=f"fp32 mixed D={D}")
    check(w, run_lib(w, num_splits=3), label=f"fp32 mixed D={D} S=3")


@pytest.mark.parametrize("D,splits", [(64, 256), (128, 86), (256, 43)])
def test_combine_second_pass_head_sizes(D, splits):
    # more splits than the combine holds in registers per pass (128 at 64
    # dims, 64 at 128, 32 at 256), float32 and bf16; 256 pages of 16 keys
    lens = [4096, 1, 700, 1500]
    for dtype in (torch.float32, torch.bfloat16):
        w = poison_unused(_custom(90 + D, lens, [1] * 4, Hq=8, Hkv=2, D=D, ps=16, dtype=dtype))
        check(w, run_lib(w, num_splits=splits), label=f"{dtype} D={D} S={splits}")


def test_fp32_mha_and_group3_not_causal():
    w = _custom(31, [70, 21], [3, 21], Hq=4, Hkv=4, D=64, ps=16, dtype=torch.float32)
    check(w, run_lib(w), label="fp32 MHA")
    w = _custom(32, [70, 21], [3, 21], Hq=6, Hkv=2, D=64, ps=32, dtype=torch.float32, causal=False)
    check(w, run_lib(w), label="fp32 G=3 non-causal")


# ---------------------------------------------------------------- bf16 decode / verify
# 11 and 19 splits: the cascade fold reads splits in groups of 8, so these
# cover whole groups followed by a partial one; 33 and 64: the combine's
# groups of threads hold up to 64 splits (128-dim heads) at once, partly and
# wholly filled (its second pass: test_combine_second_pass_head_sizes)
@pytest.mark.parametrize("splits", [0, 1, 3, 8, 11, 19, 33, 64])
def test_bf16_decode_ragged(splits):
    lens = [1, 2, 63, 64, 65, 700, 2048, 4096, 33, 129]
    w = poison_unused(_custom(40, lens, [1] * len(lens)))
    check(w, run_lib(w, num_splits=splits), label=f"bf16 decode S={splits}")


@pytest.mark.parametrize("ps", [16, 32, 128])
def test_bf16_decode_page_sizes(ps):
    lens = [5, 300, 1000, 17]
    w = poison_unused(_custom(41 + ps, lens, [1] * 4, ps=ps))
    check(w, run_lib(w), label=f"bf16 decode ps={ps}")
    check(w, run_lib(w, num_splits=3), label=f"bf16 decode ps={ps} S=3")


@pytest.mark.parametrize("D", [64, 256])
def test_bf16_decode_head_sizes(D):
    lens = [3, 500, 1500]
    w = poison_unused(_custom(50 + D, lens, [1] * 3, Hq=16, Hkv=4, D=D))
    check(w, run_lib(w), label=f"bf16 decode D={D}")


@pytest.mark.parametrize("qlens", [[2, 3, 4], [5, 1, 2], [16, 9, 1], [8, 16, 12]])
def test_bf16_verify_blocks(qlens):
    lens = [40, 300, 2049][:len(qlens)]
    w = poison_unused(_custom(60 + sum(qlens), lens, qlens))
    check(w, run_lib(w), label=f"bf16 verify {qlens}")
    check(w, run_lib(w, num_splits=8), label=f"bf16 verify {qlens} S=8")


def test_bf16_group3_and_mha():
    w = poison_unused(_custom(70, [100, 7, 1000], [1, 7, 3], Hq=6, Hkv=2))
    check(w, run_lib(w), label="bf16 G=3")
    w = poison_unused(_custom(71, [100, 70, 1000], [1, 16, 30], Hq=4, Hkv=4))
    check(w, run_lib(w), label="bf16 MHA")


# ---------------------------------------------------------------- bf16 prefill
# (128, 16/32) and (256, 32): blocks span several pages (one page id per
# 4- or 2-key group); (128, 64/128) and (256, 64/128): one page per block
@pytest.mark.parametrize("D,ps", [(128, 64), (64, 16), (256, 32), (128, 128), (128, 16), (128, 32), (256, 64),
                                  (256, 128), (256, 16)])
def test_bf16_prefill(D, ps):
    lens = [300, 700, 129]
    qlens = [300, 200, 17]
    w = poison_unused(_custom(80 + D + ps, lens, qlens, Hq=8, Hkv=2, D=D, ps=ps))
    check(w, run_lib(w), label=f"bf16 prefill D={D} ps={ps}")


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (16, 2), (4, 4)])
def test_bf16_prefill_d256_groups(Hq, Hkv):
    # 256-dim tiles hold 128 rows: 42 tokens of a 3-head group (126 rows), 16
    # tokens of an 8-head group, 128 tokens of MHA; ragged tails and a
    # non-causal sequence
    lens = [300, 190, 77]
    qlens = [300, 130, 77]
    w = poison_unused(_custom(95 + Hq, lens, qlens, Hq=Hq, Hkv=Hkv, D=256, ps=64))
    check(w, run_lib(w), label=f"bf16 prefill D=256 Hq={Hq} Hkv={Hkv}")
    w = _custom(96 + Hq, [150, 64], [150, 40], Hq=Hq, Hkv=Hkv, D=256, ps=32, causal=False)
    check(w, run_lib(w), label=f"bf16 prefill D=256 non-causal Hq={Hq}")


def test_bf16_prefill_not_causal_and_group3():
    w = _custom(90, [200, 64], [200, 40], Hq=8, Hkv=2, causal=False)
    check(w, run_lib(w), label="bf16 prefill non-causal")
    w = poison_unused(_custom(91, [260, 90], [260, 90], Hq=6, Hkv=2))
    check(w, run_lib(w), label="bf16 prefill G=3")


def test_bf16_mixed_batch_every_state():
    # mid-prefill chunk, full 16- and 21-token prompts, decodes at 70 and 130, a 5-token verify,
    # an empty sequence, and a shuffled order
    lens = [70, 400, 16, 130, 21, 0, 900]
    qlens = [1, 150, 16, 1, 21, 0, 5]
    w = poison_unused(_custom(100, lens, qlens))
    check(w, run_lib(w), label="bf16 mixed")
    check(w, run_lib(w, num_splits=3), label="bf16 mixed S=3")


# ---------------------------------------------------------------- invariants
def test_empty_and_negative_position_rows_are_zero():
    # L = 0 decode and a 3-token step over L = 1 (two tokens at negative positions)
    for dtype in (torch.float32, torch.bfloat16):
        w = poison_unused(_custom(110, [0, 1, 50], [1, 3, 1], Hq=8, Hkv=2, dtype=dtype))
        got = run_lib(w, out_fill=7.0)
        assert torch.equal(got[0:3].float(), torch.zeros_like(got[0:3].float()))
        check(w, got, label=f"zero rows {dtype}")


def test_constant_values_return_the_constant():
    for dtype in (torch.float32, torch.bfloat16):
        w = _custom(111, [600, 1500, 3], [1, 2, 3], Hq=8, Hkv=2, D=128, ps=16, dtype=dtype)
        c = torch.randn(2, 128, generator=torch.Generator().manual_seed(3)).to(dtype)
        v = w.v_pool.clone()
        v[:] = c
        w = dataclasses.replace(w, v_pool=v)
        got = run_lib(w).double()
        exp = c.double().repeat_interleave(4, dim=0)
        err = torch.max(torch.abs(got - exp)).item()
        # the weights sum to one in float32; bf16 output rounds back to the constant
        tol = 1e-6 if dtype == torch.float32 else 2 ** -8 * exp.abs().max().item()
        assert err <= tol, (dtype, err)


def test_repeated_launch_is_bitwise_identical():
    w = _custom(120, [700, 3000, 5], [1, 5, 5])
    a = run_lib(w)
    b = run_lib(w)
    assert torch.equal(a, b)
    w = _custom(121, [400, 64], [400, 1], Hq=8, Hkv=2)
    assert torch.equal(run_lib(w), run_lib(w))


def test_interleaved_pool_layout_via_strides():
    """The [P, ps, Hkv, D] storage of the pages' interface runs through the same kernels."""
    w = poison_unused(_custom(130, [500, 65, 300], [1, 5, 100], Hq=8, Hkv=2))
    check(w, run_lib(w, layout="interleaved"), label="bf16 interleaved pool")
    w = poison_unused(_custom(131, [500, 65], [1, 5], Hq=8, Hkv=2, D=64, ps=16, dtype=torch.float32))
    check(w, run_lib(w, layout="interleaved"), label="fp32 interleaved pool")
    w = poison_unused(make(2))
    check(w, run_lib(w, layout="interleaved"), label="C2 interleaved pool")


def test_kv_write_head_major_pool():
    w = _custom(132, [300], [1], Hq=8, Hkv=2)
    dev = torch.device("cuda", 0)
    kd = pa.pool_like(w.k_pool, dev, "head_major")
    vd = pa.pool_like(w.v_pool, dev, "head_major")
    g = torch.Generator().manual_seed(4)
    k_new = torch.randn(5, 2, 128, generator=g).to(torch.bfloat16)
    v_new = torch.randn(5, 2, 128, generator=g).to(torch.bfloat16)
    slots = torch.tensor([7, 64, -1, 129, 3], dtype=torch.int32)
    pa.kv_cache_write(k_new.to(dev), v_new.to(dev), kd, vd, slots.to(dev))
    torch.cuda.synchronize()
    ek, ev = kv_write_ref(k_new, v_new, w.k_pool, w.v_pool, slots)
    assert torch.equal(kd.cpu(), ek) and torch.equal(vd.cpu(), ev)


def test_length_beyond_table_is_clamped():
    w = _custom(140, [128, 64], [1, 1], Hq=8, Hkv=2, table_width=2)
    base = run_lib(w)
    w2 = dataclasses.replace(w, context_lens=torch.tensor([10 ** 6, 64], dtype=torch.int32))
    assert torch.equal(run_lib(w2), base)


# ---------------------------------------------------------------- kv write
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kv_cache_write_matches_reference(dtype):
    P, ps, Hkv, D, T = 10, 16, 4, 128, 37
    g = torch.Generator().manual_seed(5)
    k_pool = torch.randn(P, ps, Hkv, D, generator=g).to(dtype)
    v_pool = torch.randn(P, ps, Hkv, D, generator=g).to(dtype)
    k_new = torch.randn(T, Hkv, D, generator=g).to(dtype)
    v_new = torch.randn(T, Hkv, D, generator=g).to(dtype)
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int32)
    slots[3] = -1
    slots[20] = -1
    ek, ev = kv_write_ref(k_new, v_new, k_pool, v_pool, slots)
    dev = torch.device("cuda", 0)
    kd, vd = k_pool.to(dev), v_pool.to(dev)
    pa.kv_cache_write(k_new.to(dev), v_new.to(dev), kd, vd, slots.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), ek) and torch.equal(vd.cpu(), ev)


def test_write_then_attend_decode_step():
    """kv_cache_write of the step's tokens, then attention over them (the serving order)."""
    w = _custom(150, [100, 257], [1, 2], Hq=8, Hkv=2)
    t = to_dev(w)
    # rewrite the newest positions with fresh rows through the slot map
    newest = []
    for b, (L, n) in enumerate([(100, 1), (257, 2)]):
        for j in range(L - n, L):
            newest.append(int(w.block_tables[b, j // 64]) * 64 + j % 64)
    g = torch.Generator().manual_seed(9)
    k_new = torch.randn(3, 2, 128, generator=g).to(torch.bfloat16)
    v_new = torch.randn(3, 2, 128, generator=g).to(torch.bfloat16)
    slots = torch.tensor(newest, dtype=torch.int32)
    pa.kv_cache_write(k_new.cuda(), v_new.cuda(), t["k_pool"], t["v_pool"], slots.cuda())
    out = pa.paged_attention(t["q"], t["k_pool"], t["v_pool"], t["block_tables"], t["context_lens"],
                             t["query_start_loc"], w.scale)
    torch.cuda.synchronize()
    ek, ev = kv_write_ref(k_new, v_new, w.k_pool, w.v_pool, slots)
    w2 = dataclasses.replace(w, k_pool=ek, v_pool=ev)
    check(w2, out.cpu(), label="write then attend")


# ---------------------------------------------------------------- validation and errors
def test_validate_reports_bad_metadata():
    dev = torch.device("cuda", 0)
    bt = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device=dev)
    cl = torch.tensor([20, 5], dtype=torch.int32, device=dev)
    qsl = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    ok = dict(num_tokens=2, page_size=16, num_pages=4)
    assert pa.validate(bt, cl, qsl, **ok) == pa.PA_OK
    assert pa.validate(bt, torch.tensor([40, 5], dtype=torch.int32, device=dev), qsl, **ok) == pa.PA_ERR_INVALID_DATA
    assert pa.validate(torch.tensor([[0, 9], [2, 3]], dtype=torch.int32, device=dev), cl, qsl, **ok) == pa.PA_ERR_INVALID_DATA
    assert pa.validate(bt, cl, torch.tensor([0, 2, 1], dtype=torch.int32, device=dev), **ok) == pa.PA_ERR_INVALID_DATA
    assert pa.validate(bt, cl, qsl, slot_mapping=torch.tensor([3, 3], dtype=torch.int32, device=dev), **ok) == pa.PA_ERR_INVALID_DATA
    assert pa.validate(bt, cl, qsl, slot_mapping=torch.tensor([64, -1], dtype=torch.int32, device=dev), **ok) == pa.PA_ERR_INVALID_DATA
    assert pa.validate(bt, cl, qsl, slot_mapping=torch.tensor([63, -1], dtype=torch.int32, device=dev), **ok) == pa.PA_OK


def test_bad_shapes_raise_and_leave_out_untouched():
    w = _custom(160, [100], [1], Hq=8, Hkv=2)
    t = to_dev(w)
    out = torch.full_like(t["q"], 3.0)
    with pytest.raises(pa.PagedAttnError):
        # 8 query heads over 3 KV heads is not a grouping
        bad_k = torch.zeros(t["k_pool"].shape[0], 64, 3, 128, dtype=torch.bfloat16, device="cuda")
        pa.paged_attention(t["q"], bad_k, bad_k, t["block_tables"], t["context_lens"], t["query_start_loc"],
                           out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# ---------------------------------------------------------------- full-size workloads
def test_config2_full():
    w = poison_unused(make(2))
    check(w, run_lib(w), label="C2 full")


def test_config3_full():
    w = make(3)
    check(w, run_lib(w), label="C3 full")


def test_config4_full_and_shuffled():
    w = make(4)
    check(w, run_lib(w), label="C4 full")
    # shuffled sequence order: same rows, permuted batch
    B = w.num_seqs
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(4)).tolist()
    qsl = w.query_start_loc.tolist()
    q = torch.cat([w.q[qsl[b]:qsl[b + 1]] for b in perm])
    qlens = [qsl[b + 1] - qsl[b] for b in perm]
    nqsl = torch.zeros(B + 1, dtype=torch.int32)
    nqsl[1:] = torch.cumsum(torch.tensor(qlens), 0).to(torch.int32)
    w2 = dataclasses.replace(w, q=q, block_tables=w.block_tables[perm], context_lens=w.context_lens[perm],
                             query_start_loc=nqsl)
    check(w2, run_lib(w2), label="C4 shuffled")


@pytest.mark.parametrize("config", [5, 6])
def test_config5_prefill_every_row(config):
    """The 4 x 8192 causal prefills (D 128 and the D 256 variant) in the launch
    configuration the bench times: every row against the oracle, the output
    pre-filled with NaN so a row no tile writes fails."""
    w = make(config)
    got = run_lib(w, out_fill=float("nan"))
    check_every_row(w, got, label=f"C{config} every row")


def test_compact_prefill_grid_many_sequences():
    # The 64-row prefill tiles of a short prefill take a compact grid whose
    # slots each wave maps to (sequence, tile) by a scan of the step lengths,
    # 64 sequences at a time.  150 sequences (three scan chunks) with prefill
    # steps of 17-150 tokens in every chunk, among decodes and verification
    # steps: as one launch of all classes (mixed batch), and as prefill
    # alone over the same kind of spread.
    g = torch.Generator().manual_seed(31)
    qlens, lens = [], []
    for b in range(150):
        r = int(torch.randint(0, 6, (1,), generator=g))
        n = 1 if r < 3 else int(torch.randint(2, 6, (1,), generator=g)) if r == 3 else int(torch.randint(17, 151, (1,), generator=g))
        qlens.append(n)
        lens.append(n + int(torch.randint(0, 400, (1,), generator=g)))
    qlens[0], qlens[63], qlens[64], qlens[127], qlens[128], qlens[149] = 40, 17, 100, 150, 33, 64
    lens[0], lens[63], lens[64], lens[127], lens[128], lens[149] = 40, 300, 100, 500, 33, 64
    w = poison_unused(_custom(120, lens, qlens))
    got = run_lib(w, out_fill=float("nan"))
    check(w, got, label="compact prefill grid, 150 sequences, mixed")
    pre = [i for i, n in enumerate(qlens) if n > 16]
    wp = poison_unused(_custom(121, [lens[i] for i in pre], [qlens[i] for i in pre]))
    check(wp, run_lib(wp, out_fill=float("nan")), label="compact prefill grid, prefill steps only")
