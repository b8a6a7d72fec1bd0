"""GPU parity of sliding windows and attention sinks against the float64
oracle (page "32. Production attention kernels": the unified kernel's window
mask and the point on sliding windows; Stretch exercises, attention sinks).

Covers the decode, verification and prefill tiles and the float32 path, with
several split counts, windows inside and beyond the context, windows that
start mid-page and mid-chunk, sinks of both signs, and keys before every
row's window poisoned with NaN (they must not reach an output)."""
import pytest
import torch

import paged_kv_attention_amd as pa
from gpu_util import run_lib, check, check_every_row
from workloads import make_custom, make

pytestmark = pytest.mark.gpu


def _sinks(Hq, seed, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(Hq, generator=g) * scale).to(torch.float32)


def _poison_before_window(w, window):
    """Copy of w whose K/V rows before each sequence's first window start are NaN."""
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    ps = kp.shape[1]
    qsl = w.query_start_loc.tolist()
    for b, L in enumerate(w.context_lens.tolist()):
        n = qsl[b + 1] - qsl[b]
        lo = max(0, L - n - window + 1)
        for j in range(lo):
            pg = int(w.block_tables[b, j // ps])
            kp[pg, j % ps] = float("nan")
            vp[pg, j % ps] = float("nan")
    import dataclasses
    return dataclasses.replace(w, k_pool=kp, v_pool=vp)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("window,with_sinks", [(100, False), (1000, True), (5000, True), (1, False), (37, True)])
def test_bf16_decode_window_sinks(splits, window, with_sinks):
    lens = [1, 40, 100, 101, 700, 2048, 3000, 4096]
    w = make_custom(seed=500 + window, context_lens=lens, query_lens=[1] * len(lens), num_q_heads=32,
                    num_kv_heads=8, head_dim=128, page_size=64, dtype=torch.bfloat16)
    sk = _sinks(32, window) if with_sinks else None
    got = run_lib(w, num_splits=splits, window=window, sinks=sk)
    check(w, got, window=window, sinks=sk, label=f"decode window {window} splits {splits} sinks {with_sinks}")


@pytest.mark.parametrize("qlens", [[5, 1, 16], [3, 9, 2]])
def test_bf16_verify_window_sinks(qlens):
    lens = [300, 1000, 77][:len(qlens)]
    w = make_custom(seed=520, context_lens=lens, query_lens=qlens, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, dtype=torch.bfloat16)
    sk = _sinks(8, 3)
    for window in (20, 64, 129):
        got = run_lib(w, window=window, sinks=sk)
        check(w, got, window=window, sinks=sk, label=f"verify {qlens} window {window}")


@pytest.mark.parametrize("D,ps,causal", [(128, 64, True), (64, 16, True), (256, 32, True), (128, 64, False),
                                           (128, 16, True), (256, 128, True)])
@pytest.mark.parametrize("window", [100, 300, 1023])
def test_bf16_prefill_window_sinks(D, ps, causal, window):
    Hq, Hkv = (16, 4) if D == 256 else (8, 2)
    w = make_custom(seed=530 + D + window, context_lens=[1000, 700, 1500], query_lens=[1000, 300, 517],
                    num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, dtype=torch.bfloat16, causal=causal)
    sk = _sinks(Hq, 7)
    got = run_lib(w, window=window, sinks=sk)
    check(w, got, window=window, sinks=sk, label=f"prefill D {D} ps {ps} causal {causal} window {window}")


def test_bf16_mixed_batch_window_sinks():
    w = make_custom(seed=540, context_lens=[1536, 900, 2048, 33, 700], query_lens=[512, 1, 5, 1, 40],
                    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, dtype=torch.bfloat16)
    sk = _sinks(32, 8)
    for window in (64, 500):
        got = run_lib(w, window=window, sinks=sk)
        check(w, got, window=window, sinks=sk, label=f"mixed window {window}")


@pytest.mark.parametrize("splits", [0, 3])
def test_fp32_window_sinks(splits):
    w = make_custom(seed=550, context_lens=[600, 37, 1], query_lens=[4, 1, 1], num_q_heads=8, num_kv_heads=2,
                    head_dim=64, page_size=16, dtype=torch.float32, scale=0.125)
    sk = _sinks(8, 9)
    for window in (1, 50, 600):
        got = run_lib(w, num_splits=splits, window=window, sinks=sk)
        check(w, got, window=window, sinks=sk, label=f"fp32 window {window} splits {splits}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_keys_before_every_window_are_never_used(dtype):
    lens, qlens = [900, 400, 1300], [1, 6, 300]
    w = make_custom(seed=560, context_lens=lens, query_lens=qlens, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=16, dtype=dtype)
    window = 130
    pw = _poison_before_window(w, window)
    got = run_lib(pw, window=window)
    check(w, got, window=window, label=f"{dtype} poisoned before window")


def test_window_covering_context_equals_no_window_bitwise():
    w = make(2)
    a = run_lib(w)
    b = run_lib(w, window=10 ** 6)
    assert torch.equal(a, b)


def test_very_negative_sinks_change_nothing():
    w = make_custom(seed=570, context_lens=[500, 64, 1200], query_lens=[1, 5, 200], num_q_heads=8, num_kv_heads=2,
                    head_dim=128, page_size=64, dtype=torch.bfloat16)
    a = run_lib(w)
    b = run_lib(w, sinks=torch.full((8,), -1e30))
    assert torch.equal(a, b)


def _bench_sinks(Hq):
    # the bench's sink recipe: one N(0, 2^2) logit per query head, seed 777
    return torch.randn(Hq, generator=torch.Generator().manual_seed(777)) * 2.0


def test_decode_64x4096_window1024_sinks_full():
    """The measured decode variant, in its launch configuration, every row."""
    w = make(3)
    sk = _bench_sinks(w.num_q_heads)
    got = run_lib(w, window=1024, sinks=sk)
    check(w, got, window=1024, sinks=sk, label="64x4096 window 1024 sinks")


def test_prefill_4x8192_window4096_sinks_every_row():
    """The measured prefill variant, in its launch configuration: every row
    against the oracle, the output pre-filled with NaN."""
    w = make(5)
    sk = _bench_sinks(w.num_q_heads)
    got = run_lib(w, window=4096, sinks=sk, out_fill=float("nan"))
    check_every_row(w, got, window=4096, sinks=sk, label="4x8192 window 4096 sinks every row")


def _takes_balanced_launch(w, window):
    """Whether the call's plan runs its 16-row decode tiles as the balanced
    launch: only that plan's workspace ends with (B + 4 U) * t * Hq * (D + 2)
    float32 partial rows (U = ceil(2 CUs / Hkv) workgroups per KV head, t
    token slots) and two ints per sequence after the split partials."""
    import ctypes
    from paged_kv_attention_amd import _lib as L
    from gpu_util import to_dev
    t = to_dev(w)
    d = pa.make_dims(t["q"], t["k_pool"], t["block_tables"], max_query_len=w.max_query_len)
    opts = L.PaAttnOpts(int(window), 0, None, None, 0, 0)
    ws = int(L.load_library().pa_workspace_size_opts(ctypes.byref(d), L._dtype_code(w.dtype), ctypes.byref(opts)))
    B, Hq, D, Hkv = len(w.context_lens), w.q.shape[1], w.q.shape[2], w.k_pool.shape[2]
    U = -(-2 * pa.device_cu_count() // Hkv)
    row = Hq * (D + 2) * 4
    for tok in range(1, 17):
        for k in range(1, 65):
            split = (k * B * tok * row + 255) // 256 * 256
            if ws == split + (B + 4 * U) * tok * row + B * 8:
                return True
    return False


@pytest.mark.parametrize("window", [0, 11000])
def test_bf16_mixed_batch_balanced_decodes_window_sinks(window):
    # long decodes beside a prefill chunk and a verification step: one
    # launch of all tiles with the decode class as the balanced launch (its
    # splits would hold 2,048 keys or more), with and without a window that
    # cuts the first thousands of keys of every long context, and sinks
    lens = [12000, 14000, 16000, 13000, 15500, 12500, 1280, 2048, 100, 16000, 12345, 14800, 13333, 15001, 12002, 57]
    qlens = [1, 1, 1, 1, 1, 1, 256, 5, 1, 1, 1, 1, 1, 1, 1, 1]
    w = make_custom(seed=541, context_lens=lens, query_lens=qlens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    page_size=64, dtype=torch.bfloat16)
    assert _takes_balanced_launch(w, window), "batch no longer takes the balanced decode launch"
    sk = _sinks(32, 9)
    got = run_lib(w, window=window, sinks=sk, out_fill=float("nan"))
    check(w, got, window=window, sinks=sk, label=f"mixed balanced window {window}")
