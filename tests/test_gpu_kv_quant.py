"""GPU parity of the quantized KV cache (page "32. Production attention
kernels", Quantized KV caches and its tests: INT8 and FP8 caches match the
reference computed from what the cache stores; page "Attention kernels",
INT8 cache).

* kv_cache_write_quant produces the oracle's codes and scales bit for bit
  (integer and byte work), for int8 and fp8, bf16 and float32 inputs, with
  and without key smoothing, in both pool layouts;
* attention over quantized pools matches the float64 oracle over the
  dequantized values within the bf16 tolerance, for decode and verification
  tiles, with windows and sinks, and with NaN scales in unused slots;
* the 64 x 4096 decode in int8 and fp8 at full size."""
import dataclasses

import pytest
import torch

import paged_kv_attention_amd as pa
from gpu_util import TOL, check_every_row
from oracle import attention_f64, quantize_head_vectors, kv_write_quant_ref, dequantize
from workloads import make_custom, make

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _smooth(Hkv, D, seed=4):
    g = torch.Generator().manual_seed(seed)
    return (torch.rand(Hkv, D, generator=g) * 2.5 + 0.3).to(torch.float32)


def _quantized_cache(w, kind, smooth=None):
    """Oracle codes and scales of a workload's pools: [P, ps, Hkv, D], [P, ps, Hkv]."""
    P, ps, Hkv, D = w.k_pool.shape
    kc, ks = quantize_head_vectors(w.k_pool.reshape(P * ps, Hkv, D), kind, smooth)
    vc, vs = quantize_head_vectors(w.v_pool.reshape(P * ps, Hkv, D), kind)
    return (kc.reshape(P, ps, Hkv, D), vc.reshape(P, ps, Hkv, D), ks.reshape(P, ps, Hkv), vs.reshape(P, ps, Hkv))


def _to_dev_cache(kc, vc, ks, vs, kind, smooth=None, layout="head_major"):
    P, ps, Hkv, D = kc.shape
    kd = pa.empty_code_pool(P, ps, Hkv, D, kind, DEV, layout)
    vd = pa.empty_code_pool(P, ps, Hkv, D, kind, DEV, layout)
    kd.view(torch.uint8).copy_(kc.view(torch.uint8))
    vd.view(torch.uint8).copy_(vc.view(torch.uint8))
    ksd = pa.empty_scale_pool(P, ps, Hkv, DEV, layout)
    vsd = pa.empty_scale_pool(P, ps, Hkv, DEV, layout)
    ksd.copy_(ks)
    vsd.copy_(vs)
    kq = pa.KvQuant(kind, ksd, vsd, None if smooth is None else smooth.to(DEV))
    return kd, vd, kq


def _run(w, kd, vd, kq, **kw):
    q = w.q.to(DEV)
    out = pa.paged_attention(q, kd, vd, w.block_tables.to(DEV), w.context_lens.to(DEV), w.query_start_loc.to(DEV),
                             w.scale, w.causal, max_query_len=w.max_query_len, kv_quant=kq, **kw)
    torch.cuda.synchronize()
    return out.cpu()


def _ref(w, kc, vc, ks, vs, smooth=None, tokens=None, **kw):
    kp = dequantize(kc, ks, smooth)
    vp = dequantize(vc, vs)
    return attention_f64(w.q, kp, vp, w.block_tables, w.context_lens, w.query_start_loc, w.scale,
                         causal=w.causal, tokens=tokens, **kw)


def _check(got, ref, tokens=None, tol=TOL[torch.bfloat16], label=""):
    if tokens is not None:
        idx = torch.tensor(sorted(set(tokens)))
        got, ref = got.index_select(0, idx), ref.index_select(0, idx)
    g = got.double()
    assert not torch.isnan(g).any() and not torch.isinf(g).any(), label
    err = torch.max(torch.abs(g - ref)).item()
    print(f"[parity] {label}: max abs err {err:.3e}", flush=True)
    assert err <= tol, (label, err)
    return err


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D,layout,smooth", [(128, "head_major", False), (64, "interleaved", True),
                                             (256, "head_major", True)])
def test_quantizing_write_is_bit_exact(kind, new_dtype, D, layout, smooth):
    P, ps, Hkv, T = 12, 16, 4, 40
    g = torch.Generator().manual_seed(D + (kind == "fp8"))
    kn = (torch.randn(T, Hkv, D, generator=g) * 3).to(new_dtype)
    vn = (torch.randn(T, Hkv, D, generator=g) * 0.5).to(new_dtype)
    kn[3, 1] = 0                                           # all-zero head vector: the 1e-8 floor
    kn[5, 0, 7] = 60.0                                     # an outlier
    perm = torch.randperm(P * ps, generator=g)[:T].to(torch.int32)
    perm[[2, 9, 17]] = -1                                  # padding tokens write nothing
    sm = _smooth(Hkv, D) if smooth else None
    dt = torch.int8 if kind == "int8" else torch.float8_e4m3fn
    kc0 = torch.zeros(P, ps, Hkv, D, dtype=dt)
    ks0 = torch.full((P, ps, Hkv), -1.0)
    refs = kv_write_quant_ref(kn, vn, kc0, kc0.clone(), ks0, ks0.clone(), perm, kind, sm)
    kd, vd, kq = _to_dev_cache(kc0, kc0, ks0, ks0, kind, sm, layout)
    pa.kv_cache_write_quant(kn.to(DEV), vn.to(DEV), kd, vd, perm.to(DEV), kq)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu().view(torch.uint8), refs[0].view(torch.uint8))
    assert torch.equal(vd.cpu().view(torch.uint8), refs[1].view(torch.uint8))
    assert torch.equal(kq.k_scale.cpu(), refs[2])
    assert torch.equal(kq.v_scale.cpu(), refs[3])


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_quantized(kind, splits):
    lens = [1, 40, 100, 700, 2048, 3000, 17, 4096]
    w = make_custom(seed=600, context_lens=lens, query_lens=[1] * len(lens), num_q_heads=32, num_kv_heads=8,
                    head_dim=128, page_size=64, dtype=torch.bfloat16)
    kc, vc, ks, vs = _quantized_cache(w, kind)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind)
    got = _run(w, kd, vd, kq, num_splits=splits)
    _check(got, _ref(w, kc, vc, ks, vs), label=f"{kind} decode splits {splits}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("D,ps,layout", [(64, 16, "interleaved"), (128, 32, "head_major"), (256, 64, "head_major")])
def test_decode_and_verify_quantized_smoothed(kind, D, ps, layout):
    Hq, Hkv = (16, 4) if D == 256 else (8, 2)
    w = make_custom(seed=610 + D, context_lens=[300, 1000, 77, 5], query_lens=[5, 1, 16, 2], num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, page_size=ps, dtype=torch.bfloat16)
    sm = _smooth(Hkv, D, 7)
    kc, vc, ks, vs = _quantized_cache(w, kind, sm)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind, sm, layout)
    got = _run(w, kd, vd, kq)
    _check(got, _ref(w, kc, vc, ks, vs, sm), label=f"{kind} D {D} ps {ps} smoothed")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_quantized_with_window_and_sinks(kind):
    w = make_custom(seed=620, context_lens=[900, 2048, 33, 700], query_lens=[1, 5, 1, 12], num_q_heads=32,
                    num_kv_heads=8, head_dim=128, page_size=64, dtype=torch.bfloat16)
    kc, vc, ks, vs = _quantized_cache(w, kind)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind)
    sk = torch.randn(32, generator=torch.Generator().manual_seed(1)) * 2
    got = _run(w, kd, vd, kq, window=200, sinks=sk.to(DEV))
    _check(got, _ref(w, kc, vc, ks, vs, window=200, sinks=sk.double()), label=f"{kind} window 200 sinks")


def test_unused_scale_slots_never_reach_an_output():
    """NaN scales and arbitrary codes in every slot no sequence uses."""
    lens = [70, 130, 1]
    w = make_custom(seed=630, context_lens=lens, query_lens=[1, 3, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    page_size=64, dtype=torch.bfloat16, num_pages=12)
    kc, vc, ks, vs = _quantized_cache(w, "int8")
    used = set()
    for b, L in enumerate(lens):
        for j in range(L):
            used.add((int(w.block_tables[b, j // 64]), j % 64))
    ks_p, vs_p, kc_p, vc_p = ks.clone(), vs.clone(), kc.clone(), vc.clone()
    for pg in range(12):
        for sl in range(64):
            if (pg, sl) not in used:
                ks_p[pg, sl] = float("nan")
                vs_p[pg, sl] = float("nan")
                kc_p[pg, sl] = 127
                vc_p[pg, sl] = -127
    kd, vd, kq = _to_dev_cache(kc_p, vc_p, ks_p, vs_p, "int8")
    got = _run(w, kd, vd, kq, num_splits=2)
    _check(got, _ref(w, kc, vc, ks, vs), label="poisoned unused scales")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_decode_64x4096_quantized_full(kind):
    """The measured quantized decode, in its launch configuration, every row."""
    w = make(3)
    kc, vc, ks, vs = _quantized_cache(w, kind)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind)
    got = _run(w, kd, vd, kq)
    _check(got, _ref(w, kc, vc, ks, vs), label=f"64x4096 {kind}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("D,ps,layout,smooth", [(128, 64, "head_major", False), (64, 16, "interleaved", True),
                                                (256, 32, "head_major", True)])
def test_prefill_quantized(kind, D, ps, layout, smooth):
    Hq, Hkv = (16, 4) if D == 256 else (8, 2)
    w = make_custom(seed=640 + D, context_lens=[700, 1300, 90], query_lens=[700, 300, 90], num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, page_size=ps, dtype=torch.bfloat16)
    sm = _smooth(Hkv, D, 9) if smooth else None
    kc, vc, ks, vs = _quantized_cache(w, kind, sm)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind, sm, layout)
    got = _run(w, kd, vd, kq)
    _check(got, _ref(w, kc, vc, ks, vs, sm), label=f"{kind} prefill D {D} ps {ps} smooth {smooth}")


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_mixed_batch_quantized_window_sinks(kind):
    w = make_custom(seed=650, context_lens=[1536, 900, 2048, 33, 700], query_lens=[512, 1, 5, 1, 40],
                    num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, dtype=torch.bfloat16)
    sm = _smooth(8, 128, 11)
    kc, vc, ks, vs = _quantized_cache(w, kind, sm)
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, kind, sm)
    sk = torch.randn(32, generator=torch.Generator().manual_seed(2)) * 2
    got = _run(w, kd, vd, kq, window=300, sinks=sk.to(DEV))
    _check(got, _ref(w, kc, vc, ks, vs, sm, window=300, sinks=sk.double()), label=f"{kind} mixed window sinks")


def test_prefill_4x8192_int8_every_row():
    """The 4 x 8192 causal prefill over an int8 cache, as the bench times it:
    every row against the oracle over the dequantized cache, the output
    pre-filled with NaN so a row no tile writes fails."""
    w = make(5)
    kc, vc, ks, vs = _quantized_cache(w, "int8")
    kd, vd, kq = _to_dev_cache(kc, vc, ks, vs, "int8")
    q = w.q.to(DEV)
    out = torch.full_like(q, float("nan"))
    pa.paged_attention(q, kd, vd, w.block_tables.to(DEV), w.context_lens.to(DEV), w.query_start_loc.to(DEV),
                       w.scale, w.causal, out=out, max_query_len=w.max_query_len, kv_quant=kq)
    torch.cuda.synchronize()
    wd = dataclasses.replace(w, k_pool=dequantize(kc, ks), v_pool=dequantize(vc, vs))
    check_every_row(wd, out.cpu(), tol=TOL[torch.bfloat16], label="4x8192 int8 prefill every row")
