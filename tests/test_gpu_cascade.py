"""GPU parity of cascade attention (page "32. Production attention kernels",
Stretch exercises: cascade attention; Long contexts: split the keys).

Requests share a cached prefix: the prefix pass reads its K/V once for every
query token of the batch, each request attends its own suffix, and the
partials merge by log-sum-exp.  The result must equal the float64 oracle's
plain attention over each whole context, for decode and verification steps,
several head sizes and page sizes, with sinks, over an int8 cache, with
forced suffix splits, inside a captured hipGraph, and the options the
cascade cannot serve must be refused with a status."""
import pytest
import torch

import paged_kv_attention_amd as pa
from gpu_util import TOL
from oracle import attention_f64, quantize_head_vectors, dequantize
from workloads import make_shared_prefix, make_cascade_decode

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _dev(w):
    return (w.q.to(DEV), pa.pool_like(w.k_pool, DEV), pa.pool_like(w.v_pool, DEV), w.block_tables.to(DEV),
            w.context_lens.to(DEV), w.query_start_loc.to(DEV))


def _check(w, got, ref=None, label="", **kw):
    if ref is None:
        ref = attention_f64(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale, **kw)
    g = got.cpu().double()
    assert not torch.isnan(g).any() and not torch.isinf(g).any(), label
    err = torch.max(torch.abs(g - ref)).item()
    print(f"[parity] {label}: max abs err {err:.3e}", flush=True)
    assert err <= TOL[torch.bfloat16], (label, err)


def test_cascade_decode_64_requests_shared_4096_prefix():
    w = make_cascade_decode()
    q, k, v, bt, cl, qsl = _dev(w)
    assert pa.validate(bt, cl, qsl, num_tokens=w.num_tokens, page_size=64, num_pages=w.k_pool.shape[0],
                       shared_prefix_len=4096) == pa.PA_OK
    got = pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, max_query_len=1, shared_prefix_len=4096)
    torch.cuda.synchronize()
    _check(w, got, label="cascade 64 x (4096 + U{1..512})")
    plain = pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, max_query_len=1)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(plain.double() - got.double())).item() <= 2e-2


@pytest.mark.parametrize("D,ps,qlens", [(128, 64, [1, 5, 16, 2]), (64, 16, [3, 1, 1, 8]), (256, 32, [1, 2, 4, 16])])
def test_cascade_verify_blocks(D, ps, qlens):
    Hq, Hkv = (16, 4) if D == 256 else (8, 2)
    w = make_shared_prefix(seed=700 + D, prefix_len=8 * ps, suffix_lens=[40, 17, 130, 16], query_lens=qlens,
                           num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps)
    q, k, v, bt, cl, qsl = _dev(w)
    got = pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, max_query_len=max(qlens),
                             shared_prefix_len=8 * ps)
    torch.cuda.synchronize()
    _check(w, got, label=f"cascade D {D} ps {ps}")


# a 1,344-position prefix is cut into 11 key ranges (21 blocks of 64, two per
# range), so the fold and the combine also meet a partial group of 8 partials
@pytest.mark.parametrize("prefix", [1024, 1344])
@pytest.mark.parametrize("splits", [1, 3])
def test_cascade_with_sinks_and_forced_suffix_splits(splits, prefix):
    w = make_shared_prefix(seed=710, prefix_len=prefix, suffix_lens=[300, 1, 700, 64, 5], query_lens=[1, 1, 5, 2, 1],
                           num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64)
    q, k, v, bt, cl, qsl = _dev(w)
    sk = torch.randn(32, generator=torch.Generator().manual_seed(3)) * 2
    got = pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, max_query_len=5, num_splits=splits,
                             sinks=sk.to(DEV), shared_prefix_len=prefix)
    torch.cuda.synchronize()
    _check(w, got, label=f"cascade sinks splits {splits} prefix {prefix}", sinks=sk.double())


def test_cascade_over_int8_cache():
    w = make_shared_prefix(seed=720, prefix_len=2048, suffix_lens=[100, 33, 257], query_lens=[1, 4, 1],
                           num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64)
    P, ps, Hkv, D = w.k_pool.shape
    kc, ks = quantize_head_vectors(w.k_pool.reshape(P * ps, Hkv, D), "int8")
    vc, vs = quantize_head_vectors(w.v_pool.reshape(P * ps, Hkv, D), "int8")
    kc, vc, ks, vs = kc.reshape(P, ps, Hkv, D), vc.reshape(P, ps, Hkv, D), ks.reshape(P, ps, Hkv), vs.reshape(P, ps, Hkv)
    kd = pa.empty_code_pool(P, ps, Hkv, D, "int8", DEV)
    vd = pa.empty_code_pool(P, ps, Hkv, D, "int8", DEV)
    kd.copy_(kc)
    vd.copy_(vc)
    ksd, vsd = pa.empty_scale_pool(P, ps, Hkv, DEV), pa.empty_scale_pool(P, ps, Hkv, DEV)
    ksd.copy_(ks)
    vsd.copy_(vs)
    got = pa.paged_attention(w.q.to(DEV), kd, vd, w.block_tables.to(DEV), w.context_lens.to(DEV),
                             w.query_start_loc.to(DEV), w.scale, True, max_query_len=4,
                             kv_quant=pa.KvQuant("int8", ksd, vsd), shared_prefix_len=2048)
    torch.cuda.synchronize()
    ref = attention_f64(w.q, dequantize(kc, ks), dequantize(vc, vs), w.block_tables, w.context_lens,
                        w.query_start_loc, w.scale)
    _check(w, got, ref=ref, label="cascade int8")


def test_cascade_graph_replay():
    w = make_shared_prefix(seed=730, prefix_len=512, suffix_lens=[70, 3, 200], query_lens=[1, 2, 1],
                           num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64)
    q, k, v, bt, cl, qsl = _dev(w)
    out = torch.zeros_like(q)

    def call():
        pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, out=out, workspace=ws, max_query_len=2,
                           shared_prefix_len=512)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator().manual_seed(4)
    for step in range(3):
        qn = torch.randn(w.q.shape, generator=gen).to(torch.bfloat16)
        q.copy_(qn)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = attention_f64(qn, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
        _check(w, out, ref=ref, label=f"cascade graph replay {step}")


def test_cascade_refusals_and_contract():
    w = make_shared_prefix(seed=740, prefix_len=256, suffix_lens=[40, 30], query_lens=[1, 20], num_q_heads=8,
                           num_kv_heads=2, head_dim=128, page_size=64)
    q, k, v, bt, cl, qsl = _dev(w)
    with pytest.raises(pa.PagedAttnError) as e:      # a 20-token step is prefill class
        pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, max_query_len=20, shared_prefix_len=256)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
    w2 = make_shared_prefix(seed=741, prefix_len=256, suffix_lens=[40, 30], query_lens=[1, 2], num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=64)
    q, k, v, bt, cl, qsl = _dev(w2)
    with pytest.raises(pa.PagedAttnError) as e:      # with a sliding window
        pa.paged_attention(q, k, v, bt, cl, qsl, w2.scale, True, max_query_len=2, window=64, shared_prefix_len=256)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
    with pytest.raises(pa.PagedAttnError) as e:      # not a whole number of pages
        pa.paged_attention(q, k, v, bt, cl, qsl, w2.scale, True, max_query_len=2, shared_prefix_len=200)
    assert e.value.status == pa.PA_ERR_SHAPE
    n = w2.num_tokens
    assert pa.validate(bt, cl, qsl, num_tokens=n, page_size=64, num_pages=w2.k_pool.shape[0],
                       shared_prefix_len=256) == pa.PA_OK
    bad = bt.clone()
    bad[1, 2] = bad[0, 0] if int(bad[0, 0]) != int(bad[1, 2]) else int(bad[1, 2]) + 1
    assert pa.validate(bad, cl, qsl, num_tokens=n, page_size=64, num_pages=w2.k_pool.shape[0],
                       shared_prefix_len=256) == pa.PA_ERR_INVALID_DATA
