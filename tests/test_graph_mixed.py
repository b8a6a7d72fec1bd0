"""hipGraph capture of a mixed batch whose launches run on forked side streams
(decode tiles, a verification block and a prefill chunk), replayed with new
query values between replays and checked against the float64 oracle each
time; also eager repeats of the same call, which must be bit-identical
(page "32. Production attention kernels", One kernel for the whole batch; page
"Attention kernels", Walking the block table)."""
import pytest
import torch

import paged_kv_attention_amd as pa
from oracle import attention_f64
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _mixed(seed):
    # decodes, a 5-token verification block and a 100-token prefill chunk over a prefix
    return make_custom(seed=seed, context_lens=[300, 1, 777, 2048, 160], query_lens=[1, 1, 5, 1, 100],
                       num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, dtype=torch.bfloat16)


def test_mixed_batch_eager_repeat_is_bitwise_stable():
    w = _mixed(31)
    dev = torch.device("cuda", 0)
    q = w.q.to(dev)
    k = pa.pool_like(w.k_pool, dev)
    v = pa.pool_like(w.v_pool, dev)
    bt, cl, qsl = w.block_tables.to(dev), w.context_lens.to(dev), w.query_start_loc.to(dev)
    outs = []
    for _ in range(3):
        out = torch.full_like(q, float("nan"))
        pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, out=out, max_query_len=w.max_query_len)
        outs.append(out)
    torch.cuda.synchronize()
    ref = attention_f64(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    assert torch.max(torch.abs(outs[0].cpu().double() - ref)).item() <= 2e-2
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_mixed_batch_graph_replay():
    w = _mixed(32)
    dev = torch.device("cuda", 0)
    q_dev = w.q.to(dev)
    k = pa.pool_like(w.k_pool, dev)
    v = pa.pool_like(w.v_pool, dev)
    bt, cl, qsl = w.block_tables.to(dev), w.context_lens.to(dev), w.query_start_loc.to(dev)
    out = torch.zeros_like(q_dev)
    dims = pa.make_dims(q_dev, k, bt, out=out, max_query_len=w.max_query_len)
    ws = torch.zeros(max(pa.workspace_size(dims, torch.bfloat16), 16), dtype=torch.uint8, device=dev)

    def call():
        pa.paged_attention(q_dev, k, v, bt, cl, qsl, w.scale, True, out=out, workspace=ws,
                           max_query_len=w.max_query_len)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                   # creates the side streams outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(9)
    for step in range(4):
        qn = torch.randn(w.q.shape, generator=gen).to(torch.bfloat16)
        q_dev.copy_(qn)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = attention_f64(qn, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
        got = out.cpu().double()
        assert not torch.isnan(got).any(), step
        assert torch.max(torch.abs(got - ref)).item() <= 2e-2, step
        # an eager call between replays gives the same bits
        eager = torch.zeros_like(out)
        pa.paged_attention(q_dev, k, v, bt, cl, qsl, w.scale, True, out=eager, workspace=ws,
                           max_query_len=w.max_query_len)
        torch.cuda.synchronize()
        assert torch.equal(eager, out), step
