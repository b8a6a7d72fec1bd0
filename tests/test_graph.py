"""hipGraph capture and replay of one decode step (KV write + attention) while
the sequences grow: positions, lengths, page ids and write slots live in
device buffers, so the captured launches stay valid (page "Attention kernels",
Walking the block table: a graph captured once keeps working while contexts
grow).
Every replay is checked against the float64 oracle, with eager work between
replays."""
import pytest
import torch

import paged_kv_attention_amd as pa
from oracle import attention_f64, kv_write_ref
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,splits", [(torch.bfloat16, 0), (torch.bfloat16, 3), (torch.float32, 0)])
def test_graph_replay_with_growing_contexts(dtype, splits):
    Hq, Hkv, D, ps = 8, 2, 128, 16
    lens0 = [14, 70, 1, 200]
    B, W = len(lens0), 32                       # table padded for growth (W * ps = 512 positions)
    steps = 6
    w = make_custom(seed=77, context_lens=lens0, query_lens=[1] * B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    page_size=ps, dtype=dtype, num_pages=4 * W, table_width=W)
    dev = torch.device("cuda", 0)
    gen = torch.Generator().manual_seed(5)
    # pages for future growth: each sequence gets fresh pages from the unused part of the pool
    bt = w.block_tables.clone()
    used = set(int(x) for b in range(B) for x in bt[b, :(lens0[b] + ps - 1) // ps].tolist())
    free = [pg for pg in range(4 * W) if pg not in used]
    for b in range(B):
        npg = (lens0[b] + ps - 1) // ps
        for j in range(npg, npg + 2):
            bt[b, j] = free.pop()
    k_cpu, v_cpu = w.k_pool.clone(), w.v_pool.clone()
    k_dev = pa.pool_like(k_cpu, dev)
    v_dev = pa.pool_like(v_cpu, dev)
    bt_dev = bt.to(dev)
    cl_dev = torch.zeros(B, dtype=torch.int32, device=dev)
    qsl_dev = torch.arange(B + 1, dtype=torch.int32, device=dev)
    slots_dev = torch.zeros(B, dtype=torch.int32, device=dev)
    q_dev = torch.zeros(B, Hq, D, dtype=dtype, device=dev)
    kn_dev = torch.zeros(B, Hkv, D, dtype=dtype, device=dev)
    vn_dev = torch.zeros(B, Hkv, D, dtype=dtype, device=dev)
    out = torch.zeros(B, Hq, D, dtype=dtype, device=dev)
    dims = pa.make_dims(q_dev, k_dev, bt_dev, out=out, max_query_len=1, num_splits=splits)
    ws = torch.zeros(max(pa.workspace_size(dims, dtype), 16), dtype=torch.uint8, device=dev)

    def step():
        pa.kv_cache_write(kn_dev, vn_dev, k_dev, v_dev, slots_dev)
        pa.paged_attention(q_dev, k_dev, v_dev, bt_dev, cl_dev, qsl_dev, w.scale, True, out=out, workspace=ws,
                           max_query_len=1, num_splits=splits)

    def stage(t):
        """Host-side inputs of step t: each sequence appends one token at position L-1."""
        lens = [L + t + 1 for L in lens0]
        slots = [int(bt[b, (L - 1) // ps]) * ps + (L - 1) % ps for b, L in enumerate(lens)]
        q = torch.randn(B, Hq, D, generator=gen).to(dtype)
        kn = torch.randn(B, Hkv, D, generator=gen).to(dtype)
        vn = torch.randn(B, Hkv, D, generator=gen).to(dtype)
        return lens, slots, q, kn, vn

    # warm the launch path on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # the warm-up step wrote zero rows at slot 0 of page bt[0,0]... restore the pools
    k_dev.copy_(k_cpu)
    v_dev.copy_(v_cpu)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for t in range(steps):
        lens, slots, q, kn, vn = stage(t)
        # eager updates of the device buffers between replays
        cl_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        slots_dev.copy_(torch.tensor(slots, dtype=torch.int32))
        q_dev.copy_(q)
        kn_dev.copy_(kn)
        vn_dev.copy_(vn)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        k_cpu, v_cpu = kv_write_ref(kn, vn, k_cpu, v_cpu, torch.tensor(slots, dtype=torch.int32))
        ref = attention_f64(q, k_cpu, v_cpu, bt, torch.tensor(lens, dtype=torch.int32),
                            torch.arange(B + 1, dtype=torch.int32), w.scale)
        got = out.cpu().double()
        tol = 1e-5 if dtype == torch.float32 else 2e-2
        err = torch.max(torch.abs(got - ref)).item()
        assert not torch.isnan(got).any()
        assert err <= tol, (t, err)
        # the pools on the device match the host mirror bit for bit
        assert torch.equal(k_dev.cpu(), k_cpu) and torch.equal(v_dev.cpu(), v_cpu)
