"""Helpers shared by the GPU tests: run the HIP library on a workload and
compare with the float64 oracle."""
from __future__ import annotations

import sys
from typing import Iterable, Optional

import torch

import paged_kv_attention_amd as pa
from oracle import attention_f64
from workloads import Workload

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def to_dev(w: Workload, layout: str = "head_major"):
    """Device copies of a workload; pools in the given physical layout
    ("head_major": [P, Hkv, ps, D] storage, "interleaved": [P, ps, Hkv, D]),
    always passed as [P, ps, Hkv, D] views."""
    dev = torch.device("cuda", 0)
    k = pa.pool_like(w.k_pool, dev, layout)
    v = pa.pool_like(w.v_pool, dev, layout)
    return dict(q=w.q.to(dev), k_pool=k, v_pool=v, block_tables=w.block_tables.to(dev),
                context_lens=w.context_lens.to(dev), query_start_loc=w.query_start_loc.to(dev))


def run_lib(w: Workload, num_splits: int = 0, layout: str = "head_major", max_query_len: Optional[int] = None,
            out_fill: Optional[float] = None, window: int = 0, sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    t = to_dev(w, layout)
    out = None
    if out_fill is not None:
        out = torch.full_like(t["q"], out_fill)
    out = pa.paged_attention(t["q"], t["k_pool"], t["v_pool"], t["block_tables"], t["context_lens"],
                             t["query_start_loc"], w.scale, w.causal, out=out,
                             max_query_len=max_query_len if max_query_len is not None else w.max_query_len,
                             num_splits=num_splits, window=window,
                             sinks=None if sinks is None else sinks.to(torch.float32).to(t["q"].device))
    torch.cuda.synchronize()
    return out.cpu()


def covered_tokens(w: Workload):
    qsl = w.query_start_loc.tolist()
    return list(range(qsl[0], qsl[-1]))


def check(w: Workload, got: torch.Tensor, tokens: Optional[Iterable[int]] = None, tol: Optional[float] = None,
          label: str = "", window: int = 0, sinks: Optional[torch.Tensor] = None) -> float:
    tol = TOL[w.dtype] if tol is None else tol
    toks = covered_tokens(w) if tokens is None else sorted(set(tokens))
    ref = attention_f64(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale,
                        causal=w.causal, tokens=toks, window=window,
                        sinks=None if sinks is None else sinks.to(torch.float32).double())
    idx = torch.tensor(toks, dtype=torch.int64)
    g = got.index_select(0, idx).double()
    r = ref.index_select(0, idx)
    assert not torch.isnan(g).any(), f"{label}: NaN in output"
    assert not torch.isinf(g).any(), f"{label}: Inf in output"
    err = torch.max(torch.abs(g - r)).item() if g.numel() else 0.0
    print(f"[parity] {label or w.name}: max abs err {err:.3e} (tol {tol:g})", file=sys.stderr, flush=True)
    assert err <= tol, f"{label}: max abs err {err} > {tol}"
    return err
