"""Helpers shared by the GPU tests: run the HIP library on a workload and
compare with the float64 oracle."""
from __future__ import annotations

import ctypes
import dataclasses
import json
import sys
from typing import Iterable, Optional

import torch

import paged_kv_attention_amd as pa
from oracle import attention_f64
from workloads import Workload

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}

# The float64 oracle allocates large temporaries per query chunk.  Keeping
# freed host memory in the process heap (instead of returning it to the
# kernel) spares a fresh page fault per byte on every chunk; on the full-size
# prefill checks this takes a sequence from ~23 s to ~9 s of host time.
try:
    _libc = ctypes.CDLL("libc.so.6")
    _libc.mallopt(-3, 1 << 30)       # M_MMAP_THRESHOLD: blocks up to 1 GiB come from the heap
    _libc.mallopt(-1, 2 ** 31 - 1)   # M_TRIM_THRESHOLD: never hand the heap's top back
except OSError:
    pass


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
    err = log_worst_row(w, g, r, toks, label or w.name, tol)
    assert err <= tol, f"{label}: max abs err {err} > {tol}"
    return err


def log_worst_row(w: Workload, g: torch.Tensor, r: torch.Tensor, toks, label: str, tol: float) -> float:
    """Print one JSON line with the case's max abs error and its worst row:
    flat token, query head, the sequence's context length L, the largest
    |o| of the oracle's row, and the row's error.  Returns the max error."""
    if not g.numel():
        return 0.0
    row_err = torch.abs(g - r).amax(-1)                        # [tokens, Hq]
    flat = int(torch.argmax(row_err))
    ti, h = divmod(flat, row_err.shape[1])
    tok = int(toks[ti])
    qsl = w.query_start_loc.tolist()
    b = max(i for i in range(len(qsl) - 1) if qsl[i] <= tok)
    err = float(row_err.view(-1)[flat])
    rec = {"case": label, "max_abs_err": err, "tol": tol, "rows": int(row_err.numel()),
           "worst": {"token": tok, "head": h, "L": int(w.context_lens[b]), "pos": int(w.context_lens[b]) - (qsl[b + 1] - qsl[b]) + tok - qsl[b],
                     "ref_abs_max": float(r[ti, h].abs().max()), "err": err}}
    print("[parity] " + json.dumps(rec), file=sys.stderr, flush=True)
    return err


def seq_slice(w: Workload, b: int) -> Workload:
    """Sequence b of a workload alone (same pools), as a one-sequence batch."""
    qsl = w.query_start_loc.tolist()
    s0, s1 = qsl[b], qsl[b + 1]
    return dataclasses.replace(w, q=w.q[s0:s1], block_tables=w.block_tables[b:b + 1],
                               context_lens=w.context_lens[b:b + 1],
                               query_start_loc=torch.tensor([0, s1 - s0], dtype=torch.int32))


def check_every_row(w: Workload, got: torch.Tensor, label: str, tol: Optional[float] = None, window: int = 0,
                    sinks: Optional[torch.Tensor] = None, chunk: int = 128) -> float:
    """Compare every written row of `got` with the oracle, one sequence at a
    time (progress printed per sequence), after checking that no row of the
    whole output holds NaN or Inf: run with an output pre-filled with NaN, a
    row no tile wrote fails here."""
    tol = TOL[w.dtype] if tol is None else tol
    assert not torch.isnan(got).any(), f"{label}: NaN in output (a row was not written)"
    assert not torch.isinf(got).any(), f"{label}: Inf in output"
    qsl = w.query_start_loc.tolist()
    worst = 0.0
    for b in range(w.num_seqs):
        if qsl[b + 1] == qsl[b]:
            continue
        ws = seq_slice(w, b)
        ref = attention_f64(ws.q, ws.k_pool, ws.v_pool, ws.block_tables, ws.context_lens, ws.query_start_loc,
                            ws.scale, causal=ws.causal, chunk=chunk, window=window,
                            sinks=None if sinks is None else sinks.to(torch.float32).double())
        g = got[qsl[b]:qsl[b + 1]].double()
        err = log_worst_row(w, g, ref, list(range(qsl[b], qsl[b + 1])), f"{label} seq {b}", tol)
        worst = max(worst, err)
        assert err <= tol, f"{label} seq {b}: max abs err {err} > {tol}"
    return worst
