"""Float64 CPU oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module.  It imports nothing from the HIP library.

What is computed (the plain definition; every inexact input is first upcast
exactly to float64, bf16 inputs at their bf16 values):

For sequence b with ``s0 = query_start_loc[b]``, ``n = query_start_loc[b+1] - s0``
and ``L = clamp(context_lens[b], 0, W * page_size)``, query token ``t`` (flat row
``i = s0 + t``) sits at position ``pos = L - n + t``: a step's queries are the
newest positions of the sequence, and the context length already includes
them (page "32. Production attention kernels", One kernel for the whole batch,
first point after the listing; page "Attention kernels", Walking the block
table: query t at position start + t).

Query head h reads KV head ``g = h // (Hq / Hkv)`` (page "Attention and KV
Cache", Multi-head, GQA, and MQA: kv_head = q_head / n_rep).

The visible keys are ``J = {j in [0, L) : not causal or j <= pos}``; key j lives
at pool page ``block_tables[b, j // ps]``, slot ``j % ps`` (page "32. Production
attention kernels", pages are reached through the block table alone; page
"paged-attn-xpu", cache layout ``[num_blocks, block_size, num_kv_heads,
head_size]``).  With ``x_j = scale * q . k_j`` the output is
``sum_J exp(x_j - max x) v_j / sum_J exp(x_j - max x)`` (page "Attention and KV
Cache", Attention as primitive ops: scores, scale, mask, max-subtract, exp,
sum, divide, matmul), and a row with no visible key is zero (page
"paged-attn-xpu", Validation: an empty context yields zeros; page "32.
Production attention kernels": padding rows produce zeros).

Readings where the pages are silent: a length beyond the table is clamped
(page "Attention and KV Cache", Split keys, paged keys and the live length),
rows with ``pos < 0`` see nothing, and ``causal = False`` makes every ``j < L``
visible.

Two variants (page "32. Production attention kernels"):

- Sliding window (One kernel for the whole batch, the listing's window mask
  and the point on sliding windows): with ``window > 0`` a key also needs
  ``j > pos - window``, i.e. a row sees at most its last ``window``
  positions.  The same condition applies when ``causal = False`` (reading:
  the window is a lower bound on key positions, independent of the upper
  one).
- Attention sinks (Stretch exercises, attention sinks): one logit ``sink_h``
  per query head, in the units of the scaled scores, joins every softmax
  denominator and contributes no value:
  ``out = sum_J exp(x_j - M) v_j / (exp(sink_h - M) + sum_J exp(x_j - M))``
  with ``M = max(sink_h, max_J x_j)``.  A row with no visible key is still
  zero.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence

import numpy as np
import torch

__all__ = ["attention_f64", "brute_force", "split_combine_f64", "kv_write_ref"]


def _seq_meta(block_tables, context_lens, query_start_loc, page_size):
    W = int(block_tables.shape[1])
    qsl = [int(x) for x in query_start_loc.tolist()]
    lens = [int(x) for x in context_lens.tolist()]
    out = []
    for b in range(len(lens)):
        L = max(0, min(lens[b], W * page_size))
        out.append((qsl[b], qsl[b + 1] - qsl[b], L))
    return out


def _gather(pool: torch.Tensor, table_row: torch.Tensor, L: int) -> torch.Tensor:
    """Pages of one sequence as a contiguous float64 ``[L, Hkv, D]`` copy."""
    ps = pool.shape[1]
    npg = (L + ps - 1) // ps
    pages = table_row[:npg].to(torch.int64)
    g = pool.index_select(0, pages).to(torch.float64)           # [npg, ps, Hkv, D]
    return g.reshape(npg * ps, pool.shape[2], pool.shape[3])[:L]


def attention_f64(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale,
                  causal: bool = True, tokens: Optional[Iterable[int]] = None,
                  chunk: int = 1024, window: int = 0, sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gather-then-dense attention in float64.

    Follows page "paged-attn-xpu" (its validation compares against a dense
    float64 computation over the sequence's gathered pages) and the reference backend of
    page "32. Production attention kernels" (gather blocks, repeat KV heads over
    the group, dense causal attention).  Query rows are processed in chunks of
    ``chunk`` tokens only to bound memory; each row's result is the definition.

    Returns float64 ``[N, Hq, D]``.  If ``tokens`` is given only those flat
    token rows are computed; the other rows are left at zero.  ``window`` and
    ``sinks`` ([Hq] logits, or None) are the two variants of the module text.
    """
    N, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    ps = k_pool.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sc = float(scale)
    out = torch.zeros(N, Hq, D, dtype=torch.float64)
    want = None if tokens is None else sorted(set(int(t) for t in tokens))
    sk = None if sinks is None else sinks.to(torch.float64).reshape(Hq, 1)   # [Hq, 1]
    for b, (s0, n, L) in enumerate(_seq_meta(block_tables, context_lens, query_start_loc, ps)):
        if n <= 0:
            continue
        ts = list(range(n)) if want is None else [i - s0 for i in want if s0 <= i < s0 + n]
        if not ts or L == 0:
            continue                                           # no visible key: zeros
        Kb = _gather(k_pool, block_tables[b], L)               # [L, Hkv, D]
        Vb = _gather(v_pool, block_tables[b], L)
        # GQA: query head h uses KV head h // G (repeat_interleave over the group)
        Kh = Kb.repeat_interleave(G, dim=1).permute(1, 0, 2)   # [Hq, L, D]
        Vh = Vb.repeat_interleave(G, dim=1).permute(1, 0, 2)
        KhT = Kh.transpose(1, 2).contiguous()                  # [Hq, D, L]: a copy, so the products run fast
        for c0 in range(0, len(ts), chunk):
            tc = torch.tensor(ts[c0:c0 + chunk], dtype=torch.int64)
            pos = L - n + tc                                   # [T]
            hi = L if not causal else int(min(L, int(pos.max()) + 1))
            if hi <= 0:
                continue
            Q = q[s0 + tc].to(torch.float64).permute(1, 0, 2)  # [Hq, T, D]
            x = sc * torch.matmul(Q, KhT[:, :, :hi])           # [Hq, T, hi]
            j = torch.arange(hi)
            vis = j[None, :] < L
            if causal:
                vis = vis & (j[None, :] <= pos[:, None])       # [T, hi]
            if window > 0:
                vis = vis & (j[None, :] > pos[:, None] - window)
            vis = vis.unsqueeze(0).expand(Hq, -1, -1)
            x = torch.where(vis, x, torch.tensor(-math.inf, dtype=torch.float64))
            empty = ~vis.any(-1)                               # [Hq, T]
            m = x.max(-1).values
            if sk is not None:
                m = torch.where(empty, m, torch.maximum(m, sk))
            m = torch.where(empty, torch.zeros_like(m), m)
            w = torch.exp(x - m.unsqueeze(-1))                 # masked -> exp(-inf) = 0
            den = w.sum(-1)
            if sk is not None:
                den = den + torch.exp(sk - m)
            o = torch.matmul(w, Vh[:, :hi]) / torch.where(empty, torch.ones_like(den), den).unsqueeze(-1)
            o = torch.where(empty.unsqueeze(-1), torch.zeros_like(o), o)
            out[s0 + tc] = o.permute(1, 0, 2)
    return out


def brute_force(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale,
                causal: bool = True, window: int = 0, sinks=None) -> List[List[List[float]]]:
    """Scalar-loop attention with every pool address computed from strides.

    Pure Python (``math.exp``, ``math.fsum``), for tiny inputs only.  Written
    from the definition alone: for each row, list the visible keys, form each
    score as an explicit sum of products, subtract the maximum, exponentiate,
    normalise and take the weighted sum of value rows.  A sink is one more
    term of the denominator (and of the maximum) with no value row.
    """
    qa = q.to(torch.float64).contiguous()
    N, Hq, D = qa.shape
    qf = qa.reshape(-1).tolist()
    kf = k_pool.to(torch.float64).reshape(-1).tolist()
    vf = v_pool.to(torch.float64).reshape(-1).tolist()
    P, ps, Hkv, _ = k_pool.shape
    sP, sS, sH = ps * Hkv * D, Hkv * D, D                      # contiguous pool strides
    bt = block_tables.tolist()
    W = len(bt[0]) if bt else 0
    lens = context_lens.tolist()
    qsl = query_start_loc.tolist()
    rep = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(N)]
    for b in range(len(lens)):
        L = lens[b]
        if L < 0:
            L = 0
        if L > W * ps:
            L = W * ps
        n = qsl[b + 1] - qsl[b]
        for t in range(n):
            i = qsl[b] + t
            pos = L - n + t
            for h in range(Hq):
                g = h // rep
                keys = [j for j in range(L)
                        if ((not causal) or j <= pos) and (window <= 0 or j > pos - window)]
                if not keys:
                    continue
                xs = []
                for j in keys:
                    page = bt[b][j // ps]
                    base = page * sP + (j % ps) * sS + g * sH
                    dot = math.fsum(qf[(i * Hq + h) * D + d] * kf[base + d] for d in range(D))
                    xs.append(float(scale) * dot)
                extra = [] if sinks is None else [float(sinks[h])]
                mx = max(xs + extra)
                ws = [math.exp(x - mx) for x in xs]
                den = math.fsum(ws + [math.exp(e - mx) for e in extra])
                for d in range(D):
                    acc = []
                    for w, j in zip(ws, keys):
                        page = bt[b][j // ps]
                        acc.append(w * vf[page * sP + (j % ps) * sS + g * sH + d])
                    out[i][h][d] = math.fsum(acc) / den
    return out


def split_combine_f64(q, k_pool, v_pool, block_tables, context_lens, query_start_loc, scale,
                      causal: bool = True, num_splits: Optional[int] = None,
                      boundaries: Optional[Sequence[int]] = None, window: int = 0,
                      sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Split-KV attention merged by log-sum-exp weights, in float64.

    Page "32. Production attention kernels", Long contexts: split the keys.
    Each sequence's keys ``[0, L)`` are cut into ranges.  For a range s with
    visible scores x_j the partial output is the softmax-weighted average o_s
    over that range alone and ``lse_s = m_s + log sum_{j in s} exp(x_j - m_s)``;
    a range with no visible key has ``lse_s = -inf`` and weight zero.  The
    result is ``sum_s exp(lse_s - lse) o_s`` with ``lse = log sum_s exp(lse_s)``,
    and zero when every range is empty.

    ``num_splits`` cuts the sequence's pages into that many page-aligned
    ranges of ``ceil(pages / num_splits)`` pages (the split sizing of that
    page's launcher); ``boundaries`` instead gives explicit key positions
    (any cut points, page-aligned or not).  A sink enters the merge as one
    more range with ``lse = sink_h`` and a zero output; windowed keys are
    masked inside each range.
    """
    N, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    ps = k_pool.shape[1]
    G = Hq // Hkv
    sc = float(scale)
    out = torch.zeros(N, Hq, D, dtype=torch.float64)
    for b, (s0, n, L) in enumerate(_seq_meta(block_tables, context_lens, query_start_loc, ps)):
        if n <= 0 or L == 0:
            continue
        if boundaries is not None:
            cuts = sorted(set([0, L] + [c for c in boundaries if 0 < c < L]))
        else:
            S = max(1, int(num_splits or 1))
            npg = (L + ps - 1) // ps
            per = (npg + S - 1) // S
            cuts = sorted(set([min(L, s * per * ps) for s in range(S + 1)] + [L]))
        Kb = _gather(k_pool, block_tables[b], L).repeat_interleave(G, dim=1).permute(1, 0, 2)
        Vb = _gather(v_pool, block_tables[b], L).repeat_interleave(G, dim=1).permute(1, 0, 2)
        tc = torch.arange(n)
        pos = L - n + tc
        Q = q[s0 + tc].to(torch.float64).permute(1, 0, 2)      # [Hq, n, D]
        parts, lses = [], []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            j = torch.arange(lo, hi)
            x = sc * torch.matmul(Q, Kb[:, lo:hi].transpose(1, 2))     # [Hq, n, hi-lo]
            vis = (j[None, :] <= pos[:, None]) if causal else torch.ones(n, hi - lo, dtype=torch.bool)
            if window > 0:
                vis = vis & (j[None, :] > pos[:, None] - window)
            vis = vis.unsqueeze(0).expand(Hq, -1, -1)
            x = torch.where(vis, x, torch.tensor(-math.inf, dtype=torch.float64))
            empty = ~vis.any(-1)
            m = torch.where(empty, torch.zeros(()), x.max(-1).values)
            w = torch.exp(x - m.unsqueeze(-1))
            l = w.sum(-1)
            o_s = torch.matmul(w, Vb[:, lo:hi]) / torch.where(empty, torch.ones_like(l), l).unsqueeze(-1)
            lse_s = torch.where(empty, torch.tensor(-math.inf, dtype=torch.float64),
                                m + torch.log(torch.where(empty, torch.ones_like(l), l)))
            parts.append(o_s)
            lses.append(lse_s)
        if sinks is not None:
            parts.append(torch.zeros(Hq, n, D, dtype=torch.float64))
            lses.append(sinks.to(torch.float64).reshape(Hq, 1).expand(Hq, n))
        lse_all = torch.stack(lses)                             # [S, Hq, n]
        top = lse_all.max(0).values
        none = torch.isinf(top) & (top < 0)
        top = torch.where(none, torch.zeros_like(top), top)
        wts = torch.exp(lse_all - top)                          # exp(-inf) = 0 for empty ranges
        tot = wts.sum(0)
        o = sum(wts[s].unsqueeze(-1) * parts[s] for s in range(len(parts)))
        o = o / torch.where(none, torch.ones_like(tot), tot).unsqueeze(-1)
        o = torch.where(none.unsqueeze(-1), torch.zeros_like(o), o)
        out[s0 + tc] = o.permute(1, 0, 2)
    return out


def kv_write_ref(k_new, v_new, k_pool, v_pool, slot_mapping):
    """Scatter token i's K/V rows to flat pool slot ``slot_mapping[i]``.

    Slot ``s`` is page ``s // page_size``, offset ``s % page_size``; ``-1``
    writes nothing (page "Attention and KV Cache", Paged KV: the write map;
    page "32. Production attention kernels": write through slot_mapping).
    Returns new pool tensors; inputs are not modified.
    """
    kp = k_pool.clone()
    vp = v_pool.clone()
    ps = kp.shape[1]
    for i, s in enumerate(slot_mapping.tolist()):
        if s < 0:
            continue
        kp[s // ps, s % ps] = k_new[i]
        vp[s // ps, s % ps] = v_new[i]
    return kp, vp
