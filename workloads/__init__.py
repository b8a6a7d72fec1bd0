"""Seeded synthetic inputs for paged KV attention.

This module only draws and lays out inputs: context lengths, block tables, query
start offsets, q, and the K/V page pools.  It holds none of the attention
arithmetic, so both the float64 oracle (``oracle/``) and the HIP library
(``paged_kv_attention_amd``) can be fed from it without sharing any of the
method's code.

Shapes follow the workloads the pages describe:

* the fp32 single-sequence decode of paged-attn-xpu's validation (8 query heads
  over 2 KV heads, head size 64, contexts of 600; page "paged-attn-xpu",
  Validation),
* Qwen3-8B-shaped decode (32 query heads, 8 KV heads, head dim 128, 64 requests
  at 4,096 tokens; page "32. Production attention kernels", What the reference
  backend costs),
* the mixed flattened batch of that page (a 512-token prefill chunk, 30 decode
  tokens and a 5-token verification block; One kernel for the whole batch),
* and long causal prefill (page "Attention kernels", Prefill and Open questions).

Draw order is fixed so a seed reproduces every tensor bit for bit:
(1) context lengths, (2) pool permutation, (3) q, (4) k_pool, (5) v_pool.
Values are float32 N(0, 1) draws cast (round-to-nearest-even) to the
workload's dtype.  Pool layout is ``[num_pages, page_size, num_kv_heads,
head_dim]`` and block tables are int32, zero-padded to the table width.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

__all__ = ["Workload", "make", "make_custom", "poison_unused", "CONFIG_NAMES"]


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    q: torch.Tensor              # [N, Hq, D]
    k_pool: torch.Tensor         # [P, ps, Hkv, D]
    v_pool: torch.Tensor         # [P, ps, Hkv, D]
    block_tables: torch.Tensor   # [B, W] int32
    context_lens: torch.Tensor   # [B] int32 (includes the step's new tokens)
    query_start_loc: torch.Tensor  # [B + 1] int32
    scale: float                 # float32-representable
    causal: bool = True

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def page_size(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def table_width(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def query_lens(self) -> List[int]:
        qsl = self.query_start_loc.tolist()
        return [qsl[i + 1] - qsl[i] for i in range(len(qsl) - 1)]

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return max(ql) if ql else 0


CONFIG_NAMES = {
    1: "fp32 single-sequence decode: 8/2 heads, D 64, page 16, ctx 600",
    2: "bf16 ragged decode: 32 seqs, 32/8 heads, D 128, page 64, ctx U{1..4096}",
    3: "bf16 decode 64 seqs x 4096 ctx, 32/8 heads, D 128, page 64",
    4: "bf16 mixed batch: 512-token chunk over 1024 prefix + 30 decodes + 5-token verify",
    5: "bf16 causal prefill 4 x 8192, 32/8 heads, D 128, page 64",
    6: "bf16 causal prefill 4 x 8192, 16/4 heads, D 256, page 64",
}


def _f32(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).item())


def _draw(gen: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def _tables_from_perm(perm: torch.Tensor, pages_per_seq: List[int], width: int) -> torch.Tensor:
    bt = torch.zeros(len(pages_per_seq), width, dtype=torch.int32)
    off = 0
    for b, npg in enumerate(pages_per_seq):
        assert npg <= width, (npg, width)
        bt[b, :npg] = perm[off:off + npg].to(torch.int32)
        off += npg
    return bt


def make_custom(*, seed: int, context_lens: List[int], query_lens: List[int], num_q_heads: int,
                num_kv_heads: int, head_dim: int, page_size: int, dtype: torch.dtype = torch.float32,
                num_pages: Optional[int] = None, table_width: Optional[int] = None,
                scale: Optional[float] = None, causal: bool = True, name: str = "custom",
                shuffle_pool: bool = True) -> Workload:
    """Build a workload with explicit per-sequence lengths.

    The pool holds ``num_pages`` pages (default: exactly the pages the sequences
    need).  Each sequence's pages are a slice of one random permutation of the
    pool, so consecutive logical pages sit at scattered physical pages.
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    B = len(context_lens)
    assert len(query_lens) == B
    pages_per_seq = [(max(L, 0) + page_size - 1) // page_size for L in context_lens]
    need = sum(pages_per_seq)
    P = need if num_pages is None else num_pages
    assert P >= need, (P, need)
    P = max(P, 1)
    W = table_width if table_width is not None else max(max(pages_per_seq, default=1), 1)
    perm = torch.randperm(P, generator=gen) if shuffle_pool else torch.arange(P)
    bt = _tables_from_perm(perm, pages_per_seq, W)
    N = sum(query_lens)
    q = _draw(gen, (N, num_q_heads, head_dim), dtype)
    k_pool = _draw(gen, (P, page_size, num_kv_heads, head_dim), dtype)
    v_pool = _draw(gen, (P, page_size, num_kv_heads, head_dim), dtype)
    qsl = torch.zeros(B + 1, dtype=torch.int32)
    if B:
        qsl[1:] = torch.cumsum(torch.tensor(query_lens, dtype=torch.int64), 0).to(torch.int32)
    sc = _f32(1.0 / math.sqrt(head_dim)) if scale is None else _f32(scale)
    return Workload(name=name, dtype=dtype, q=q, k_pool=k_pool, v_pool=v_pool, block_tables=bt,
                    context_lens=torch.tensor(context_lens, dtype=torch.int32), query_start_loc=qsl,
                    scale=sc, causal=causal)


def make_shared_prefix(*, seed: int, prefix_len: int, suffix_lens: List[int], query_lens: List[int],
                       num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                       dtype: torch.dtype = torch.bfloat16, name: str = "shared prefix") -> Workload:
    """Requests that share their first ``prefix_len`` cached positions.

    ``prefix_len`` is a whole number of pages.  The prefix pages are drawn once
    and every block table starts with the same page ids (a cached system
    prompt, page "32. Production attention kernels", Stretch exercises:
    cascade attention); request b then owns ``suffix_lens[b]`` further
    positions (its step's ``query_lens[b]`` tokens included) on pages of its
    own.  Draw order: (1) pool permutation, (2) q, (3) k_pool, (4) v_pool.
    """
    assert prefix_len % page_size == 0 and prefix_len > 0
    gen = torch.Generator("cpu").manual_seed(seed)
    B = len(suffix_lens)
    assert len(query_lens) == B and all(n <= s for n, s in zip(query_lens, suffix_lens))
    npre = prefix_len // page_size
    nsuf = [(s + page_size - 1) // page_size for s in suffix_lens]
    P = npre + sum(nsuf)
    W = npre + max(nsuf)
    perm = torch.randperm(P, generator=gen).to(torch.int32)
    bt = torch.zeros(B, W, dtype=torch.int32)
    off = npre
    for b in range(B):
        bt[b, :npre] = perm[:npre]
        bt[b, npre:npre + nsuf[b]] = perm[off:off + nsuf[b]]
        off += nsuf[b]
    N = sum(query_lens)
    q = _draw(gen, (N, num_q_heads, head_dim), dtype)
    k_pool = _draw(gen, (P, page_size, num_kv_heads, head_dim), dtype)
    v_pool = _draw(gen, (P, page_size, num_kv_heads, head_dim), dtype)
    qsl = torch.zeros(B + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(query_lens, dtype=torch.int64), 0).to(torch.int32)
    lens = torch.tensor([prefix_len + s for s in suffix_lens], dtype=torch.int32)
    return Workload(name=name, dtype=dtype, q=q, k_pool=k_pool, v_pool=v_pool, block_tables=bt,
                    context_lens=lens, query_start_loc=qsl, scale=_f32(1.0 / math.sqrt(head_dim)))


def make_cascade_decode(seed: int = 7) -> Workload:
    """64 decoding requests sharing a 4,096-position cached prefix (64 pages
    of 64), each with its own suffix of U{1..512} positions; 32 query / 8 KV
    heads, head dim 128, bf16 (the shared-system-prompt case of page "32.
    Production attention kernels", Stretch exercises: cascade attention, with
    its ~4,000-token prompt rounded to whole pages)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    suffix = torch.randint(1, 513, (64,), generator=gen).tolist()
    return make_shared_prefix(seed=seed + 1000, prefix_len=4096, suffix_lens=suffix, query_lens=[1] * 64,
                              num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                              name="cascade decode: 64 requests, shared 4096-position prefix, suffixes U{1..512}")


def make(config: int, seed: Optional[int] = None, *, padded_width: bool = False) -> Workload:
    """The five measured workloads (6 = the head-dim-256 prefill variant).

    ``seed`` defaults to the config number.
    """
    seed = config if seed is None else seed
    gen = torch.Generator("cpu").manual_seed(seed)
    if config == 1:
        B, Hq, Hkv, D, ps, P, dtype = 1, 8, 2, 64, 16, 64, torch.float32
        lens = [600]
        # (1) lengths are fixed; (2) pool permutation
        perm = torch.randperm(P, generator=gen)
        npg = (600 + ps - 1) // ps  # 38
        W = 48 if padded_width else npg
        bt = torch.zeros(1, W, dtype=torch.int32)
        bt[0, :npg] = perm[:npg].to(torch.int32)
        qlens = [1]
        scale = 0.125
    elif config in (2, 3):
        B, Hq, Hkv, D, ps, dtype = (32 if config == 2 else 64), 32, 8, 128, 64, torch.bfloat16
        if config == 2:
            lens = torch.randint(1, 4097, (B,), generator=gen).tolist()
        else:
            lens = [4096] * B
        npgs = [(L + ps - 1) // ps for L in lens]
        P = sum(npgs)
        perm = torch.randperm(P, generator=gen)
        W = 64
        bt = _tables_from_perm(perm, npgs, W)
        qlens = [1] * B
        scale = _f32(1.0 / math.sqrt(D))
    elif config == 4:
        Hq, Hkv, D, ps, dtype = 32, 8, 128, 64, torch.bfloat16
        dec = torch.randint(256, 8193, (30,), generator=gen).tolist()
        lens = [1536] + dec + [2048]
        qlens = [512] + [1] * 30 + [5]
        B = len(lens)
        npgs = [(L + ps - 1) // ps for L in lens]
        P = sum(npgs)
        perm = torch.randperm(P, generator=gen)
        W = 128
        bt = _tables_from_perm(perm, npgs, W)
        scale = _f32(1.0 / math.sqrt(D))
    elif config in (5, 6):
        if config == 5:
            Hq, Hkv, D = 32, 8, 128
        else:
            Hq, Hkv, D = 16, 4, 256
        B, ps, dtype, Lp = 4, 64, torch.bfloat16, 8192
        lens = [Lp] * B
        qlens = [Lp] * B
        npgs = [Lp // ps] * B
        P = sum(npgs)
        perm = torch.randperm(P, generator=gen)
        W = 128
        bt = _tables_from_perm(perm, npgs, W)
        scale = _f32(1.0 / math.sqrt(D))
    else:
        raise ValueError(f"unknown config {config}")
    N = sum(qlens)
    q = _draw(gen, (N, Hq, D), dtype)
    k_pool = _draw(gen, (P, ps, Hkv, D), dtype)
    v_pool = _draw(gen, (P, ps, Hkv, D), dtype)
    qsl = torch.zeros(len(qlens) + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(qlens, dtype=torch.int64), 0).to(torch.int32)
    return Workload(name=CONFIG_NAMES[config], dtype=dtype, q=q, k_pool=k_pool, v_pool=v_pool,
                    block_tables=bt, context_lens=torch.tensor(lens, dtype=torch.int32),
                    query_start_loc=qsl, scale=scale, causal=True)


def poison_unused(w: Workload, value: float = float("nan")) -> Workload:
    """Return a copy whose pool slots that no sequence may read hold ``value``.

    Poisoned: every page no block table names within its sequence's length,
    and the slots of each last page past the context length.  Table entries
    past a sequence's pages are left as they are (zero padding), so they point
    at page 0, which may belong to another sequence: a kernel must not read them.
    """
    k = w.k_pool.clone()
    v = w.v_pool.clone()
    P, ps = k.shape[0], k.shape[1]
    used = torch.zeros(P, ps, dtype=torch.bool)
    W = w.block_tables.shape[1]
    for b in range(w.num_seqs):
        L = max(0, min(int(w.context_lens[b]), W * ps))
        for j in range(L):
            used[int(w.block_tables[b, j // ps]), j % ps] = True
    k[~used] = value
    v[~used] = value
    return dataclasses.replace(w, k_pool=k, v_pool=v)
