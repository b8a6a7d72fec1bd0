"""Benchmark of the paged KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5]

A step is one pass of the whole path over one batch: kv_cache_write of the
step's new K/V rows, then paged_attention (decode kernel, plus the combine when
split) for the headline decode workload -- 64 sequences x 4096 context,
32 query / 8 KV heads, head dim 128, page 64, bf16 (the Qwen3-8B-shaped step of
page "32. Production attention kernels").  Pools are rotated over 4 distinct
sets ("layers", 4.3 GB) so the 256 MB Infinity Cache cannot hold the working
set.  A second measured object covers long causal prefill (4 x 8192 tokens,
same heads), reported in TFLOP/s.

Prints ONE JSON line.  `value` is decode GB/s of algorithmic bytes (K and V
once per GQA group + q + out + page ids + lengths) over the timed step time.
`roofline` is for the decode kernel: algorithmic bytes per launch over its
average launch time, measured with HIP events on the launch stream.
`cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention HBM GB/s (% of peak) at 64×4096 ctx; prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
# Prefill launches (~2 ms each) speed up over the first ~10 after an idle
# period while the clock settles under load: the prefill legs warm up with at
# least this many launches before timing, so they report the steady state.
PREFILL_WARMUP = 10
CSRC = os.path.join(ROOT, "paged_kv_attention_amd", "csrc")
# Measured HBM traffic per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by
# a plain copy's counts) is kept next to the hash of the sources it was taken
# from; a kernel changed since then reports traffic null.
TRAFFIC_FILES = {"decode": (os.path.join(ROOT, "profiles", "decode_c3_traffic.json"), ("decode.hip", "decode_tile.h")),
                 "prefill": (os.path.join(ROOT, "profiles", "prefill_c5_traffic.json"), ("prefill.hip",)),
                 "prefill_d256": (os.path.join(ROOT, "profiles", "prefill_c6_traffic.json"),
                                  ("prefill16.hip", "prefill16_tile.h")),
                 "mixed": (os.path.join(ROOT, "profiles", "mixed_c4_traffic.json"),
                           ("mixed.hip", "decode_tile.h", "prefill16_tile.h"))}
# kernel (name prefix, with its head-dim template argument) each traffic file is about
TRAFFIC_KERNELS = {"decode": "pa::decode_splitkv_kernel<128, 1,", "prefill": "pa::prefill_kernel<128,",
                   "prefill_d256": "pa::prefill16_kernel<256, 8, false, 0>", "mixed": "pa::mixed_kernel<"}


# ----------------------------------------------------------------------------- accounting
def _key_range(L, n, window):
    """Positions [lo, hi) some query row of the step can see (causal or not:
    keys past L never exist; a sliding window drops keys before the first
    row's window start)."""
    L = max(0, L)
    lo = max(0, L - n - window + 1) if window > 0 else 0
    return lo, L


def algorithmic_bytes(context_lens, query_lens, num_q_heads, num_kv_heads, head_dim, page_size, elem_bytes,
                      window=0, kv_code_bytes=None, scale_bytes=0):
    """Bytes the method must move: K and V of every visible position once per
    GQA group, q read and out written once, the page ids of the pages used,
    the lengths and query offsets.  (Page "32. Production attention kernels",
    What the reference backend costs: 2 x Hkv x D values per token per layer.)
    With a sliding window only the positions some row can see count.  A
    quantized cache stores ``kv_code_bytes`` per element plus ``scale_bytes``
    per (position, KV head) vector (page "32. Production attention kernels",
    Quantized KV caches: a float32 scale, 4 bytes, beside each vector of D
    codes)."""
    per_vec = head_dim * (elem_bytes if kv_code_bytes is None else kv_code_bytes) + scale_bytes
    kv = ids = 0
    for L, n in zip(context_lens, query_lens):
        lo, hi = _key_range(L, n, window)
        kv += (hi - lo) * num_kv_heads * 2 * per_vec
        ids += ((hi + page_size - 1) // page_size - lo // page_size) * 4 if hi > lo else 0
    n = sum(query_lens)
    qo = n * num_q_heads * head_dim * elem_bytes * 2
    meta = (2 * len(context_lens) + 1) * 4
    return kv + qo + ids + meta


def algorithmic_flops(context_lens, query_lens, num_q_heads, head_dim, causal=True, window=0):
    """4 * D * Hq per visible (query, key) pair: 2 for q.k and 2 for p.v."""
    pairs = 0
    for L, n in zip(context_lens, query_lens):
        for t in range(n):
            pos = L - n + t
            hi = max(0, min(L, pos + 1)) if causal else max(0, L)
            lo = max(0, pos - window + 1) if window > 0 else 0
            pairs += max(0, hi - lo)
    return 4 * head_dim * num_q_heads * pairs


def kv_write_bytes(tokens, num_kv_heads, head_dim, elem_bytes):
    return 2 * 2 * tokens * num_kv_heads * head_dim * elem_bytes + 4 * tokens


def kernel_src_hash(kernel_files):
    """Hash of a kernel's sources and the device headers it includes."""
    h = hashlib.sha256()
    for name in (*kernel_files, "pa_device.h", "pa_params.h"):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(which):
    path, src = TRAFFIC_FILES[which]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    return tr.get("bytes_per_launch") if tr.get("src_sha256_16") == kernel_src_hash(src) else None


# ----------------------------------------------------------------------------- GPU workloads
class DecodeBench:
    """Headline decode workload with rotated pool sets."""

    def __init__(self, layers=4, num_splits=0):
        import torch
        import paged_kv_attention_amd as pa
        from workloads import make
        self.torch, self.pa = torch, pa
        self.w = make(3)
        dev = torch.device("cuda", 0)
        w = self.w
        self.q = w.q.to(dev)
        self.bt = w.block_tables.to(dev)
        self.cl = w.context_lens.to(dev)
        self.qsl = w.query_start_loc.to(dev)
        self.pools = [(pa.pool_like(w.k_pool, dev), pa.pool_like(w.v_pool, dev))]
        gen = torch.Generator(device=dev).manual_seed(1234)
        P, ps, Hkv, D = w.k_pool.shape
        for _ in range(layers - 1):
            k = pa.empty_pool(P, ps, Hkv, D, device=dev)
            v = pa.empty_pool(P, ps, Hkv, D, device=dev)
            k.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
            v.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
            self.pools.append((k, v))
        self.out = torch.empty_like(self.q)
        self.dims = pa.make_dims(self.q, self.pools[0][0], self.bt, out=self.out, max_query_len=1,
                                 num_splits=num_splits)
        ws = pa.workspace_size(self.dims, torch.bfloat16)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.splits = pa.choose_splits(self.dims)
        self.num_splits = num_splits
        # the step's new token of each sequence sits at its newest position L-1
        lens = w.context_lens.tolist()
        ps = w.page_size
        slots = [int(w.block_tables[b, (L - 1) // ps]) * ps + (L - 1) % ps for b, L in enumerate(lens)]
        self.slots = torch.tensor(slots, dtype=torch.int32, device=dev)
        self.k_new = torch.randn(len(lens), w.num_kv_heads, w.head_dim, generator=gen, device=dev).to(torch.bfloat16)
        self.v_new = torch.randn(len(lens), w.num_kv_heads, w.head_dim, generator=gen, device=dev).to(torch.bfloat16)
        self.attn_bytes = algorithmic_bytes(lens, w.query_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, ps, 2)
        self.write_bytes = kv_write_bytes(len(lens), w.num_kv_heads, w.head_dim, 2)

    def attend(self, layer):
        k, v = self.pools[layer % len(self.pools)]
        return self.pa.paged_attention(self.q, k, v, self.bt, self.cl, self.qsl, self.w.scale, True, out=self.out,
                                       workspace=self.ws, max_query_len=1, num_splits=self.num_splits)

    def write(self, layer):
        k, v = self.pools[layer % len(self.pools)]
        self.pa.kv_cache_write(self.k_new, self.v_new, k, v, self.slots)

    def step(self, layer):
        """The decode step as one call: the new rows go in with the attention
        (the decode launch writes them before reading a key)."""
        k, v = self.pools[layer % len(self.pools)]
        return self.pa.paged_attention(self.q, k, v, self.bt, self.cl, self.qsl, self.w.scale, True, out=self.out,
                                       workspace=self.ws, max_query_len=1, num_splits=self.num_splits,
                                       k_new=self.k_new, v_new=self.v_new, slot_mapping=self.slots)



class PrefillBench:
    def __init__(self, config=5):
        import torch
        import paged_kv_attention_amd as pa
        from workloads import make
        self.torch, self.pa = torch, pa
        self.w = w = make(config)
        dev = torch.device("cuda", 0)
        self.q = w.q.to(dev)
        self.k, self.v = pa.pool_like(w.k_pool, dev), pa.pool_like(w.v_pool, dev)
        self.bt = w.block_tables.to(dev)
        self.cl = w.context_lens.to(dev)
        self.qsl = w.query_start_loc.to(dev)
        self.out = torch.empty_like(self.q)
        self.mql = w.max_query_len
        lens = w.context_lens.tolist()
        ps = w.page_size
        # the prompt's K/V rows are written through the slot map in the same step
        slots = []
        for b, L in enumerate(lens):
            for j in range(L):
                slots.append(int(w.block_tables[b, j // ps]) * ps + j % ps)
        self.slots = torch.tensor(slots, dtype=torch.int32, device=dev)
        gen = torch.Generator(device=dev).manual_seed(99)
        T = len(slots)
        self.k_new = torch.randn(T, w.num_kv_heads, w.head_dim, generator=gen, device=dev).to(torch.bfloat16)
        self.v_new = torch.randn(T, w.num_kv_heads, w.head_dim, generator=gen, device=dev).to(torch.bfloat16)
        self.flops = algorithmic_flops(lens, w.query_lens, w.num_q_heads, w.head_dim)

    def write(self):
        self.pa.kv_cache_write(self.k_new, self.v_new, self.k, self.v, self.slots)

    def attend(self):
        return self.pa.paged_attention(self.q, self.k, self.v, self.bt, self.cl, self.qsl, self.w.scale, True,
                                       out=self.out, max_query_len=self.mql)


class WorkloadBench:
    """Any seeded workload on device, pools rotated over `layers` sets.
    `config` is a config number of workloads.make, or a Workload."""

    def __init__(self, config, layers=1, window=0, sinks=False, kv_kind=None, num_splits=0):
        import torch
        import paged_kv_attention_amd as pa
        from workloads import make
        self.torch, self.pa = torch, pa
        self.w = w = make(config) if isinstance(config, int) else config
        self.num_splits = num_splits
        self.window = window
        # sink logits: one per query head, drawn from their own seeded stream
        self.sinks_cpu = (torch.randn(w.num_q_heads, generator=torch.Generator().manual_seed(777)) * 2.0
                          if sinks else None)
        dev = torch.device("cuda", 0)
        self.q = w.q.to(dev)
        self.bt = w.block_tables.to(dev)
        self.cl = w.context_lens.to(dev)
        self.qsl = w.query_start_loc.to(dev)
        self.pools = [(pa.pool_like(w.k_pool, dev), pa.pool_like(w.v_pool, dev))]
        gen = torch.Generator(device=dev).manual_seed(4321)
        P, ps, Hkv, D = w.k_pool.shape
        for _ in range(layers - 1):
            k = pa.empty_pool(P, ps, Hkv, D, dtype=w.dtype, device=dev)
            v = pa.empty_pool(P, ps, Hkv, D, dtype=w.dtype, device=dev)
            k.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
            v.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
            self.pools.append((k, v))
        self.kv_kind = kv_kind
        self.quant = [None] * len(self.pools)
        if kv_kind is not None:
            # quantize every pool set on the device with the library's own write
            qpools = []
            slots = torch.arange(P * ps, dtype=torch.int32, device=dev)
            for i, (k, v) in enumerate(self.pools):
                kc = pa.empty_code_pool(P, ps, Hkv, D, kv_kind, dev)
                vc = pa.empty_code_pool(P, ps, Hkv, D, kv_kind, dev)
                kq = pa.KvQuant(kv_kind, pa.empty_scale_pool(P, ps, Hkv, dev), pa.empty_scale_pool(P, ps, Hkv, dev))
                pa.kv_cache_write_quant(k.reshape(P * ps, Hkv, D), v.reshape(P * ps, Hkv, D), kc, vc, slots, kq)
                qpools.append((kc, vc))
                self.quant[i] = kq
            torch.cuda.synchronize()
            self.pools = qpools
        self.out = torch.empty_like(self.q)
        dims = pa.make_dims(self.q, self.pools[0][0], self.bt, out=self.out, max_query_len=w.max_query_len,
                            num_splits=num_splits)
        self.ws = torch.empty(max(pa.workspace_size(dims, w.dtype), 16), dtype=torch.uint8, device=dev)
        # pa_choose_splits gives the bf16 count; float32 calls follow their own rule
        self.splits = pa.choose_splits(dims) if w.dtype != torch.float32 else "float32 rule"
        lens = w.context_lens.tolist()
        e = 4 if w.dtype == torch.float32 else 2
        self.bytes = algorithmic_bytes(lens, w.query_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, ps, e,
                                       window=window, kv_code_bytes=None if kv_kind is None else 1,
                                       scale_bytes=0 if kv_kind is None else 4)
        self.flops = algorithmic_flops(lens, w.query_lens, w.num_q_heads, w.head_dim, causal=w.causal,
                                       window=window)
        self.sinks = None if self.sinks_cpu is None else self.sinks_cpu.to(dev)

    def attend(self, layer):
        k, v = self.pools[layer % len(self.pools)]
        w = self.w
        return self.pa.paged_attention(self.q, k, v, self.bt, self.cl, self.qsl, w.scale, w.causal, out=self.out,
                                       workspace=self.ws, max_query_len=w.max_query_len, window=self.window,
                                       sinks=self.sinks, kv_quant=self.quant[layer % len(self.pools)],
                                       num_splits=self.num_splits)



def _hbm_entry(name, wb, steps, warmup, layers):
    """Per-call, GPU-side and back-to-back times of one workload and its HBM
    roofline (algorithmic bytes over the GPU-side time per call)."""
    import torch
    _, per = _time_steps([wb.attend], steps, warmup)
    ms = per[0]
    gpu = _time_queued(wb.attend, steps, warmup)
    # calls back to back: two events around all calls and none between
    # them, so the host's launch path runs ahead of the GPU's work
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        wb.attend(i)
    e1.record()
    torch.cuda.synchronize()
    ms_b2b = e0.elapsed_time(e1) / steps
    gbs = wb.bytes / (gpu["median"] * 1e-3) / 1e9
    return {"workload": name, "ms": round(ms, 5), "gpu_ms": gpu["median"], "gpu_ms_min": gpu["min"],
            "ms_back_to_back": round(ms_b2b, 5), "splits": wb.splits, "algorithmic_bytes": wb.bytes,
            "algorithmic_flops": wb.flops, "GB_s": round(gbs, 2), "hbm_frac_per_call": round(wb.bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_frac_back_to_back": round(wb.bytes / (ms_b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "time": "gpu_ms (queued)"},
            "pool_sets_rotated": layers}


def other_workloads(steps, warmup):
    """The other configurations and the decode shapes the headline leaves out:
    the fp32 single-sequence decode (latency), the ragged decode batch, the
    mixed batch, one long bf16 sequence at 4096 and 32768 positions (one
    sequence must still fill the chip), the ragged batch at contexts up to
    16384 (the balanced decode launch) and a batch of 16-token verification
    steps; each with its HBM roofline.  Pools are rotated so the Infinity
    Cache cannot hold them.  `ms` brackets each call with events (the host's
    launch path included); `gpu_ms` is the GPU time per call with the host
    running ahead (see _time_queued); the roofline uses gpu_ms."""
    import torch
    from workloads import make_custom
    res = {}
    one = lambda L, seed: make_custom(seed=seed, context_lens=[L], query_lens=[1], num_q_heads=32, num_kv_heads=8,
                                      head_dim=128, page_size=64, dtype=torch.bfloat16,
                                      name=f"bf16 decode of one sequence at {L} positions, 32/8 heads, D 128, page 64")
    verify = make_custom(seed=13, context_lens=[2048] * 64, query_lens=[16] * 64, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, page_size=64, dtype=torch.bfloat16,
                         name="bf16 verification: 64 seqs x 16-token steps at 2048 positions, 32/8 heads, D 128, page 64")
    # the ragged decode batch at four times the context: splits of 5504 keys,
    # so the 16-row tiles run as the balanced launch
    g = torch.Generator().manual_seed(11)
    long_lens = torch.randint(1, 16385, (32,), generator=g).tolist()
    ragged_long = make_custom(seed=12, context_lens=long_lens, query_lens=[1] * 32, num_q_heads=32, num_kv_heads=8,
                              head_dim=128, page_size=64, dtype=torch.bfloat16,
                              name="bf16 ragged decode, 32 seqs, ctx U{1..16384}, 32/8 heads, D 128, page 64")
    for key, cfg, layers, name in [
            ("config1", 1, 1, "fp32 single-sequence decode, 8/2 heads, D 64, page 16, ctx 600"),
            ("config2", 2, 8, "bf16 ragged decode, 32 seqs, ctx U{1..4096}, 32/8 heads, D 128, page 64"),
            ("config4", 4, 8, "bf16 mixed batch: 512-token chunk over 1024 prefix + 30 decodes + 5-token verify"),
            ("decode_1x4096", one(4096, 11), 32, None),
            ("decode_1x32768", one(32768, 12), 8, None),
            ("decode_ragged_32x16k", ragged_long, 4, None),
            ("verify_64x16_at_2048", verify, 4, None)]:
        print(f"[bench] other workload {key}: building inputs", file=sys.stderr, flush=True)
        wb = WorkloadBench(cfg, layers)
        res[key] = _hbm_entry(name or wb.w.name, wb, steps, warmup, layers)
        if key == "config4":
            # the mixed batch is one launch (and the combine): its measured HBM bytes
            res[key]["roofline"]["traffic"] = measured_traffic("mixed")
        del wb
        torch.cuda.empty_cache()
    return res


def variant_workloads(steps, warmup):
    """The variants at the headline shapes: the 64 x 4096 decode with a
    1024-position window (HBM-bound: only the window's K/V count) and the
    4 x 8192 causal prefill with a 4096-position window (MFMA-bound: only the
    band's pairs count), both with one sink logit per query head; and the
    decode over int8 and fp8 caches (bytes: 1-byte codes plus a float32
    scale per position and KV head), and the prefill over an int8 cache."""
    import torch
    res = {}
    for cfg, layers, window, sinks, kind, bound, key, name in [
            (3, 4, 1024, True, None, "hbm", "config3_window1024_sinks",
             "bf16 decode 64 x 4096, 32/8 heads, D 128, page 64, window 1024, sinks"),
            (5, 1, 4096, True, None, "mfma", "config5_window4096_sinks",
             "bf16 causal prefill 4 x 8192, 32/8 heads, D 128, page 64, window 4096, sinks"),
            (3, 4, 0, False, "int8", "hbm", "config3_int8_kv",
             "decode 64 x 4096, 32/8 heads, D 128, page 64, bf16 q over an int8 KV cache (scale per token and head)"),
            (3, 4, 0, False, "fp8", "hbm", "config3_fp8_kv",
             "decode 64 x 4096, 32/8 heads, D 128, page 64, bf16 q over an fp8 E4M3 KV cache (scale per token and head)"),
            (5, 1, 0, False, "int8", "mfma", "config5_int8_kv",
             "causal prefill 4 x 8192, 32/8 heads, D 128, page 64, bf16 q over an int8 KV cache")]:
        print(f"[bench] variant: {name}", file=sys.stderr, flush=True)
        wb = WorkloadBench(cfg, layers, window=window, sinks=sinks, kv_kind=kind)
        vsteps = steps if bound == "hbm" else max(3, min(steps, 10))
        # MFMA-bound launches run ~2 ms each; the clock settles over the first
        # ~10 of them, so these take at least 10 warm-up launches
        _, per = _time_steps([wb.attend], vsteps, warmup if bound == "hbm" else max(warmup, PREFILL_WARMUP))
        ms = per[0]
        entry = {"workload": name, "ms": round(ms, 5), "window": window, "kv_cache": kind or "bf16", "splits": wb.splits,
                 "algorithmic_bytes": wb.bytes, "algorithmic_flops": wb.flops, "pool_sets_rotated": layers}
        if bound == "hbm":
            gbs = wb.bytes / (ms * 1e-3) / 1e9
            entry.update({"GB_s": round(gbs, 2), "roofline": {"bound": "hbm", "achieved": round(gbs, 2),
                                                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                              "frac": round(gbs / HBM_PEAK_GBS, 4)}})
        else:
            tf = wb.flops / (ms * 1e-3) / 1e12
            entry.update({"TFLOP_s": round(tf, 2), "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                                                                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                                                "frac": round(tf / BF16_PEAK_TFLOPS, 4)}})
        res[key] = entry
        del wb
        torch.cuda.empty_cache()
    return res


def cascade_workload(steps, warmup):
    """64 decoding requests sharing a 4,096-position prefix (suffixes
    U{1..512}): the cascade call against the plain call on the same inputs,
    pools rotated over 4 sets.  Algorithmic bytes of the cascade: the
    prefix's K/V once, every suffix's K/V, q and out, page ids."""
    import torch
    import paged_kv_attention_amd as pa
    from workloads import make_cascade_decode
    w = make_cascade_decode()
    dev = torch.device("cuda", 0)
    q, bt, cl, qsl = w.q.to(dev), w.block_tables.to(dev), w.context_lens.to(dev), w.query_start_loc.to(dev)
    P, ps, Hkv, D = w.k_pool.shape
    gen = torch.Generator(device=dev).manual_seed(99)
    pools = [(pa.pool_like(w.k_pool, dev), pa.pool_like(w.v_pool, dev))]
    for _ in range(3):
        k = pa.empty_pool(P, ps, Hkv, D, device=dev)
        v = pa.empty_pool(P, ps, Hkv, D, device=dev)
        k.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
        v.copy_(torch.randn(P, ps, Hkv, D, generator=gen, device=dev))
        pools.append((k, v))
    out = torch.empty_like(q)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    prefix = 4096
    lens = w.context_lens.tolist()

    def run(cascade):
        def f(i):
            k, v = pools[i % len(pools)]
            pa.paged_attention(q, k, v, bt, cl, qsl, w.scale, True, out=out, workspace=ws, max_query_len=1,
                               shared_prefix_len=prefix if cascade else 0)
        return f
    _, per_c = _time_steps([run(True)], steps, warmup)
    _, per_p = _time_steps([run(False)], steps, warmup)
    suffix_keys = sum(L - prefix for L in lens)
    kv_vec = Hkv * D * 2 * 2                                   # K and V bytes per position
    casc_bytes = (prefix + suffix_keys) * kv_vec + w.num_tokens * w.num_q_heads * D * 2 * 2 + \
        (prefix // ps + sum((L - prefix + ps - 1) // ps for L in lens)) * 4 + (2 * len(lens) + 1) * 4
    plain_bytes = algorithmic_bytes(lens, w.query_lens, w.num_q_heads, Hkv, D, ps, 2)
    gbs = casc_bytes / (per_c[0] * 1e-3) / 1e9
    return {"workload": w.name, "cascade_ms": round(per_c[0], 5), "plain_ms": round(per_p[0], 5),
            "speedup": round(per_p[0] / per_c[0], 2), "cascade_algorithmic_bytes": casc_bytes,
            "plain_algorithmic_bytes": plain_bytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "plain_GB_s": round(plain_bytes / (per_p[0] * 1e-3) / 1e9, 2), "pool_sets_rotated": len(pools)}


def graph_step(db, steps):
    """The decode step (write + attention) of every rotated pool set captured
    in one hipGraph, as a model step captures all its layers, and replayed:
    host launch overhead removed.  Returns ms per step (per pool set)."""
    import torch
    layers = len(db.pools)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for layer in range(layers):              # warm the launch path on this stream
            db.write(layer)
            db.attend(layer)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for layer in range(layers):
            db.write(layer)
            db.attend(layer)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // layers)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * layers)


def _time_steps(step_fns, steps, warmup):
    """Run warmup, then time `steps` steps; each fn in step_fns is timed with
    HIP events on the current stream.  Returns (total_ms, [avg ms per fn])."""
    import torch
    for i in range(warmup):
        for f in step_fns:
            f(i)
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in step_fns]
           for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        for j, f in enumerate(step_fns):
            evs[i][j][0].record()
            f(warmup + i)
            evs[i][j][1].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    times = [[evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)] for j in range(len(step_fns))]
    per = [sum(t) / steps for t in times]
    _time_steps.last = times
    return total, per


_SPIN_CYCLES_PER_MS = None


def _time_queued(step_fn, steps, warmup):
    """GPU time per call with the host running ahead of the GPU: a spin
    kernel holds the GPU while every call and its pair of events are
    enqueued, so each pair brackets the call's own GPU work (its launches and
    the gaps between them) rather than the host's launch path.  Returns the
    median and minimum in ms."""
    import torch
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    for i in range(warmup):
        step_fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    # hold the GPU for about 0.2 ms per call to be enqueued (the host needs
    # well under that per call)
    torch.cuda._sleep(int(_SPIN_CYCLES_PER_MS * (1.0 + 0.2 * steps)))
    for i in range(steps):
        evs[i][0].record()
        step_fn(warmup + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return _spread([a.elapsed_time(b) for a, b in evs])


def _spread(times):
    """Median and minimum of one function's per-step times (ms)."""
    t = sorted(times)
    n = len(t)
    med = t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])
    return {"median": round(med, 5), "min": round(t[0], 5)}


def read_ceiling(reps=10):
    """HBM streaming-read rate of the library's read probe (16-byte
    nontemporal loads over a 4 GiB buffer, best of `reps`): the practical
    ceiling for a kernel that streams K/V pages, which the decode kernel's
    read rate is compared with."""
    import torch
    import paged_kv_attention_amd as pa
    buf = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    sink = torch.empty(pa.READ_PROBE_SINK_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        pa.read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        e0.record()
        pa.read_probe(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del buf, sink
    torch.cuda.empty_cache()
    return round(4 * (1 << 30) / (best * 1e-3) / 1e9, 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds_target=12.0):
    """The float64 oracle, as it stands, on a bounded sample of the decode
    workload: whole sequences (all heads) in order, cycling, until about
    `seconds_target` seconds of host work are done."""
    import torch
    from oracle import attention_f64
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    qsl = w.query_start_loc.tolist()
    lens = w.context_lens.tolist()
    done_seqs, done_bytes = 0, 0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < seconds_target:
        b = done_seqs % w.num_seqs
        sub_qsl = torch.tensor([0, qsl[b + 1] - qsl[b]], dtype=torch.int32)
        attention_f64(w.q[qsl[b]:qsl[b + 1]], w.k_pool, w.v_pool, w.block_tables[b:b + 1],
                      w.context_lens[b:b + 1], sub_qsl, w.scale)
        done_bytes += algorithmic_bytes([lens[b]], [qsl[b + 1] - qsl[b]], w.num_q_heads, w.num_kv_heads,
                                        w.head_dim, w.page_size, 2)
        done_seqs += 1
    el = time.perf_counter() - t_start
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done_seqs} sequence passes (64 x 4096 decode step, one sequence with all 32 heads "
                      f"per pass), float64, {el:.1f} s"}


def cpu_baseline_configs(seconds_per_config=3.0):
    """The oracle on a bounded sample of every configuration, with the same
    algorithmic bytes (decode configs, GB/s) or flops (prefill configs,
    TFLOP/s) as the GPU rows: whole sequences in turn for the decode
    configurations, the last query rows of sequence 0 (the longest rows of a
    causal prompt) for the prefills."""
    import torch
    from oracle import attention_f64
    from workloads import make
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    res = {}
    for cfg in (1, 2, 3, 4, 5, 6):
        w = make(cfg)
        qsl = w.query_start_loc.tolist()
        lens = w.context_lens.tolist()
        e = 4 if w.dtype == torch.float32 else 2
        t0 = time.perf_counter()
        units, done_b, done_f = 0, 0, 0
        if cfg in (5, 6):
            rows = 64
            while time.perf_counter() - t0 < seconds_per_config or units == 0:
                toks = list(range(qsl[1] - rows * (units + 1), qsl[1] - rows * units))
                attention_f64(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale,
                              tokens=toks)
                L = lens[0]
                done_f += sum(4 * w.head_dim * w.num_q_heads * (L - (qsl[1] - t) + 1) for t in toks)
                units += 1
            el = time.perf_counter() - t0
            res[f"config{cfg}"] = {"value": round(done_f / el / 1e12, 6), "unit": "TFLOP/s", "seconds": round(el, 2),
                                   "sample": f"{units * rows} query tokens (all heads) at the end of sequence 0"}
        else:
            while time.perf_counter() - t0 < seconds_per_config or units == 0:
                b = units % w.num_seqs
                sub = torch.tensor([0, qsl[b + 1] - qsl[b]], dtype=torch.int32)
                attention_f64(w.q[qsl[b]:qsl[b + 1]], w.k_pool, w.v_pool, w.block_tables[b:b + 1],
                              w.context_lens[b:b + 1], sub, w.scale)
                done_b += algorithmic_bytes([lens[b]], [qsl[b + 1] - qsl[b]], w.num_q_heads, w.num_kv_heads,
                                            w.head_dim, w.page_size, e)
                units += 1
            el = time.perf_counter() - t0
            res[f"config{cfg}"] = {"value": round(done_b / el / 1e9, 4), "unit": "GB/s", "seconds": round(el, 2),
                                   "sample": f"{units} sequence passes (all heads)"}
        del w
    res["cores"] = torch.get_num_threads()
    res["cpu_model"] = cpu_model()
    return res


def _counter_rows(path, counter):
    """(dispatch id, kernel name, value) of one counter from a rocprofv3
    counter_collection CSV, in dispatch order."""
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


def traffic_summary(which, fetch_csv, write_csv):
    """HBM bytes per launch of the kernel `which` stands for, from a
    FETCH_SIZE and a WRITE_SIZE counter run (KiB per dispatch) of
    `bench.py --only ... --copy-calibration`: each counter is scaled by what
    it reads for the 1 GiB calibration copy (the runtime's copy kernel), then
    compared with the algorithmic bytes of one launch.
    Writes the traffic JSON the bench reads and returns the text summary."""
    from workloads import make
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    kname = TRAFFIC_KERNELS[which]
    # the calibration is the 1 GiB device-to-device copy (the runtime's copy
    # kernel); the fill that prepares its source writes as much but reads
    # nothing
    cal_w = max((r for r in write if "copyBuffer" in r[1]), key=lambda r: r[2])
    cal_f = max((r for r in fetch if "copyBuffer" in r[1]), key=lambda r: r[2])
    cal_name = cal_w[1]
    gib_kib = float(1 << 20)
    f_scale, w_scale = gib_kib / cal_f[2], gib_kib / cal_w[2]
    fk = [r[2] for r in fetch if r[1].startswith(kname) or ("void " + kname) in r[1]]
    wk = [r[2] for r in write if r[1].startswith(kname) or ("void " + kname) in r[1]]
    fb = sum(fk) / len(fk) * 1024 * f_scale
    wb = sum(wk) / len(wk) * 1024 * w_scale
    cfg = {"decode": 3, "prefill": 5, "prefill_d256": 6, "mixed": 4}[which]
    w = make(cfg)
    alg = algorithmic_bytes(w.context_lens.tolist(), w.query_lens, w.num_q_heads, w.num_kv_heads, w.head_dim,
                            w.page_size, 2)
    src = TRAFFIC_FILES[which][1]
    rec = {"kernel": kname, "workload": w.name, "bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
           "write_bytes": int(round(wb)), "algorithmic_bytes": alg, "src_sha256_16": kernel_src_hash(src),
           "source": os.path.relpath(TRAFFIC_FILES[which][0].replace("_traffic.json", "_hbm_traffic.txt"), ROOT)}
    with open(TRAFFIC_FILES[which][0], "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"copy calibration ({cal_name[:40]}): FETCH_SIZE {cal_f[2]:.1f} KiB, WRITE_SIZE {cal_w[2]:.1f} KiB for 1 GiB",
             f"scale factors: fetch {f_scale:.4f}, write {w_scale:.4f} (bytes per counter byte)",
             f"FETCH_SIZE per dispatch (KiB): {[round(x, 1) for x in fk]}",
             f"WRITE_SIZE per dispatch (KiB): {[round(x, 1) for x in wk]}",
             f"scaled traffic per launch: fetch {int(fb)} B + write {int(wb)} B = {int(fb + wb)} B",
             f"algorithmic bytes per launch: {alg} B -> traffic / algorithmic = {(fb + wb) / alg:.4f}",
             f"source hash ({' + '.join(src)} + pa_device.h + pa_params.h, sha256[:16]): {rec['src_sha256_16']}"]
    return "\n".join(lines)


def counter_summary(csv_paths, kernel, drop):
    """Average counter values per dispatch of `kernel` (a name prefix) over
    rocprofv3 counter_collection CSVs, after the first `drop` dispatches, and
    the figures derived from them: the clock the kernel ran at, MFMA busy
    per SIMD, VALU / LDS / transcendental instructions per MFMA, and the L2
    hit rate.  MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU."""
    import csv
    vals, times = {}, {}
    for path in csv_paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if not (r["Kernel_Name"].startswith(kernel) or ("void " + kernel) in r["Kernel_Name"]):
                    continue
                d = int(r["Dispatch_Id"])
                vals.setdefault(r["Counter_Name"], {})[d] = float(r["Counter_Value"])
                times[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    avg = {}
    for name, per in vals.items():
        ds = sorted(per)[drop:] or sorted(per)
        avg[name] = sum(per[d] for d in ds) / len(ds)
    ds = sorted(times)[drop:] or sorted(times)
    t_ns = sum(times[d] for d in ds) / len(ds)
    lines = [f"{k:28s} {v:12.4g}" for k, v in sorted(avg.items())]
    lines.append(f"kernel time per dispatch (counter run): {t_ns / 1000:.1f} us over {len(ds)} dispatches")
    if "GRBM_GUI_ACTIVE" in avg:
        clk = avg["GRBM_GUI_ACTIVE"] / 8 / t_ns
        lines.append(f"clock over the kernel, GRBM_GUI_ACTIVE / 8 XCDs / time: {clk:.3f} GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            lines.append(f"MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8) = "
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (avg['GRBM_GUI_ACTIVE'] / 8):.3f}")
    if "SQ_INSTS_MFMA" in avg and avg["SQ_INSTS_MFMA"] > 0:
        m = avg["SQ_INSTS_MFMA"]
        parts = [f"MFMA instructions per SIMD: {m / 1024:.0f}"]
        for k, label in (("SQ_INSTS_VALU", "VALU (incl. MFMA)"), ("SQ_INSTS_VALU_TRANS_F32", "exp2"),
                         ("SQ_INSTS_LDS", "LDS")):
            if k in avg:
                parts.append(f"{label} per MFMA: {avg[k] / m:.2f}")
        lines.append("; ".join(parts))
    if "SQ_WAVE_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        # SQ_WAVE_CYCLES counts resident-wave time in quad-cycles on this chip
        occ = 4 * avg["SQ_WAVE_CYCLES"] / 1024 / (avg["GRBM_GUI_ACTIVE"] / 8)
        lines.append(f"achieved occupancy: 4 x SQ_WAVE_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8) = {occ:.2f} waves per SIMD")
    if "SQ_WAVE_CYCLES" in avg and "SQ_WAIT_ANY" in avg:
        lines.append(f"SQ_WAIT_ANY / SQ_WAVE_CYCLES: {avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.3f}")
    if "SQ_WAVE_CYCLES" in avg and "SQ_WAIT_INST_LDS" in avg:
        lines.append(f"SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES: {avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.3f}")
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
        lines.append(f"L2 hit rate: {avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.3f}")
    return "\n".join(lines)


def trace_summary(path, drop):
    """Per-kernel durations from a rocprofv3 kernel trace (a results
    database, or the kernel_trace CSV of --output-format csv), in launch order
    per kernel and grid: all dispatches, and the dispatches after the first
    `drop` of each (the warm-up launches)."""
    import csv
    import re
    import sqlite3
    if path.endswith(".csv"):
        with open(path) as f:
            rows = [(r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), int(r["Grid_Size_X"]),
                     int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]), int(r["Workgroup_Size_X"]))
                    for r in csv.DictReader(f)]
    else:
        con = sqlite3.connect(path)
        rows = list(con.execute("select name, duration, grid_x, grid_y, grid_z, workgroup_x from kernels order by start"))
    groups = {}
    for name, dur, gx, gy, gz, wx in rows:
        short = re.sub(r"\(.*", "", name)
        groups.setdefault((short, gx // max(wx, 1), gy, gz), []).append(dur / 1000.0)
    lines = [f"{'kernel':70s} {'grid (workgroups)':>22s} {'n':>4s} {'avg_us':>9s} {'n_timed':>7s} {'avg_timed_us':>12s} {'min_us':>8s}"]
    for (short, gx, gy, gz), ds in groups.items():
        timed = ds[drop:] if len(ds) > drop else ds
        lines.append(f"{short[:70]:70s} {f'({gx},{gy},{gz})':>22s} {len(ds):4d} {sum(ds) / len(ds):9.2f} "
                     f"{len(timed):7d} {sum(timed) / len(timed):12.2f} {min(ds):8.2f}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other measured workloads")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay of the decode step")
    ap.add_argument("--no-variants", action="store_true", help="skip the sliding-window / sink workloads")
    ap.add_argument("--only", choices=["decode", "prefill", "prefill_d256", "mixed"], default=None,
                    help="time one workload only (for profiler runs)")
    ap.add_argument("--trace-summary", metavar="DB", default=None,
                    help="print per-kernel durations from a rocprofv3 results database and exit")
    ap.add_argument("--drop", type=int, default=0,
                    help="with --trace-summary: dispatches of each kernel counted as warm-up")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV"), default=None,
                    help="decode|prefill|prefill_d256 and the FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                         "--copy-calibration run: write the traffic JSON under profiles/ and print the summary")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG", default=None,
                    help="KERNEL_PREFIX CSV [CSV ...]: average counters of that kernel (after --drop dispatches) "
                         "over counter_collection CSVs and print the derived figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (scales profiler byte counters)")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.drop))
        return
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary[1:], args.counter_summary[0], args.drop))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design note, "
              "not a built path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import paged_kv_attention_amd as pa
    pa.load_library()
    result = {}
    decode_w = None

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: 1 GiB device copy done", file=sys.stderr, flush=True)

    if args.only in (None, "decode"):
        print("[bench] decode: building inputs", file=sys.stderr, flush=True)
        db = DecodeBench(layers=args.layers, num_splits=args.num_splits)
        # the step: kv_cache_write of the 64 new rows, then paged_attention
        total, per = _time_steps([db.write, db.attend], args.steps, args.warmup)
        ms = total / args.steps
        value = db.attn_bytes / (ms * 1e-3) / 1e9
        kern_ms = per[1]
        kern_spread = _spread(_time_steps.last[1])
        achieved = db.attn_bytes / (kern_ms * 1e-3) / 1e9
        traffic = measured_traffic("decode")
        result.update({
            "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "decode step: 64 seqs x 4096 ctx, 32 q / 8 kv heads, head_dim 128, page 64, "
                                   "bf16; kv_cache_write of 64 new tokens + paged_attention",
                       "pool_layout": "head-major pages [P, Hkv, ps, D]",
                       "seqs": 64, "context": 4096, "q_heads": 32, "kv_heads": 8, "head_dim": 128,
                       "page_size": 64, "splits": db.splits, "pool_sets_rotated": args.layers,
                       "algorithmic_bytes_per_step": db.attn_bytes},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "kernel": "decode_splitkv_kernel<128,1>", "kernel_ms": round(kern_ms, 5),
                         "kernel_ms_median": kern_spread["median"], "kernel_ms_min": kern_spread["min"],
                         "bytes_per_launch": db.attn_bytes},
            "kv_write_ms": round(per[0], 5),
        })
        if args.only is None:
            # the same step as one call: paged_attention with the new rows,
            # which its decode launch writes before reading a key
            total2, per2 = _time_steps([db.step], args.steps, args.warmup)
            result["one_call_step"] = {
                "ms_per_step": round(total2 / args.steps, 5),
                "GB_s": round(db.attn_bytes / (total2 / args.steps * 1e-3) / 1e9, 2),
                "kernel_ms": round(per2[0], 5),
                "note": "paged_attention(k_new, v_new, slot_mapping): one decode launch writes and attends"}
        if not args.no_graph:
            g_ms = graph_step(db, args.steps)
            result["graph_step"] = {"ms_per_step": round(g_ms, 5),
                                    "GB_s": round(db.attn_bytes / (g_ms * 1e-3) / 1e9, 2),
                                    "note": "kv_cache_write + paged_attention of all rotated pool sets captured in one hipGraph"}
        decode_w = db.w
        del db
        torch.cuda.empty_cache()
        if args.only is None:
            ceil = read_ceiling()
            result["read_ceiling"] = {"GB_s": ceil, "decode_frac": round(achieved / ceil, 4),
                                      "how": "library read probe (pa_read_probe): 16-byte streaming loads "
                                             "over a 4 GiB buffer, best of 10"}

    for leg, cfg in (("prefill", 5), ("prefill_d256", 6)):
        if args.only not in (None, leg) or args.no_prefill:
            continue
        print(f"[bench] {leg}: building inputs", file=sys.stderr, flush=True)
        pb = PrefillBench(cfg)
        psteps = max(3, min(args.steps, 10))
        pwarm = max(args.warmup, PREFILL_WARMUP)
        total, per = _time_steps([lambda i: pb.write(), lambda i: pb.attend()], psteps, pwarm)
        kern_ms = per[1]
        kern_spread = _spread(_time_steps.last[1])
        step_ms = total / psteps
        tflops_kernel = pb.flops / (kern_ms * 1e-3) / 1e12
        tflops_step = pb.flops / (step_ms * 1e-3) / 1e12
        w = pb.w
        pre = {"workload": f"causal prefill 4 x 8192, {w.num_q_heads} q / {w.num_kv_heads} kv heads, "
                           f"head_dim {w.head_dim}, page 64, bf16; kv_cache_write of 32768 tokens + paged_attention",
               "steps": psteps, "warmup": pwarm, "ms_per_step": round(step_ms, 4),
               "tflops_step": round(tflops_step, 2),
               "algorithmic_flops": pb.flops,
               "roofline": {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tflops_kernel / BF16_PEAK_TFLOPS, 4),
                            "traffic": measured_traffic(leg) if leg in TRAFFIC_FILES else None,
                            "kernel": "prefill16_kernel<256>" if w.head_dim == 256 else f"prefill_kernel<{w.head_dim}>",
                            "kernel_ms": round(kern_ms, 4), "kernel_ms_median": kern_spread["median"],
                            "kernel_ms_min": kern_spread["min"]}}
        if args.only == leg:
            result.update({"metric": METRIC, "value": round(tflops_kernel, 2), "unit": "TFLOP/s", "n_gpus": 1,
                           "steps": psteps, "warmup": pwarm, "ms_per_step": round(step_ms, 4),
                           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                           "data": "synthetic", "config": {"workload": pre["workload"]},
                           "roofline": pre["roofline"]})
        else:
            result[leg] = pre
        del pb
        torch.cuda.empty_cache()

    if args.only == "mixed":
        # the mixed batch alone (its one launch and the combine), for profiler runs
        print("[bench] mixed batch: building inputs", file=sys.stderr, flush=True)
        wb = WorkloadBench(4, 8)
        entry = _hbm_entry("bf16 mixed batch: 512-token chunk over 1024 prefix + 30 decodes + 5-token verify", wb,
                           args.steps, args.warmup, 8)
        result.update({"metric": METRIC, "value": entry["GB_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                       "warmup": args.warmup, "ms_per_step": entry["gpu_ms"], "higher_is_better": True,
                       "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                       "config": {"workload": entry["workload"]},
                       "roofline": dict(entry["roofline"], traffic=measured_traffic("mixed"))})

    if args.only is None and not args.no_others:
        result["other_workloads"] = other_workloads(args.steps, args.warmup)

    if args.only is None and not args.no_variants:
        result["variants"] = variant_workloads(args.steps, args.warmup)
        print("[bench] cascade: 64 requests sharing a 4096-position prefix", file=sys.stderr, flush=True)
        result["variants"]["cascade_decode"] = cascade_workload(args.steps, args.warmup)

    if not args.no_cpu_baseline and args.only is None and decode_w is not None:
        print("[bench] cpu baseline: timing the float64 oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(decode_w)
        print("[bench] cpu baseline: the oracle on every configuration", file=sys.stderr, flush=True)
        result["cpu_baseline_configs"] = cpu_baseline_configs()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
