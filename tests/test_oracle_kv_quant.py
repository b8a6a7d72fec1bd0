"""Pins of the quantized-cache oracle (page "32. Production attention
kernels", Quantized KV caches and its printed byte counts; page "Attention
kernels", INT8 cache).  CPU only.

* error bounds: int8 codes reconstruct every element within half a step
  (scale / 2), fp8 within half an E4M3 step (relative 2^-4 of the element's
  binade), and the largest element lands exactly on the code range's edge
  (a wrong q_max, a missing round or clamp fails here);
* the float8 E4M3 conversion against values worked out by hand (448, 1, the
  smallest subnormal, ties to even) -- the library routine the oracle uses;
* key smoothing leaves the scores unchanged: attention over the smoothed,
  dequantized keys with the smoothing multiplied back equals attention over
  the plain dequantized keys up to float64 rounding (a factor applied on the
  wrong side fails here);
* the printed cache sizes: 76,032 bytes per token for Qwen3-8B's 36 layers
  with an int8 cache (8 KV heads x (128 codes + 4 scale bytes) x 2 x 36) and
  13,152 tokens per GB;
* the slot-mapped write: -1 skips, codes and scales land at page s // ps,
  offset s % ps.
"""
import json
import math
import os

import pytest
import torch

from oracle import quantize_head_vectors, kv_write_quant_ref, dequantize, attention_f64, KV_QMAX
from workloads import make_custom

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _x(seed, T=37, Hkv=3, D=64, spread=3.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, Hkv, D, generator=g) * spread
    x[0, 0, 5] = 40.0                  # an outlier channel
    x[1, 1] = 0.0                      # an all-zero head vector
    return x


def test_int8_reconstruction_bound_and_edge():
    x = _x(1)
    codes, scale = quantize_head_vectors(x, "int8")
    assert codes.dtype == torch.int8 and scale.dtype == torch.float32
    rec = codes.double() * scale.double().unsqueeze(-1)
    err = (rec - x.double()).abs()
    assert torch.all(err <= scale.double().unsqueeze(-1) * 0.5 * (1 + 1e-6))
    nz = x.abs().amax(-1) > 0
    top = codes.abs().amax(-1)
    assert torch.all(top[nz] == 127)
    # an all-zero vector keeps the 1e-8 floor and codes 0
    assert scale[1, 1].item() == pytest.approx(1e-8 / 127, rel=1e-6)
    assert torch.all(codes[1, 1] == 0)


def test_fp8_reconstruction_bound_and_edge():
    x = _x(2)
    codes, scale = quantize_head_vectors(x, "fp8")
    assert codes.dtype == torch.float8_e4m3fn
    s = scale.double().unsqueeze(-1)
    vals = codes.double()                                   # in code units
    target = x.double() / s
    # half a step of E4M3: 2^(e-3) / 2 above the subnormal range, 2^-10 below it
    e = torch.floor(torch.log2(target.abs().clamp_min(2.0 ** -6)))
    half = torch.where(target.abs() < 2.0 ** -6, torch.full_like(target, 2.0 ** -10), 2.0 ** (e - 4))
    assert torch.all((vals - target).abs() <= half * (1 + 1e-6) + 1e-12)
    nz = x.abs().amax(-1) > 0
    assert torch.all(codes.float().abs().amax(-1)[nz] == 448.0)


def test_fp8_conversion_hand_values():
    vals = torch.tensor([448.0, 1.0, 2.0 ** -9, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, -3.25, 0.0])
    bits = vals.to(torch.float8_e4m3fn).view(torch.uint8).tolist()
    # 448 = 1.75 * 2^8 -> exponent field 15, mantissa 6; 1.0 -> exponent 7; smallest subnormal -> 1;
    # halfway cases round to even: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2; -3.25 = -1.625 * 2^1 -> 0x80 | 8 << 3 | 5
    assert bits == [0x7E, 0x38, 0x01, 0x00, 0x02, 0x02, 0x80 | (8 << 3) | 5, 0x00]


def test_smoothing_leaves_scores_unchanged():
    Hkv, D = 2, 16
    w = make_custom(seed=21, context_lens=[13, 6], query_lens=[3, 1], num_q_heads=4, num_kv_heads=Hkv, head_dim=D,
                    page_size=4, scale=0.25)
    g = torch.Generator().manual_seed(5)
    smooth = torch.rand(Hkv, D, generator=g) * 3 + 0.25
    P, ps = w.k_pool.shape[:2]
    flat = w.k_pool.reshape(P * ps, Hkv, D)
    c_s, s_s = quantize_head_vectors(flat, "int8", smooth)
    k_smoothed = dequantize(c_s.reshape(P, ps, Hkv, D), s_s.reshape(P, ps, Hkv), smooth)
    # the smoothed cache stands for keys close to the originals ...
    step = (s_s.double().reshape(P, ps, Hkv, 1) * smooth.double().reshape(1, 1, Hkv, D)) * 0.5
    assert torch.all((k_smoothed - w.k_pool.double()).abs() <= step * (1 + 1e-6) + 1e-12)
    # ... and attention over them equals attention with the factors moved onto q
    q_s = (w.q.double().reshape(-1, Hkv, 2, D) * smooth.double().reshape(1, Hkv, 1, D)).reshape(w.q.shape)
    k_div = k_smoothed / smooth.double().reshape(1, 1, Hkv, D)
    a = attention_f64(w.q.double(), k_smoothed, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    b = attention_f64(q_s, k_div, w.v_pool, w.block_tables, w.context_lens, w.query_start_loc, w.scale)
    assert torch.max(torch.abs(a - b)).item() <= 1e-12


def test_printed_cache_sizes():
    layers, Hkv, D = 36, 8, 128
    int8_bytes = layers * 2 * Hkv * (D * 1 + 4)             # codes plus one float32 scale per head vector
    assert int8_bytes == GOLD["qwen3_8b_int8_bytes_per_token_36_layers"]["value"]
    assert int(1e9 // int8_bytes) == GOLD["qwen3_8b_int8_tokens_per_GB"]["value"]


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_write_map(kind):
    P, ps, Hkv, D = 5, 4, 2, 8
    dt = torch.int8 if kind == "int8" else torch.float8_e4m3fn
    kc = torch.zeros(P, ps, Hkv, D, dtype=dt)
    vc = torch.zeros_like(kc)
    ks = torch.zeros(P, ps, Hkv)
    vs = torch.zeros(P, ps, Hkv)
    g = torch.Generator().manual_seed(3)
    kn = torch.randn(4, Hkv, D, generator=g)
    vn = torch.randn(4, Hkv, D, generator=g)
    slots = torch.tensor([7, -1, 0, 19], dtype=torch.int32)
    kc2, vc2, ks2, vs2 = kv_write_quant_ref(kn, vn, kc, vc, ks, vs, slots, kind)
    c, s = quantize_head_vectors(kn, kind)
    for i, sl in enumerate(slots.tolist()):
        if sl < 0:
            continue
        assert torch.equal(kc2[sl // ps, sl % ps].view(torch.uint8), c[i].view(torch.uint8))
        assert torch.equal(ks2[sl // ps, sl % ps], s[i])
    written = {7, 0, 19}
    for sl in range(P * ps):
        if sl not in written:
            assert torch.all(kc2[sl // ps, sl % ps].view(torch.uint8) == 0) and torch.all(ks2[sl // ps, sl % ps] == 0)
