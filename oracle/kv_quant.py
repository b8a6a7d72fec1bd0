"""Quantized KV cache reference -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module.  It imports nothing from the HIP library.

What is computed (page "32. Production attention kernels", Quantized KV
caches; page "Attention kernels", INT8 cache):

* Quantize on write, one float32 scale per (token, KV head).  A head vector
  v of D float32 values gets the step ``max(max_d |v_d|, 1e-8) / top``, where
  top is the largest code (127 for int8, 448 for fp8 E4M3); each value is
  divided by the step and stored as the nearest int8 (ties to even, kept
  within +-127) or the nearest E4M3 value (ties to even).  The largest value
  maps onto the edge of the code range, so nothing overflows.  Each of these
  is one float32 operation, taken in this order, so a kernel that takes the
  same operations in float32 reproduces codes and steps bit for bit.
* Key smoothing (page "Attention kernels", INT8 cache: smoothing of the keys
  is compensated on the query side): with per-channel factors
  ``smooth [Hkv, D]`` keys are divided by them (float32) before quantization.  The key a cached code stands for is
  then ``code * scale * smooth``, and the scores are unchanged:
  ``q . (k / s * s) = (q * s) . (k / s)``.  No smoothing means factors of 1.
* The cache is read back as ``code * scale`` (times ``smooth`` for keys),
  exactly, in float64; attention over that read-back is the target the
  quantized kernels are compared with (page "32. Production attention
  kernels", The tests and the measurements: the INT8 and FP8 caches are
  checked against a reference computed from what the cache stores).
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

__all__ = ["KV_QMAX", "KV_CODE_DTYPE", "quantize_head_vectors", "kv_write_quant_ref", "dequantize"]

KV_QMAX = {"int8": 127.0, "fp8": 448.0}
KV_CODE_DTYPE = {"int8": torch.int8, "fp8": torch.float8_e4m3fn}


def _step(v: torch.Tensor, top_code: float) -> torch.Tensor:
    """Float32 step of each head vector (last axis): the vector's largest
    magnitude, never below 1e-8, over the largest code."""
    floor = torch.full((), 1e-8, dtype=torch.float32)
    peak = torch.maximum(v.abs().max(dim=-1).values, floor)
    return peak / torch.tensor(top_code, dtype=torch.float32)


def _to_codes(ratio: torch.Tensor, kind: str) -> torch.Tensor:
    """Float32 multiples of the step -> 1-byte codes: nearest integer (ties to
    even) kept within +-127 for int8; the E4M3 value nearest (ties to even)
    for fp8."""
    if kind == "int8":
        return torch.clamp(torch.round(ratio), -127.0, 127.0).to(torch.int8)
    return ratio.to(torch.float8_e4m3fn)


def quantize_head_vectors(x: torch.Tensor, kind: str,
                          smooth: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """x [T, Hkv, D] -> (codes [T, Hkv, D] int8 / float8_e4m3fn, steps [T, Hkv] float32).

    Each head vector v (float32; keys divided by their smoothing factors
    first) is stored as codes c with v ~ c * step, step as defined above."""
    v = x.to(torch.float32)
    if smooth is not None:
        v = v / smooth.to(torch.float32)[None]
    step = _step(v, KV_QMAX[kind])
    return _to_codes(v / step[..., None], kind), step


def kv_write_quant_ref(k_new, v_new, k_codes, v_codes, k_scale, v_scale, slot_mapping, kind: str,
                       k_smooth: Optional[torch.Tensor] = None):
    """Quantize token i's K/V head vectors and scatter codes and scales to
    flat slot ``slot_mapping[i]`` (page s // ps, offset s % ps); -1 writes
    nothing.  Code pools are [P, ps, Hkv, D], scale pools [P, ps, Hkv].
    Returns new tensors; inputs are not modified."""
    kc, ks = quantize_head_vectors(k_new, kind, k_smooth)
    vc, vs = quantize_head_vectors(v_new, kind)
    out = [t.clone() for t in (k_codes, v_codes, k_scale, v_scale)]
    ps = out[0].shape[1]
    for i, s in enumerate(slot_mapping.tolist()):
        if s < 0:
            continue
        pg, sl = s // ps, s % ps
        # copy through the bytes: a dtype is only an interpretation of them
        out[0].view(torch.uint8)[pg, sl] = kc[i].view(torch.uint8)
        out[1].view(torch.uint8)[pg, sl] = vc[i].view(torch.uint8)
        out[2][pg, sl] = ks[i]
        out[3][pg, sl] = vs[i]
    return tuple(out)


def dequantize(codes: torch.Tensor, scales: torch.Tensor, smooth: Optional[torch.Tensor] = None) -> torch.Tensor:
    """codes [P, ps, Hkv, D], scales [P, ps, Hkv] -> float64 values code * scale (* smooth [Hkv, D])."""
    v = codes.to(torch.float64) * scales.to(torch.float64).unsqueeze(-1)
    if smooth is not None:
        v = v * smooth.to(torch.float64).reshape(1, 1, *smooth.shape)
    return v
