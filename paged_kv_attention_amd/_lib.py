"""ctypes binding of libpagedattn.so (argument marshalling only).

Every step of the attention path runs in the HIP kernels of the library; this
module only turns torch tensors into pointers, strides and the ``pa_dims``
block, passes the current HIP stream, and raises on a non-OK status.  There is
no fallback: if the library is missing, importing the functions fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

(PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH, PA_ERR_INVALID_DATA,
 PA_ERR_SCRATCH_LIMIT) = range(8)
# bytes of the library's static device buffer used by paged_attention_noalloc
STATIC_SCRATCH_BYTES = 32 << 20
PA_F32, PA_BF16 = 0, 1

EXPORTED = ("paged_attention", "paged_attention_opts", "paged_attention_noalloc", "kv_cache_write", "kv_cache_write_quant", "pa_workspace_size",
            "pa_workspace_size_opts", "pa_choose_splits", "pa_validate", "pa_validate_opts", "pa_status_string",
            "pa_device_cu_count", "pa_read_probe")


class PaDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("max_query_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("table_width", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
        ("kv_stride_page", ctypes.c_int64), ("kv_stride_slot", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
    ]


class PaKvQuant(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("scale_stride_page", ctypes.c_int64),
                ("scale_stride_slot", ctypes.c_int64), ("scale_stride_head", ctypes.c_int64),
                ("k_smooth", ctypes.c_void_p)]


class PaAttnOpts(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("sinks", ctypes.c_void_p),
                ("kv_quant", ctypes.POINTER(PaKvQuant)), ("shared_prefix_len", ctypes.c_int32),
                ("reserved1", ctypes.c_int32), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("slot_mapping", ctypes.c_void_p), ("new_stride_tok", ctypes.c_int64),
                ("new_stride_head", ctypes.c_int64)]


PA_KV_INT8, PA_KV_FP8_E4M3 = 1, 2
_KV_KIND = {"int8": PA_KV_INT8, "fp8": PA_KV_FP8_E4M3}
CODE_DTYPES = (torch.int8, torch.uint8, torch.float8_e4m3fn)


class KvQuant:
    """A quantized cache's side data: ``kind`` "int8" or "fp8" (E4M3), the K
    and V scale pools (float32 ``[P, ps, Hkv]`` views, any strides, the same
    for both) and optional key smoothing factors (float32 ``[Hkv, D]``)."""

    def __init__(self, kind: str, k_scale: torch.Tensor, v_scale: torch.Tensor,
                 k_smooth: Optional[torch.Tensor] = None):
        if kind not in _KV_KIND:
            raise ValueError(f"kind must be int8 or fp8, not {kind!r}")
        if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32 or k_scale.dim() != 3:
            raise TypeError("scale pools must be float32 [P, ps, Hkv]")
        if k_scale.shape != v_scale.shape or k_scale.stride() != v_scale.stride():
            raise ValueError("k_scale and v_scale must have the same shape and strides")
        if k_smooth is not None:
            if k_smooth.dtype != torch.float32 or k_smooth.dim() != 2:
                raise TypeError("k_smooth must be float32 [Hkv, D]")
            k_smooth = k_smooth.contiguous()
        self.kind, self.k_scale, self.v_scale, self.k_smooth = kind, k_scale, v_scale, k_smooth

    def struct(self) -> PaKvQuant:
        q = PaKvQuant()
        q.kv_dtype = _KV_KIND[self.kind]
        q.k_scale, q.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
        q.scale_stride_page, q.scale_stride_slot, q.scale_stride_head = self.k_scale.stride()
        q.k_smooth = self.k_smooth.data_ptr() if self.k_smooth is not None else None
        return q


def empty_code_pool(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int, kind: str = "int8",
                    device="cuda", layout: str = "head_major") -> torch.Tensor:
    """A 1-byte code pool (int8, or float8_e4m3fn for "fp8") as a ``[P, ps, Hkv, D]`` view."""
    dt = torch.int8 if kind == "int8" else torch.float8_e4m3fn
    return empty_pool(num_pages, page_size, num_kv_heads, head_dim, dtype=dt, device=device, layout=layout)


def empty_scale_pool(num_pages: int, page_size: int, num_kv_heads: int, device="cuda",
                     layout: str = "head_major") -> torch.Tensor:
    """A float32 scale pool as a ``[P, ps, Hkv]`` view (``[P, Hkv, ps]`` in memory for "head_major")."""
    if layout == "head_major":
        return torch.empty(num_pages, num_kv_heads, page_size, dtype=torch.float32, device=device).permute(0, 2, 1)
    if layout == "interleaved":
        return torch.empty(num_pages, page_size, num_kv_heads, dtype=torch.float32, device=device)
    raise ValueError(f"unknown pool layout {layout!r}")


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_attention_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    lib.paged_attention.restype = ctypes.c_int
    lib.paged_attention.argtypes = [vp, vp, vp, i32p, i32p, i32p, ctypes.c_float, ctypes.c_int, vp, vp,
                                    ctypes.c_size_t, ctypes.POINTER(PaDims), ctypes.c_int, vp]
    lib.paged_attention_opts.restype = ctypes.c_int
    lib.paged_attention_opts.argtypes = [vp, vp, vp, i32p, i32p, i32p, ctypes.c_float, ctypes.c_int, vp, vp,
                                         ctypes.c_size_t, ctypes.POINTER(PaDims), ctypes.c_int,
                                         ctypes.POINTER(PaAttnOpts), vp]
    lib.paged_attention_noalloc.restype = ctypes.c_int
    lib.paged_attention_noalloc.argtypes = [vp, vp, vp, i32p, i32p, i32p, ctypes.c_float, ctypes.c_int, vp,
                                            ctypes.POINTER(PaDims), ctypes.c_int, vp]
    lib.kv_cache_write_quant.restype = ctypes.c_int
    lib.kv_cache_write_quant.argtypes = [vp, vp, vp, vp, i32p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.POINTER(PaDims), ctypes.c_int, ctypes.POINTER(PaKvQuant), vp]
    lib.kv_cache_write.restype = ctypes.c_int
    lib.kv_cache_write.argtypes = [vp, vp, vp, vp, i32p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.POINTER(PaDims), ctypes.c_int, vp]
    lib.pa_workspace_size.restype = ctypes.c_size_t
    lib.pa_workspace_size.argtypes = [ctypes.POINTER(PaDims), ctypes.c_int]
    lib.pa_workspace_size_opts.restype = ctypes.c_size_t
    lib.pa_workspace_size_opts.argtypes = [ctypes.POINTER(PaDims), ctypes.c_int, ctypes.POINTER(PaAttnOpts)]
    lib.pa_validate_opts.restype = ctypes.c_int
    lib.pa_validate_opts.argtypes = [i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(PaDims),
                                     ctypes.POINTER(PaAttnOpts), vp]
    lib.pa_choose_splits.restype = ctypes.c_int32
    lib.pa_choose_splits.argtypes = [ctypes.POINTER(PaDims)]
    lib.pa_validate.restype = ctypes.c_int
    lib.pa_validate.argtypes = [i32p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_int, ctypes.POINTER(PaDims), vp]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_device_cu_count.restype = ctypes.c_int32
    lib.pa_device_cu_count.argtypes = []
    lib.pa_read_probe.restype = ctypes.c_int
    lib.pa_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return PA_F32
    if t == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t}: float32 or bfloat16")


# The current device's current stream as a raw pointer, without building a
# torch Stream object (0.35 us per call against 2.8 us through
# torch.cuda.current_stream() on the GPU host).
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream) -> int:
    if stream is None:
        if _RAW_STREAM is not None:
            return _RAW_STREAM(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# Dims structs (and their plain workspace sizes) of recent call shapes: a
# serving loop repeats a few shapes, and building the struct field by field
# is most of the binding's host time.  The cached struct is never modified.
_DIMS_CACHE: dict = {}


def _cached_dims(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor, out: torch.Tensor,
                 max_query_len: Optional[int], num_splits: int):
    key = (q.shape, q.stride(), q.dtype, k_pool.shape, k_pool.stride(), block_tables.shape, out.stride(),
           max_query_len, num_splits)
    hit = _DIMS_CACHE.get(key)
    if hit is None:
        d = make_dims(q, k_pool, block_tables, out=out, max_query_len=max_query_len, num_splits=num_splits)
        need = int(load_library().pa_workspace_size(ctypes.byref(d), _dtype_code(q.dtype)))
        if len(_DIMS_CACHE) >= 256:
            _DIMS_CACHE.clear()
        hit = _DIMS_CACHE[key] = (d, need)
    return hit


def make_dims(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor, *, out: Optional[torch.Tensor] = None,
              max_query_len: Optional[int] = None, num_splits: int = 0) -> PaDims:
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [N, Hq, D] and the pools [P, ps, Hkv, D]")
    N, Hq, D = q.shape
    P, ps, Hkv, Dk = k_pool.shape
    if Dk != D:
        raise ValueError(f"head_dim mismatch: q has {D}, pools have {Dk}")
    if q.stride(2) != 1 or k_pool.stride(3) != 1 or (out is not None and out.stride(2) != 1):
        raise ValueError("the head dimension must be contiguous")
    o = out if out is not None else q
    d = PaDims()
    d.num_seqs = int(block_tables.shape[0])
    d.num_tokens = int(N)
    d.max_query_len = int(max_query_len or 0)
    d.num_q_heads, d.num_kv_heads, d.head_dim = int(Hq), int(Hkv), int(D)
    d.page_size, d.num_pages, d.table_width = int(ps), int(P), int(block_tables.shape[1])
    d.num_splits = int(num_splits)
    d.q_stride_tok, d.q_stride_head = q.stride(0), q.stride(1)
    d.o_stride_tok, d.o_stride_head = o.stride(0), o.stride(1)
    d.kv_stride_page, d.kv_stride_slot, d.kv_stride_head = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    return d


def empty_pool(num_pages: int, page_size: int, num_kv_heads: int, head_dim: int, dtype=torch.bfloat16,
               device="cuda", layout: str = "head_major") -> torch.Tensor:
    """Allocate one K or V pool and return it as a ``[P, ps, Hkv, D]`` view.

    ``layout="head_major"`` stores each page as ``Hkv`` dense ``[ps, D]`` tiles
    (``[P, Hkv, ps, D]`` in memory), so one (page, KV head) is one contiguous
    run of ``ps * D`` elements; this is the layout the decode kernel reads
    fastest.  ``layout="interleaved"`` stores ``[P, ps, Hkv, D]`` as is.
    """
    if layout == "head_major":
        return torch.empty(num_pages, num_kv_heads, page_size, head_dim, dtype=dtype, device=device).permute(0, 2, 1, 3)
    if layout == "interleaved":
        return torch.empty(num_pages, page_size, num_kv_heads, head_dim, dtype=dtype, device=device)
    raise ValueError(f"unknown pool layout {layout!r}")


def pool_like(pool: torch.Tensor, device="cuda", layout: str = "head_major") -> torch.Tensor:
    """Copy a logical ``[P, ps, Hkv, D]`` pool into device memory in the given layout."""
    out = empty_pool(*pool.shape[:1], pool.shape[1], pool.shape[2], pool.shape[3], dtype=pool.dtype, device=device,
                     layout=layout)
    out.copy_(pool)
    return out


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32 (convert int64 metadata once, outside timed regions)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def workspace_size(dims: PaDims, dtype: torch.dtype) -> int:
    return int(load_library().pa_workspace_size(ctypes.byref(dims), _dtype_code(dtype)))


def choose_splits(dims: PaDims) -> int:
    return int(load_library().pa_choose_splits(ctypes.byref(dims)))


def device_cu_count() -> int:
    return int(load_library().pa_device_cu_count())


def paged_attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, query_start_loc: torch.Tensor, scale: Optional[float] = None,
                    causal: bool = True, *, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, max_query_len: Optional[int] = None,
                    num_splits: int = 0, window: int = 0, sinks: Optional[torch.Tensor] = None,
                    kv_quant: Optional[KvQuant] = None, shared_prefix_len: int = 0,
                    k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                    slot_mapping: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal GQA attention of q over the paged pools; returns ``out`` [N, Hq, D].

    ``scale`` defaults to 1/sqrt(D).  ``max_query_len`` is a host bound on any
    sequence's query tokens (default N); ``num_splits`` 0 picks the split count.
    ``window`` > 0 is a sliding window (a row sees its last ``window``
    positions) and ``sinks`` a float32 [Hq] device tensor of sink logits; with
    either set the call goes through ``paged_attention_opts``.  With
    ``kv_quant`` the pools are 1-byte code pools (int8 / float8_e4m3fn) and
    q must be bfloat16.  ``shared_prefix_len`` > 0 runs cascade attention
    over a prefix every sequence shares (same first pages, queries after it).
    ``k_new`` / ``v_new`` ([N, Hkv, D], q's dtype) with ``slot_mapping`` (int32
    [N]) write the step's new rows into the pools before attending, as
    ``kv_cache_write`` would; a batch of decode tokens alone does the write
    inside its decode launch.
    """
    lib = load_library()
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    if kv_quant is not None:
        if k_pool.dtype not in CODE_DTYPES or v_pool.dtype not in CODE_DTYPES:
            raise TypeError("quantized pools hold 1-byte codes (int8 or float8_e4m3fn)")
    elif q.dtype != k_pool.dtype or q.dtype != v_pool.dtype:
        raise TypeError("q and the pools must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    dims, need_plain = _cached_dims(q, k_pool, block_tables, out, max_query_len, num_splits)
    bt = _i32(block_tables, "block_tables")
    cl = _i32(context_lens, "context_lens")
    qsl = _i32(query_start_loc, "query_start_loc")
    code = _dtype_code(q.dtype)
    opts = None
    if k_new is not None:
        if v_new is None or slot_mapping is None:
            raise ValueError("k_new needs v_new and slot_mapping")
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dim() != 3:
            raise ValueError("k_new and v_new must be [N, Hkv, D] with the same strides")
        if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
            raise TypeError("new rows must have q's dtype")
        if k_new.stride(2) != 1:
            raise ValueError("the head dimension of the new rows must be contiguous")
        if k_new.shape[0] != q.shape[0] or tuple(k_new.shape[1:]) != (k_pool.shape[2], k_pool.shape[3]):
            raise ValueError("k_new must be [N, Hkv, D]: one new row per query token and KV head")
        slot_mapping = _i32(slot_mapping, "slot_mapping")
    if window or sinks is not None or kv_quant is not None or shared_prefix_len or k_new is not None:
        if sinks is not None:
            if sinks.dtype != torch.float32 or sinks.device != q.device or sinks.numel() != q.shape[1]:
                raise ValueError("sinks must be a float32 tensor of num_q_heads values on q's device")
            sinks = sinks.contiguous()
        kq = kv_quant.struct() if kv_quant is not None else None
        opts = PaAttnOpts(int(window), 0, sinks.data_ptr() if sinks is not None else None,
                          ctypes.pointer(kq) if kq is not None else None, int(shared_prefix_len), 0)
        if k_new is not None:
            opts.k_new, opts.v_new, opts.slot_mapping = k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr()
            opts.new_stride_tok, opts.new_stride_head = k_new.stride(0), k_new.stride(1)
        need = int(lib.pa_workspace_size_opts(ctypes.byref(dims), code, ctypes.byref(opts)))
    else:
        need = need_plain
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if opts is not None:
        st = lib.paged_attention_opts(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), bt.data_ptr(),
                                      cl.data_ptr(), qsl.data_ptr(), float(scale), 1 if causal else 0,
                                      out.data_ptr(), ws_ptr, ws_bytes, ctypes.byref(dims), code,
                                      ctypes.byref(opts), _stream_ptr(stream))
    else:
        st = lib.paged_attention(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), bt.data_ptr(), cl.data_ptr(),
                                 qsl.data_ptr(), float(scale), 1 if causal else 0, out.data_ptr(), ws_ptr, ws_bytes,
                                 ctypes.byref(dims), code, _stream_ptr(stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attention")
    return out


def paged_attention_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                            scale: Optional[float] = None, causal: bool = True, *, out: torch.Tensor,
                            max_query_len: Optional[int] = None, num_splits: int = 0, stream=None) -> torch.Tensor:
    """``paged_attention`` without a workspace: the split partials go to the
    library's static device buffer (``STATIC_SCRATCH_BYTES`` per device), so
    the call allocates nothing.  ``out`` must be given.  Calls that overlap in
    time on one device race on that buffer."""
    lib = load_library()
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    if q.dtype != k_pool.dtype or q.dtype != v_pool.dtype or out.dtype != q.dtype:
        raise TypeError("q, out and the pools must share one dtype")
    dims = make_dims(q, k_pool, block_tables, out=out, max_query_len=max_query_len, num_splits=num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    st = lib.paged_attention_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                     _i32(block_tables, "block_tables").data_ptr(),
                                     _i32(context_lens, "context_lens").data_ptr(),
                                     _i32(query_start_loc, "query_start_loc").data_ptr(), float(scale),
                                     1 if causal else 0, out.data_ptr(), ctypes.byref(dims), _dtype_code(q.dtype),
                                     _stream_ptr(stream))
    if st != PA_OK:
        raise PagedAttnError(st, "paged_attention_noalloc")
    return out


READ_PROBE_SINK_BYTES = 65536


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream ``buf`` (a contiguous device tensor) once through the library's
    read probe; ``sink`` is a device tensor of at least 65536 bytes.  A
    measurement aid for the HBM read ceiling, not part of attention."""
    if not buf.is_contiguous() or not sink.is_contiguous():
        raise ValueError("buf and sink must be contiguous")
    st = load_library().pa_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                      sink.numel() * sink.element_size(), _stream_ptr(stream))
    if st != PA_OK:
        raise PagedAttnError(st, "pa_read_probe")


def kv_cache_write(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter k_new/v_new [T, Hkv, D] into the pools at slot_mapping[T] (-1 = skip)."""
    lib = load_library()
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must have the same shape and strides")
    if k_new.dtype != k_pool.dtype:
        raise TypeError("new rows and pools must share one dtype")
    if k_new.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous")
    dims = PaDims()
    P, ps, Hkv, D = k_pool.shape
    dims.num_kv_heads, dims.head_dim, dims.page_size, dims.num_pages = int(Hkv), int(D), int(ps), int(P)
    dims.kv_stride_page, dims.kv_stride_slot, dims.kv_stride_head = k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)
    sm = _i32(slot_mapping, "slot_mapping")
    st = lib.kv_cache_write(k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), sm.data_ptr(),
                            int(k_new.shape[0]), k_new.stride(0), k_new.stride(1), ctypes.byref(dims),
                            _dtype_code(k_new.dtype), _stream_ptr(stream))
    if st != PA_OK:
        raise PagedAttnError(st, "kv_cache_write")


def kv_cache_write_quant(k_new: torch.Tensor, v_new: torch.Tensor, k_codes: torch.Tensor, v_codes: torch.Tensor,
                         slot_mapping: torch.Tensor, kv_quant: KvQuant, stream=None) -> None:
    """Quantize k_new/v_new [T, Hkv, D] (bf16 or float32) into the code and
    scale pools at slot_mapping[T] (-1 = skip)."""
    lib = load_library()
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must have the same shape and strides")
    if k_new.stride(2) != 1:
        raise ValueError("the head dimension must be contiguous")
    if k_codes.dtype not in CODE_DTYPES or k_codes.shape != v_codes.shape or k_codes.stride() != v_codes.stride():
        raise TypeError("code pools must be matching 1-byte [P, ps, Hkv, D] tensors")
    dims = PaDims()
    P, ps, Hkv, D = k_codes.shape
    dims.num_kv_heads, dims.head_dim, dims.page_size, dims.num_pages = int(Hkv), int(D), int(ps), int(P)
    dims.kv_stride_page, dims.kv_stride_slot, dims.kv_stride_head = k_codes.stride(0), k_codes.stride(1), k_codes.stride(2)
    sm = _i32(slot_mapping, "slot_mapping")
    kq = kv_quant.struct()
    st = lib.kv_cache_write_quant(k_new.data_ptr(), v_new.data_ptr(), k_codes.data_ptr(), v_codes.data_ptr(),
                                  sm.data_ptr(), int(k_new.shape[0]), k_new.stride(0), k_new.stride(1),
                                  ctypes.byref(dims), _dtype_code(k_new.dtype), ctypes.byref(kq), _stream_ptr(stream))
    if st != PA_OK:
        raise PagedAttnError(st, "kv_cache_write_quant")


def validate(block_tables: torch.Tensor, context_lens: torch.Tensor, query_start_loc: torch.Tensor, *,
             num_tokens: int, page_size: int, num_pages: int, slot_mapping: Optional[torch.Tensor] = None,
             causal: bool = True, window: int = 0, shared_prefix_len: int = 0, stream=None) -> int:
    """Synchronous metadata check (debug/test only); returns the status code.
    With ``shared_prefix_len`` it also checks the shared-prefix contract."""
    lib = load_library()
    dims = PaDims()
    dims.num_seqs = int(block_tables.shape[0])
    dims.table_width = int(block_tables.shape[1])
    dims.num_tokens = int(num_tokens)
    dims.page_size, dims.num_pages = int(page_size), int(num_pages)
    sm_ptr, ns = (None, 0)
    if slot_mapping is not None:
        sm = _i32(slot_mapping, "slot_mapping")
        sm_ptr, ns = sm.data_ptr(), int(sm.numel())
    opts = PaAttnOpts(int(window), 0, None, None, int(shared_prefix_len), 0)
    return int(lib.pa_validate_opts(_i32(block_tables, "block_tables").data_ptr(),
                                    _i32(context_lens, "context_lens").data_ptr(),
                                    _i32(query_start_loc, "query_start_loc").data_ptr(), sm_ptr, ns,
                                    1 if causal else 0, ctypes.byref(dims), ctypes.byref(opts), _stream_ptr(stream)))
