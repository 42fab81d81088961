"""ctypes binding of libwf (include/wf.h), argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into device pointers, Python lists into host arrays and the
current torch stream into a hipStream_t, and raises WFError on a non-zero
status.  torch provides device memory and streams, nothing else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwf.so")

WF_OK, WF_ERR_INVALID, WF_ERR_UNSUPPORTED, WF_ERR_HIP = 0, -1, -2, -3
WF_BF16, WF_FP32 = 0, 1
WF_STATUS_BAD_PAGE = 1


class WFError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libwf error {code}: {msg}")
        self.code = code


class wf_kv_pool(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("num_logical_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class wf_rope(ctypes.Structure):
    _fields_ = [("d_t", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32),
                ("theta", ctypes.c_double)]


class wf_kv_run(ctypes.Structure):
    _fields_ = [("kv_start", ctypes.c_int32), ("kv_len", ctypes.c_int32)]


class wf_query_group(ctypes.Structure):
    _fields_ = [("q_row_start", ctypes.c_int32), ("q_row_end", ctypes.c_int32),
                ("run_begin", ctypes.c_int32), ("run_end", ctypes.c_int32)]


class wf_mx_keys(ctypes.Structure):
    _fields_ = [("k8_pages", ctypes.c_void_p), ("k8_scales", ctypes.c_void_p)]


class wf_segment(ctypes.Structure):
    _fields_ = [("kv_start", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("slot", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libwf.so (built in-tree by chunk_wise_causal_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m chunk_wise_causal_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.wf_kv_publish.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_rope),
                                    vp, i64, vp, i64, vp, i32, i32, vp, i64, vp]
        L.wf_kv_publish.restype = ctypes.c_int
        L.wf_chunk_attn.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_segment), i32,
                                    vp, i64, ctypes.POINTER(i32), i32, i32, ctypes.c_float,
                                    vp, i64, vp, vp]
        L.wf_chunk_attn.restype = ctypes.c_int
        L.wf_group_attn.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_kv_run), i32,
                                    ctypes.POINTER(wf_query_group), i32, vp, i64, ctypes.c_float,
                                    vp, i64, vp, i64, vp]
        L.wf_group_attn.restype = ctypes.c_int
        L.wf_kv_publish_mx.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_mx_keys),
                                       ctypes.POINTER(wf_rope), vp, i64, vp, i64, vp, i32, i32,
                                       vp, i64, vp]
        L.wf_kv_publish_mx.restype = ctypes.c_int
        L.wf_chunk_attn_mx.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_mx_keys),
                                       ctypes.POINTER(wf_segment), i32, vp, i64,
                                       ctypes.POINTER(i32), i32, i32, ctypes.c_float, vp, i64,
                                       vp, vp]
        L.wf_chunk_attn_mx.restype = ctypes.c_int
        L.wf_qkv_publish.argtypes = [ctypes.POINTER(wf_kv_pool), ctypes.POINTER(wf_rope), vp, i64,
                                     i32, vp, vp, vp, i32, i32, vp, i64, vp]
        L.wf_qkv_publish.restype = ctypes.c_int
        L.wf_history_rotate.argtypes = [vp, i32, i32, i32, i32, i32, vp]
        L.wf_history_rotate.restype = ctypes.c_int
        L.wf_last_error.restype = ctypes.c_char_p
        L.wf_last_error.argtypes = []
        L.wf_version.restype = ctypes.c_char_p
        L.wf_version.argtypes = []
        L.wf_device_status.argtypes = [ctypes.POINTER(i32), i32]
        L.wf_device_status.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != WF_OK:
        raise WFError(rc, lib().wf_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _row_stride(t: torch.Tensor, name: str) -> int:
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: expected [rows, heads, head_dim] with contiguous rows")
    return t.stride(0)


# ---- argument checks the C side cannot make --------------------------------
# The library sees raw pointers: it checks strides, alignment and NULLs, but
# not where a buffer lives, its element type or how many rows it holds.  These
# checks run before any library call, so a bad argument raises ValueError
# instead of sending a host pointer or a short buffer to a kernel.  Shape and
# type checks come first, the device check last.

def _on_device(t: torch.Tensor, dev: torch.device, name: str) -> None:
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name}: must be a GPU tensor on {dev}, got {t.device}")


def _pool_device(pool: "KVPool") -> torch.device:
    dev = pool.k_pages.device
    if not pool.k_pages.is_cuda:
        raise ValueError(f"pool: page arrays must be GPU tensors, got {dev}")
    for t, name in ((pool.v_pages, "pool.v_pages"), (pool.page_table, "pool.page_table")):
        _on_device(t, dev, name)
    return dev


def _head_rows(pool: "KVPool", t: torch.Tensor, name: str, rows: int) -> int:
    """t is [>= rows, H, D] of the pool's element type with contiguous rows;
    returns its row stride (elements)."""
    H, D = pool.desc.num_heads, pool.desc.head_dim
    if t.dim() != 3 or tuple(t.shape[1:]) != (H, D):
        raise ValueError(f"{name}: expected [rows, {H}, {D}], got {list(t.shape)}")
    if t.dtype != pool.k_pages.dtype:
        raise ValueError(f"{name}: dtype {t.dtype} differs from the pool's {pool.k_pages.dtype}")
    if t.shape[0] < rows:
        raise ValueError(f"{name}: {t.shape[0]} rows, the call reads or writes {rows}")
    return _row_stride(t, name)


def _positions(pos: Optional[torch.Tensor], n: int, rope) -> None:
    if pos is None:
        if rope is not None and n > 0:
            raise ValueError("pos: required with rope")
        return
    if pos.dtype != torch.int32 or not pos.is_contiguous() or tuple(pos.shape) != (n, 3):
        raise ValueError(f"pos must be a contiguous int32 [{n}, 3] tensor, got "
                         f"{pos.dtype} {list(pos.shape)}")


def _lse(lse: torch.Tensor, H: int, rows: int, exact: bool) -> int:
    """lse is float32 [H, n] with contiguous rows and n == rows (exact) or
    n >= rows; returns its row stride."""
    if lse.dim() != 2 or lse.dtype != torch.float32 or lse.stride(1) != 1:
        raise ValueError("lse: expected [heads, n] float32 with contiguous rows")
    if lse.shape[0] != H or (lse.shape[1] != rows if exact else lse.shape[1] < rows):
        want = f"[{H}, {rows}]" if exact else f"[{H}, >= {rows}]"
        raise ValueError(f"lse: expected {want}, got {list(lse.shape)}")
    if exact and rows > 0 and lse.stride(0) != rows:   # (torch gives [H, 0] a stride of 1)
        raise ValueError("lse: expected a contiguous [heads, rows] tensor")
    return lse.stride(0)


class KVPool:
    """A paged K/V pool in device memory (layout of include/wf.h):
    k_pages [num_pages, H, page_size, D], v_pages [num_pages, H, D, page_size]
    and the page table [num_logical_pages] (int32)."""

    def __init__(self, k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor):
        n, H, ps, D = k_pages.shape
        if tuple(v_pages.shape) != (n, H, D, ps):
            raise ValueError("v_pages must be [num_pages, H, D, page_size]")
        if page_table.dtype != torch.int32 or page_table.dim() != 1:
            raise ValueError("page_table must be a 1-D int32 tensor")
        if not (k_pages.is_contiguous() and v_pages.is_contiguous() and page_table.is_contiguous()):
            raise ValueError("pool tensors must be contiguous")
        self.k_pages, self.v_pages, self.page_table = k_pages, v_pages, page_table
        self.dtype = {torch.bfloat16: WF_BF16, torch.float32: WF_FP32}[k_pages.dtype]
        self.desc = wf_kv_pool(k_pages.data_ptr(), v_pages.data_ptr(), page_table.data_ptr(),
                               n, page_table.numel(), ps, H, D, self.dtype)

    @classmethod
    def empty(cls, num_pages: int, heads: int, page_size: int, head_dim: int,
              page_table: torch.Tensor, dtype=torch.bfloat16, device="cuda", fill=None):
        k = torch.empty(num_pages, heads, page_size, head_dim, dtype=dtype, device=device)
        v = torch.empty(num_pages, heads, head_dim, page_size, dtype=dtype, device=device)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        return cls(k, v, page_table.to(device=device, dtype=torch.int32).contiguous())

    @property
    def page_size(self) -> int:
        return self.desc.page_size


def wf_kv_publish(pool: KVPool, k: torch.Tensor, v: torch.Tensor, dst_start: int,
                  pos: Optional[torch.Tensor] = None,
                  rope: Optional[Tuple[Tuple[int, int, int], float]] = None,
                  q: Optional[torch.Tensor] = None, stream=None) -> None:
    """RoPE K (and q, in place) with `pos` and scatter K, V into the pool at
    logical rows dst_start.. (C: wf_kv_publish)."""
    n = k.shape[0] if k.dim() > 0 else 0
    ks = _head_rows(pool, k, "k", n)
    vs = _head_rows(pool, v, "v", n)
    qs = _head_rows(pool, q, "q", n) if q is not None else 0
    _positions(pos, n, rope)
    dev = _pool_device(pool)
    for t, name in ((k, "k"), (v, "v"), (q, "q"), (pos, "pos")):
        if t is not None:
            _on_device(t, dev, name)
    r = None
    if rope is not None:
        (dt, dh, dw), theta = rope
        r = wf_rope(dt, dh, dw, float(theta))
    rc = lib().wf_kv_publish(ctypes.byref(pool.desc), ctypes.byref(r) if r else None,
                             _ptr(k), ks, _ptr(v), vs, _ptr(pos), n, dst_start,
                             _ptr(q), qs, _stream(stream))
    _check(rc)


def wf_chunk_attn(pool: KVPool, segments: Sequence[Tuple[int, int, int]], q: torch.Tensor,
                  q_slot_start: Sequence[int], first_slot: int = 0,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunk-wise causal attention of the query slots over the pool
    (C: wf_chunk_attn).  Returns `out` ([rows, H, D], allocated if None);
    lse, if given, is float32 [H, q_slot_start[-1]]."""
    rows = int(q_slot_start[-1]) if len(q_slot_start) else 0
    qs = _head_rows(pool, q, "q", rows)
    if out is None:
        out = torch.empty_like(q)
    os_ = _head_rows(pool, out, "out", rows)
    if lse is not None:
        _lse(lse, pool.desc.num_heads, rows, exact=True)
    dev = _pool_device(pool)
    for t, name in ((q, "q"), (out, "out"), (lse, "lse")):
        if t is not None:
            _on_device(t, dev, name)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    segs = (wf_segment * len(segments))(*[wf_segment(*s) for s in segments])
    qss = (ctypes.c_int32 * len(q_slot_start))(*q_slot_start)
    rc = lib().wf_chunk_attn(ctypes.byref(pool.desc), segs, len(segments), _ptr(q), qs, qss,
                             len(q_slot_start) - 1, first_slot, float(scale), _ptr(out), os_,
                             _ptr(lse), _stream(stream))
    _check(rc)
    return out


def wf_group_attn(pool: KVPool, runs: Sequence[Tuple[int, int]],
                  groups: Sequence[Tuple[int, int, int, int]], q: torch.Tensor,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention of arbitrary query groups over the pool (C: wf_group_attn).
    runs: (kv_start, kv_len); groups: (q_row_start, q_row_end, run_begin,
    run_end).  lse, if given, is [H, n] float32 with n >= every q_row_end.
    Returns `out` ([rows, H, D], allocated if None)."""
    rows = max([int(g[1]) for g in groups], default=0)
    qs = _head_rows(pool, q, "q", rows)
    if out is None:
        out = torch.empty_like(q)
    os_ = _head_rows(pool, out, "out", rows)
    lse_stride = _lse(lse, pool.desc.num_heads, rows, exact=False) if lse is not None else 0
    dev = _pool_device(pool)
    for t, name in ((q, "q"), (out, "out"), (lse, "lse")):
        if t is not None:
            _on_device(t, dev, name)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    rs = (wf_kv_run * len(runs))(*[wf_kv_run(*r) for r in runs])
    gs = (wf_query_group * len(groups))(*[wf_query_group(*g) for g in groups])
    rc = lib().wf_group_attn(ctypes.byref(pool.desc), rs, len(runs), gs, len(groups), _ptr(q),
                             qs, float(scale), _ptr(out), os_, _ptr(lse), lse_stride,
                             _stream(stream))
    _check(rc)
    return out


class MXKeys:
    """MXFP8 keys beside a pool (layout of include/wf.h): codes
    [num_pages, H, page_size, D] uint8 and scales [num_pages, H, page_size,
    D // 32] uint8."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
            raise ValueError("MX keys are uint8 tensors")
        n, H, ps, D = codes.shape
        if tuple(scales.shape) != (n, H, ps, D // 32):
            raise ValueError("scales must be [num_pages, H, page_size, head_dim // 32]")
        if not (codes.is_contiguous() and scales.is_contiguous()):
            raise ValueError("MX key tensors must be contiguous")
        self.codes, self.scales = codes, scales
        self.desc = wf_mx_keys(codes.data_ptr(), scales.data_ptr())

    @classmethod
    def empty(cls, num_pages: int, heads: int, page_size: int, head_dim: int, device="cuda"):
        return cls(torch.empty(num_pages, heads, page_size, head_dim, dtype=torch.uint8,
                               device=device),
                   torch.empty(num_pages, heads, page_size, head_dim // 32, dtype=torch.uint8,
                               device=device))


def _mx_shape(keys: "MXKeys", pool: KVPool) -> None:
    if tuple(keys.codes.shape) != (pool.desc.num_pages, pool.desc.num_heads,
                                   pool.desc.page_size, pool.desc.head_dim):
        raise ValueError("MX keys: codes must be [num_pages, H, page_size, head_dim] of the pool")


def _mx_device(keys: "MXKeys", dev: torch.device) -> None:
    _on_device(keys.codes, dev, "keys.codes")
    _on_device(keys.scales, dev, "keys.scales")


def wf_kv_publish_mx(pool: KVPool, keys: MXKeys, k: torch.Tensor, v: torch.Tensor,
                     dst_start: int, pos: Optional[torch.Tensor] = None,
                     rope: Optional[Tuple[Tuple[int, int, int], float]] = None,
                     q: Optional[torch.Tensor] = None, stream=None) -> None:
    """wf_kv_publish with K quantized to MXFP8 into `keys` (C: wf_kv_publish_mx)."""
    n = k.shape[0] if k.dim() > 0 else 0
    ks = _head_rows(pool, k, "k", n)
    vs = _head_rows(pool, v, "v", n)
    qs = _head_rows(pool, q, "q", n) if q is not None else 0
    _positions(pos, n, rope)
    _mx_shape(keys, pool)
    dev = _pool_device(pool)
    _mx_device(keys, dev)
    for t, name in ((k, "k"), (v, "v"), (q, "q"), (pos, "pos")):
        if t is not None:
            _on_device(t, dev, name)
    r = None
    if rope is not None:
        (dt, dh, dw), theta = rope
        r = wf_rope(dt, dh, dw, float(theta))
    rc = lib().wf_kv_publish_mx(ctypes.byref(pool.desc), ctypes.byref(keys.desc),
                                ctypes.byref(r) if r else None, _ptr(k), ks, _ptr(v), vs,
                                _ptr(pos), n, dst_start, _ptr(q), qs, _stream(stream))
    _check(rc)


def wf_chunk_attn_mx(pool: KVPool, keys: MXKeys, segments: Sequence[Tuple[int, int, int]],
                     q: torch.Tensor, q_slot_start: Sequence[int], first_slot: int = 0,
                     scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunk-wise causal attention with the 8-bit QK^T (C: wf_chunk_attn_mx)."""
    rows = int(q_slot_start[-1]) if len(q_slot_start) else 0
    qs = _head_rows(pool, q, "q", rows)
    if out is None:
        out = torch.empty_like(q)
    os_ = _head_rows(pool, out, "out", rows)
    if lse is not None:
        _lse(lse, pool.desc.num_heads, rows, exact=True)
    _mx_shape(keys, pool)
    dev = _pool_device(pool)
    _mx_device(keys, dev)
    for t, name in ((q, "q"), (out, "out"), (lse, "lse")):
        if t is not None:
            _on_device(t, dev, name)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    segs = (wf_segment * len(segments))(*[wf_segment(*s) for s in segments])
    qss = (ctypes.c_int32 * len(q_slot_start))(*q_slot_start)
    rc = lib().wf_chunk_attn_mx(ctypes.byref(pool.desc), ctypes.byref(keys.desc), segs,
                                len(segments), _ptr(q), qs, qss, len(q_slot_start) - 1,
                                first_slot, float(scale), _ptr(out), os_, _ptr(lse),
                                _stream(stream))
    _check(rc)
    return out


def wf_qkv_publish(pool: KVPool, x: torch.Tensor, w_qkv: torch.Tensor, dst_start: int,
                   pos: Optional[torch.Tensor] = None,
                   rope: Optional[Tuple[Tuple[int, int, int], float]] = None,
                   bias: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """QKV projection of x [n, hidden] with w_qkv [3*H*D, hidden] (+ bias),
    published like wf_kv_publish; the rotated Q goes to q_out [n, H, D]
    if given (C: wf_qkv_publish)."""
    if x.dim() != 2 or x.stride(1) != 1 or w_qkv.dim() != 2 or not w_qkv.is_contiguous():
        raise ValueError("x: [n, hidden] with contiguous rows; w_qkv: contiguous [3*H*D, hidden]")
    n, hidden = x.shape
    F = 3 * pool.desc.num_heads * pool.desc.head_dim
    if tuple(w_qkv.shape) != (F, hidden):
        raise ValueError(f"w_qkv: expected [{F}, {hidden}], got {list(w_qkv.shape)}")
    for t, name in ((x, "x"), (w_qkv, "w_qkv"), (bias, "bias")):
        if t is not None and t.dtype != pool.k_pages.dtype:
            raise ValueError(f"{name}: dtype {t.dtype} differs from the pool's {pool.k_pages.dtype}")
    if bias is not None and (not bias.is_contiguous() or tuple(bias.shape) != (F,)):
        raise ValueError(f"bias must be a contiguous [{F}] tensor")
    _positions(pos, n, rope)
    qs = _head_rows(pool, q_out, "q_out", n) if q_out is not None else 0
    dev = _pool_device(pool)
    for t, name in ((x, "x"), (w_qkv, "w_qkv"), (bias, "bias"), (pos, "pos"), (q_out, "q_out")):
        if t is not None:
            _on_device(t, dev, name)
    r = None
    if rope is not None:
        (dt, dh, dw), theta = rope
        r = wf_rope(dt, dh, dw, float(theta))
    rc = lib().wf_qkv_publish(ctypes.byref(pool.desc), ctypes.byref(r) if r else None, _ptr(x),
                              x.stride(0), hidden, _ptr(w_qkv), _ptr(bias), _ptr(pos),
                              n, dst_start, _ptr(q_out), qs, _stream(stream))
    _check(rc)


def wf_history_rotate(pool: KVPool, window_start: int, chunk_stride: int, n_chunks: int,
                      stream=None) -> None:
    """End-of-round history rotation (C: wf_history_rotate): the pool's page
    table entries of the window [window_start, window_start + n_chunks *
    chunk_stride) rotate left by one chunk, in place; no page moves."""
    t = pool.page_table
    _pool_device(pool)
    rc = lib().wf_history_rotate(_ptr(t), t.numel(), pool.page_size, window_start,
                                 chunk_stride, n_chunks, _stream(stream))
    _check(rc)


def wf_device_status(clear: bool = True) -> int:
    """OR of WF_STATUS_* bits raised on the current device (synchronizes)."""
    v = ctypes.c_int32(0)
    _check(lib().wf_device_status(ctypes.byref(v), 1 if clear else 0))
    return v.value


def version() -> str:
    return lib().wf_version().decode()
