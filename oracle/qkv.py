"""QKV projection fused with the publish (oracle; test infrastructure).

[WF] §4.2: K/V are published right after the QKV projection and RoPE.  The
fused form computes the projection of a chunk's hidden states and publishes
straight from its result, so K and V never make a round trip through HBM.
What it must produce is exactly the unfused pipeline's:

    qkv = bf16(x W^T (+ bias))          projection, rounded to the storage
                                        type like any bfloat16 GEMM output
    q, k, v = the three H*D slices of qkv (in that order), each [n, H, D]
    K', Q' = RoPE(k), RoPE(q)           as wf_kv_publish rotates them
    pool  <- K', v                       the paged scatter of wf_kv_publish

x is [n, hidden], W is [3*H*D, hidden] (one row per output feature), bias
[3*H*D]; all bfloat16 storage arrays (uint16 bit patterns).  The projection
is evaluated in float64 (a plain matrix product) before the rounding.
"""
from __future__ import annotations

import numpy as np

from .numerics import f32_to_bf16, to_f32
from .publish import publish


def f64_to_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits with a single rounding to nearest, ties to
    even (going through float32 would round twice)."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.abs(a)
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    # 8 significant bits; below bfloat16's normal range the step is 2^-133
    step = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    q = np.round(a / step) * step                 # numpy rounds halves to even
    return f32_to_bf16(q.astype(np.float32))      # exact: q is representable


def qkv_project(x: np.ndarray, w: np.ndarray, heads: int, head_dim: int, bias=None):
    """(q, k, v) bf16 storage arrays [n, H, D] of the projection."""
    acc = to_f32(x, "bf16").astype(np.float64) @ to_f32(w, "bf16").astype(np.float64).T
    if bias is not None:
        acc = acc + to_f32(bias, "bf16").astype(np.float64)[None, :]
    out = f64_to_bf16(acc)
    n, hd = x.shape[0], heads * head_dim
    return (out[:, :hd].reshape(n, heads, head_dim), out[:, hd:2 * hd].reshape(n, heads, head_dim),
            out[:, 2 * hd:].reshape(n, heads, head_dim))


def qkv_publish(k_pool, v_pool, page_table, page_size: int, x, w, heads: int, head_dim: int,
                pos, dst_start: int, rope, bias=None):
    """Projection, then wf_kv_publish's RoPE and scatter (in place on the
    pools).  Returns the rotated Q (bf16 storage [n, H, D]; unrotated when
    rope is None)."""
    q, k, v = qkv_project(x, w, heads, head_dim, bias)
    _, q_rot = publish(k_pool, v_pool, page_table, page_size, k, v, pos, dst_start, "bf16",
                       rope=rope, q=q)
    return q_rot
