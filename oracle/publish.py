"""Paged K/V publish (oracle; test infrastructure).

[WF] §4.2: K/V are published after the QKV projection and RoPE, written
directly into ordered paged attention slots.  Pool layout (the library's
documented layout, see include/wf.h):

    k_pool [num_pages][H][page_size][D]     a token's head vector contiguous
    v_pool [num_pages][H][D][page_size]     d-major inside a page

Logical token L lives in logical page L // page_size at row L % page_size;
the page table maps logical to physical pages.  Storage arrays are uint16 bit
patterns for bfloat16 and float32 for fp32.
"""
from __future__ import annotations

import numpy as np

from .numerics import to_f32
from .rope import apply_rope


def publish(k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
            page_size: int, k: np.ndarray, v: np.ndarray, pos, dst_start: int,
            dtype: str, rope=None, q: np.ndarray = None):
    """Write tokens t = 0..n-1 to logical rows dst_start + t, in place.

    k, v: storage arrays [n, H, D].  rope: None or (split, theta).  If q is
    given (storage array [n, H, D]) its rotated copy is returned as well.
    Returns the storage-type K actually written (after RoPE) and rotated Q.
    """
    n = k.shape[0]
    if rope is not None:
        split, theta = rope
        k_out = apply_rope(to_f32(k, dtype), pos, split, theta, dtype)
        q_out = None if q is None else apply_rope(to_f32(q, dtype), pos, split, theta, dtype)
    else:
        k_out = np.array(k, copy=True)
        q_out = None if q is None else np.array(q, copy=True)
    for t in range(n):
        L = dst_start + t
        page = int(page_table[L // page_size])
        r = L % page_size
        k_pool[page, :, r, :] = k_out[t]
        v_pool[page, :, :, r] = v[t]
    return k_out, q_out


def gather(k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
           page_size: int, tokens: np.ndarray):
    """Read logical tokens back from the pool: K [n, H, D], V [n, H, D]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    pages = np.asarray(page_table, dtype=np.int64)[tokens // page_size]
    rows = tokens % page_size
    # numpy places the broadcast advanced index (the token) first: [n, H, D]
    k = k_pool[pages, :, rows, :]
    v = v_pool[pages, :, :, rows]
    return k, v
