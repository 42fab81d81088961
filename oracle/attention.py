"""Chunk-wise causal attention over the paged pool (oracle; test
infrastructure).

[WF] §3.1: inside a chunk attention is full; a query of denoising slot s sees
the K/V of slot j iff j >= s, and every query sees the anchor, the clean
history and the live store.  That is an exact mask on ordinary softmax
attention, so this oracle is the plain definition, in float64:

    vis(s)  = union of segments with slot < 0 or slot >= s
    z_L     = scale * <q, k_L>                      L in vis(s)
    out     = sum_L exp(z_L - m) v_L / sum_L exp(z_L - m),   m = max_L z_L
    lse     = m + log(sum_L exp(z_L - m))

K and V are read through the page table ([WF] §4.2, paged attention slots)
with the pool layout of oracle.publish.  The GPU kernel reaches the same
numbers differently (tile skipping, online softmax, bf16 products); none of
that appears here.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

from .numerics import to_f32
from .publish import gather


def visible_tokens(segments, s: int) -> np.ndarray:
    """Sorted logical tokens a query of slot s sees."""
    parts = [np.arange(st, st + ln, dtype=np.int64)
             for (st, ln, slot) in segments if slot < 0 or slot >= s]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.sort(np.concatenate(parts))


def _softmax_attend(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float):
    """qh [n, D], kh/vh [m, D] float64 -> out [n, D], lse [n]."""
    z = scale * (qh @ kh.T)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ vh) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def chunk_attention(k_pool, v_pool, page_table, page_size: int, segments,
                    q: np.ndarray, q_slot_start, first_slot: int, scale: float,
                    dtype: str, heads: Optional[Iterable[int]] = None,
                    rows: Optional[Dict[int, np.ndarray]] = None,
                    block: int = 1024):
    """Attention for every query row (or only `rows[g]`, absolute row ids of
    group g, and only `heads`).

    q: storage array [n_rows, H, D].  Returns (out, lse) as float64 arrays of
    shape [n_rows, H, D] and [H, n_rows]; rows/heads not computed are NaN.
    """
    n_rows, H, D = q.shape
    heads = range(H) if heads is None else list(heads)
    out = np.full((n_rows, H, D), np.nan)
    lse = np.full((H, n_rows), np.nan)
    for g in range(len(q_slot_start) - 1):
        s = first_slot + g
        r0, r1 = q_slot_start[g], q_slot_start[g + 1]
        sel = np.arange(r0, r1) if rows is None else np.asarray(rows.get(g, []), dtype=np.int64)
        if len(sel) == 0:
            continue
        vis = visible_tokens(segments, s)
        for h in heads:
            kh, vh = gather(k_pool[:, h:h + 1], v_pool[:, h:h + 1], page_table,
                            page_size, vis)
            kh = to_f32(kh[:, 0], dtype).astype(np.float64)
            vh = to_f32(vh[:, 0], dtype).astype(np.float64)
            for b in range(0, len(sel), block):
                idx = sel[b:b + block]
                qh = to_f32(q[idx, h], dtype).astype(np.float64)
                o, l = _softmax_attend(qh, kh, vh, scale)
                out[idx, h] = o
                lse[h, idx] = l
    return out, lse


def run_tokens(runs) -> np.ndarray:
    """Sorted logical tokens of a union of (kv_start, kv_len) runs."""
    parts = [np.arange(st, st + ln, dtype=np.int64) for (st, ln) in runs]
    if not parts:
        return np.zeros(0, dtype=np.int64)
    return np.sort(np.concatenate(parts))


def group_attention(k_pool, v_pool, page_table, page_size: int, runs, groups,
                    q: np.ndarray, scale: float, dtype: str,
                    heads: Optional[Iterable[int]] = None, block: int = 1024):
    """Attention of arbitrary query groups: group (r0, r1, b, e) is rows
    [r0, r1) attending, fully, to the union of runs[b:e].  The store stage
    ([WF] overview and §B.1; §3.1 context order) is the group of the store
    chunk's rows over anchor | history | store.  Same definition as
    chunk_attention with the visible set given per group.  Returns (out,
    lse) as float64 [n_rows, H, D] and [H, n_rows]; rows outside every group
    are NaN."""
    n_rows, H, D = q.shape
    heads = range(H) if heads is None else list(heads)
    out = np.full((n_rows, H, D), np.nan)
    lse = np.full((H, n_rows), np.nan)
    for (r0, r1, b, e) in groups:
        if r1 <= r0:
            continue
        vis = run_tokens(runs[b:e])
        for h in heads:
            kh, vh = gather(k_pool[:, h:h + 1], v_pool[:, h:h + 1], page_table,
                            page_size, vis)
            kh = to_f32(kh[:, 0], dtype).astype(np.float64)
            vh = to_f32(vh[:, 0], dtype).astype(np.float64)
            for i in range(r0, r1, block):
                idx = np.arange(i, min(r1, i + block))
                qh = to_f32(q[idx, h], dtype).astype(np.float64)
                o, l = _softmax_attend(qh, kh, vh, scale)
                out[idx, h] = o
                lse[h, idx] = l
    return out, lse


def probabilities(k_pool, v_pool, page_table, page_size: int, segments,
                  q_rows: np.ndarray, s: int, h: int, scale: float, dtype: str):
    """Softmax weights [n, |vis(s)|] of the given query rows (storage
    array [n, D]) for one head: the rows of the attention matrix."""
    vis = visible_tokens(segments, s)
    kh, _ = gather(k_pool[:, h:h + 1], v_pool[:, h:h + 1], page_table, page_size, vis)
    kh = to_f32(kh[:, 0], dtype).astype(np.float64)
    z = scale * (to_f32(q_rows, dtype).astype(np.float64) @ kh.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)
