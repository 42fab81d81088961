"""Test glue: run a seeded workload through the CPU oracle.

Builds the pool the way a layer does it: the prefix that is already resident
(anchor and clean history) is published once at set-up, then one round's
publish writes the live store and the W slot chunks, then attention runs.
Everything here calls oracle/ only.
"""
from __future__ import annotations

import numpy as np
import torch

from chunk_wise_causal_amd.workloads import Workload
from oracle import publish as opub
from oracle.numerics import to_f32

# a quiet-NaN fill: any read of unwritten pool memory poisons the output
NAN_BF16 = np.uint16(0x7FC1)
NAN_F32 = np.float32(np.nan)


def storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """torch CPU tensor -> oracle storage array (bf16 bits / float32)."""
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()
    return t.contiguous().numpy().astype(np.float32)


def empty_pool(wl: Workload, fill: str = "nan"):
    c = wl.cfg
    shape_k = (c.n_pages, c.heads, c.page_size, c.head_dim)
    shape_v = (c.n_pages, c.heads, c.head_dim, c.page_size)
    if c.dtype == "bf16":
        val = NAN_BF16 if fill == "nan" else np.uint16(0)
        kp = np.full(shape_k, val, dtype=np.uint16)
        vp = np.full(shape_v, val, dtype=np.uint16)
    else:
        val = NAN_F32 if fill == "nan" else np.float32(0)
        kp = np.full(shape_k, val, dtype=np.float32)
        vp = np.full(shape_v, val, dtype=np.float32)
    if len(wl.stale_pages):
        kp[wl.stale_pages] = storage(wl.stale_k, c.dtype)
        vp[wl.stale_pages] = storage(wl.stale_v, c.dtype)
    return kp, vp


def oracle_layer(wl: Workload, fill: str = "nan", rope: bool = True):
    """Publish set-up + one round through the oracle.  Returns a dict with
    the pools, the RoPE'd logical K (storage), V and Q storage arrays."""
    c = wl.cfg
    kp, vp = empty_pool(wl, fill)
    k = storage(wl.k, c.dtype)
    v = storage(wl.v, c.dtype)
    rp = (c.rope, c.theta) if rope else None
    ss = c.store_start
    k_rot = np.empty_like(k)
    if ss:
        k_rot[:ss], _ = opub.publish(kp, vp, wl.page_table, c.page_size, k[:ss], v[:ss],
                                     wl.pos[:ss], 0, c.dtype, rope=rp)
    k_rot[ss:], _ = opub.publish(kp, vp, wl.page_table, c.page_size, k[ss:], v[ss:],
                                 wl.pos[ss:], ss, c.dtype, rope=rp)
    return dict(k_pool=kp, v_pool=vp, k_rot=k_rot, v=v, q=storage(wl.q, c.dtype))


def f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return to_f32(a, dtype).astype(np.float64)


def oracle_stream(cfg, table: np.ndarray, n_rounds: int, seed: int = 0, rope: bool = True):
    """Streaming rounds on the page-aligned layout through the oracle.

    Set-up publishes the anchor and the history chunks.  Each round then
    publishes the store chunk and the W slot chunks (each at its own
    page-aligned start), runs the chunk-wise causal attention of the slot
    queries, and rotates the history (the store becomes the newest history
    chunk).  Yields one dict per round: out, lse (float64), the pools
    (updated in place across rounds), the table the round read and the table
    after its rotation."""
    from chunk_wise_causal_amd.workloads import AlignedLayout, initial_context, round_inputs
    from oracle.attention import chunk_attention
    from oracle.history import rotate_history

    lay = AlignedLayout(cfg)
    ps = cfg.page_size
    n_pages = int(np.max(table)) + 1
    shape_k = (n_pages, cfg.heads, ps, cfg.head_dim)
    shape_v = (n_pages, cfg.heads, cfg.head_dim, ps)
    if cfg.dtype == "bf16":
        kp, vp = np.full(shape_k, NAN_BF16, np.uint16), np.full(shape_v, NAN_BF16, np.uint16)
    else:
        kp, vp = np.full(shape_k, NAN_F32, np.float32), np.full(shape_v, NAN_F32, np.float32)
    rp = (cfg.rope, cfg.theta) if rope else None
    (ka, va, pa), (kh, vh, ph) = initial_context(cfg, seed)
    table = np.asarray(table, dtype=np.int32).copy()
    if cfg.anchor_tokens:
        opub.publish(kp, vp, table, ps, storage(ka, cfg.dtype), storage(va, cfg.dtype), pa, 0,
                     cfg.dtype, rope=rp)
    for k in range(cfg.n_hist):
        opub.publish(kp, vp, table, ps, storage(kh[k], cfg.dtype), storage(vh[k], cfg.dtype),
                     ph[k], lay.hist_start(k), cfg.dtype, rope=rp)
    for r in range(n_rounds):
        k, v, q, pos = round_inputs(cfg, r, seed)
        starts = [lay.store_start] + [lay.slot_start(j) for j in range(cfg.slots)]
        for c, st in enumerate(starts):
            opub.publish(kp, vp, table, ps, storage(k[c], cfg.dtype), storage(v[c], cfg.dtype),
                         pos[c], st, cfg.dtype, rope=rp)
        qs = storage(q, cfg.dtype)
        out, lse = chunk_attention(kp, vp, table, ps, lay.segments(), qs, cfg.q_slot_start(), 0,
                                   cfg.scale, cfg.dtype)
        after = rotate_history(table, ps, lay.window_start, lay.chunk_stride, lay.window_chunks)
        yield dict(out=out, lse=lse, k_pool=kp, v_pool=vp, table=table, table_after=after, q=qs)
        table = after
