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
