"""Brute-force chunk-wise causal attention (oracle; test infrastructure).

The same definition as oracle.attention, written the slow way for tiny
inputs: explicit loops over heads, query rows and keys, with the visibility
of every key decided on its own by comparing its segment's slot with the
query's slot ([WF] §3.1: slot s sees slot j iff j >= s; slot < 0 context is
seen by all).  It reads the logical (unpaged) K and V, so it also checks the
paging done by oracle.publish / oracle.attention.gather.
"""
from __future__ import annotations

import math

import numpy as np


def brute_attention(q: np.ndarray, k_logical: np.ndarray, v_logical: np.ndarray,
                    segments, q_slot_start, first_slot: int, scale: float):
    """q [n_rows, H, D], k_logical/v_logical [n_kv, H, D], all float64.
    Returns out [n_rows, H, D] and lse [H, n_rows] (natural log)."""
    n_rows, H, D = q.shape
    out = np.full((n_rows, H, D), np.nan)
    lse = np.full((H, n_rows), np.nan)
    for h in range(H):
        for g in range(len(q_slot_start) - 1):
            s = first_slot + g
            for i in range(q_slot_start[g], q_slot_start[g + 1]):
                scores = []
                values = []
                for (start, length, slot) in segments:
                    visible = slot < 0 or slot >= s
                    if not visible:
                        continue
                    for L in range(start, start + length):
                        scores.append(scale * float(np.dot(q[i, h], k_logical[L, h])))
                        values.append(v_logical[L, h])
                m = max(scores)
                w = [math.exp(z - m) for z in scores]
                l = math.fsum(w)
                acc = np.zeros(D)
                for wk, vk in zip(w, values):
                    acc += wk * vk
                out[i, h] = acc / l
                lse[h, i] = m + math.log(l)
    return out, lse


def brute_group_attention(q: np.ndarray, k_logical: np.ndarray, v_logical: np.ndarray,
                          runs, groups, scale: float):
    """Query groups with explicit key runs, the slow way: for each row of
    group (r0, r1, b, e), every logical token L is tested on its own for
    membership in one of runs[b:e].  float64 in, out [n_rows, H, D] and
    lse [H, n_rows] out (NaN outside every group)."""
    n_rows, H, D = q.shape
    n_kv = k_logical.shape[0]
    out = np.full((n_rows, H, D), np.nan)
    lse = np.full((H, n_rows), np.nan)
    for (r0, r1, b, e) in groups:
        for h in range(H):
            for i in range(r0, r1):
                scores, values = [], []
                for L in range(n_kv):
                    if not any(st <= L < st + ln for (st, ln) in runs[b:e]):
                        continue
                    scores.append(scale * float(np.dot(q[i, h], k_logical[L, h])))
                    values.append(v_logical[L, h])
                m = max(scores)
                w = [math.exp(z - m) for z in scores]
                l = math.fsum(w)
                acc = np.zeros(D)
                for wi, vi in zip(w, values):
                    acc += wi * vi
                out[i, h] = acc / l
                lse[h, i] = m + math.log(l)
    return out, lse
