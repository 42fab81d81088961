"""Pins for the history rotation oracle (oracle/history.py).

[WF] §3.1: the context is anchor | bounded clean history (oldest first) |
live store | denoising slots; a completed round moves the store into the
history as its newest chunk and drops the oldest one.  The pins:
  - a hand-worked table (values written out by hand from that rule);
  - the token-level reading: after the rotation, the logical tokens of the
    window read what the tokens one chunk further read before (np.roll of
    the token window), checked through the pool gather;
  - invariants: a permutation of the window, nothing outside it changes,
    n_chunks rotations are the identity;
  - a streaming composition: rounds of publish + attention + rotation on the
    paged pool against a token-level model of the context (logical K/V
    arrays rolled by one chunk per round) attended by brute force.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd.workloads import (AlignedLayout, initial_context, round_inputs,
                                             small_config)
from oracle.brute import brute_attention
from oracle.history import rotate_history
from oracle.publish import gather
from oracle.rope import apply_rope
from tests._pipeline import oracle_stream


def test_hand_worked_example():
    # pages 2..7 hold three 2-page chunks: history [9,1], [4,8], store [2,6]
    table = np.array([7, 3, 9, 1, 4, 8, 2, 6], dtype=np.int32)
    got = rotate_history(table, 16, 32, 32, 3)
    # history now [4,8] (was second), [2,6] (old store); store <- [9,1] (evicted)
    assert got.tolist() == [7, 3, 4, 8, 2, 6, 9, 1]
    assert table.tolist() == [7, 3, 9, 1, 4, 8, 2, 6]      # input untouched
    # one chunk of one page: nothing moves
    assert rotate_history(table, 16, 0, 16, 1).tolist() == table.tolist()


def _address_pool(n_pages, ps):
    """K pool whose element (page p, row r) holds p * ps + r: a gather then
    shows which physical row every logical token maps to."""
    k = np.zeros((n_pages, 1, ps, 1), dtype=np.int64)
    k[:, 0, :, 0] = np.arange(n_pages)[:, None] * ps + np.arange(ps)[None, :]
    v = np.zeros((n_pages, 1, 1, ps), dtype=np.int64)
    return k, v


@pytest.mark.parametrize("ps,start,stride,n,n_log", [
    (16, 0, 16, 2, 2), (16, 32, 48, 3, 12), (64, 128, 192, 5, 20), (256, 256, 4864, 3, 140),
])
def test_token_level_reading_and_invariants(ps, start, stride, n, n_log):
    rng = np.random.default_rng(ps + stride + n)
    n_pages = n_log + 5
    table = rng.permutation(n_pages)[:n_log].astype(np.int32)
    kp, vp = _address_pool(n_pages, ps)
    toks = np.arange(n_log * ps)
    before = gather(kp, vp, table, ps, toks)[0][:, 0, 0]
    new = rotate_history(table, ps, start, stride, n)
    after = gather(kp, vp, new, ps, toks)[0][:, 0, 0]
    w0, w1 = start, start + n * stride
    # the window reads what the tokens one chunk further read (cyclically)
    assert np.array_equal(after[w0:w1], np.roll(before[w0:w1], -stride))
    # outside the window nothing changes
    assert np.array_equal(after[:w0], before[:w0]) and np.array_equal(after[w1:], before[w1:])
    # a permutation of the window's entries
    f, e = start // ps, w1 // ps
    assert sorted(new[f:e].tolist()) == sorted(table[f:e].tolist())
    # n rotations give the table back
    t = table
    for _ in range(n):
        t = rotate_history(t, ps, start, stride, n)
    assert np.array_equal(t, table)


def test_store_becomes_newest_history():
    """Tag every chunk's logical tokens with its age; after a rotation the
    history reads, oldest first, the old history without its oldest chunk
    and then the old store."""
    cfg = small_config(frame_rows=3, frame_cols=7, frames_per_chunk=2, anchor_tokens=10,
                       n_hist=3, slots=2, page_size=16)
    lay = AlignedLayout(cfg)
    ps = cfg.page_size
    rng = np.random.default_rng(5)
    table = rng.permutation(lay.n_logical_pages).astype(np.int32)
    kp, vp = _address_pool(lay.n_logical_pages, ps)

    def chunk_rows(t, start):
        return gather(kp, vp, t, ps, np.arange(start, start + cfg.chunk))[0][:, 0, 0]

    old = [chunk_rows(table, lay.hist_start(k)) for k in range(cfg.n_hist)]
    old_store = chunk_rows(table, lay.store_start)
    new = rotate_history(table, ps, lay.window_start, lay.chunk_stride, lay.window_chunks)
    now = [chunk_rows(new, lay.hist_start(k)) for k in range(cfg.n_hist)]
    for k in range(cfg.n_hist - 1):
        assert np.array_equal(now[k], old[k + 1])
    assert np.array_equal(now[-1], old_store)
    # the evicted chunk's rows are where the next store is written
    assert np.array_equal(chunk_rows(new, lay.store_start), old[0])
    # anchor and slots unchanged
    assert np.array_equal(chunk_rows(new, lay.slot_start(0)), chunk_rows(table, lay.slot_start(0)))
    a = np.arange(cfg.anchor_tokens)
    assert np.array_equal(gather(kp, vp, new, ps, a)[0], gather(kp, vp, table, ps, a)[0])


def test_streaming_rounds_against_token_model():
    """Three rounds through the paged oracle (publish, attention, rotation)
    against a token-level model of the context: logical K/V arrays that get
    each round's new chunks written in place and whose history + store window
    rolls by one chunk per round, attended by brute force."""
    cfg = small_config(dtype="fp32", head_dim=64, rope=(24, 20, 20), frame_rows=3,
                       frame_cols=7, frames_per_chunk=2, anchor_tokens=10, n_hist=2, slots=2,
                       page_size=16)
    lay = AlignedLayout(cfg)
    assert cfg.chunk % cfg.page_size != 0          # chunks end inside a page: gaps exist
    rng = np.random.default_rng(9)
    table = rng.permutation(lay.n_logical_pages).astype(np.int32)
    H, D = cfg.heads, cfg.head_dim
    kl = np.full((lay.span, H, D), np.nan)
    vl = np.full((lay.span, H, D), np.nan)

    def put(start, k, v, pos):
        k32 = k.numpy().astype(np.float32)
        kl[start:start + len(k)] = apply_rope(k32, pos, cfg.rope, cfg.theta, "fp32")
        vl[start:start + len(v)] = v.numpy()

    (ka, va, pa), (kh, vh, ph) = initial_context(cfg)
    put(0, ka, va, pa)
    for k in range(cfg.n_hist):
        put(lay.hist_start(k), kh[k], vh[k], ph[k])
    w0 = lay.window_start
    w1 = w0 + lay.window_chunks * lay.chunk_stride
    for r, res in enumerate(oracle_stream(cfg, table, 3)):
        k, v, q, pos = round_inputs(cfg, r)
        starts = [lay.store_start] + [lay.slot_start(j) for j in range(cfg.slots)]
        for c, st in enumerate(starts):
            put(st, k[c], v[c], pos[c])
        ref, ref_lse = brute_attention(q.numpy().astype(np.float64), kl, vl, lay.segments(),
                                       cfg.q_slot_start(), 0, cfg.scale)
        np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(res["lse"], ref_lse, rtol=0, atol=1e-12)
        kl[w0:w1] = np.roll(kl[w0:w1], -lay.chunk_stride, axis=0)
        vl[w0:w1] = np.roll(vl[w0:w1], -lay.chunk_stride, axis=0)
