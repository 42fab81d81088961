"""History rotation at the end of a round (oracle; test infrastructure).

[WF] §3.1: the per-layer context is the anchor, then a bounded clean
history (oldest chunk first), then the live store, then the denoising
slots.  When a round completes a chunk, the store becomes the newest history
chunk and the oldest history chunk leaves the bounded history.

With every chunk starting on a page boundary and spanning a whole number of
pages, this is a reordering of the page-table entries of the window that
holds history + store; no K/V value changes.  The page that held the oldest
chunk ends up at the store's place, where the next round publishes the new
store.
"""
from __future__ import annotations

import numpy as np


def rotate_history(page_table: np.ndarray, page_size: int, window_start: int,
                   chunk_stride: int, n_chunks: int) -> np.ndarray:
    """Return the page table after one rotation (the input is not changed).

    The window [window_start, window_start + n_chunks * chunk_stride) of
    logical tokens holds n_chunks chunks of chunk_stride tokens: the history,
    oldest first, then the store.  Both window_start and chunk_stride are
    whole pages.
    """
    assert window_start % page_size == 0 and chunk_stride % page_size == 0
    table = [int(x) for x in page_table]
    first = window_start // page_size
    per = chunk_stride // page_size
    chunks = [table[first + c * per: first + (c + 1) * per] for c in range(n_chunks)]
    # oldest history chunk leaves the front; its pages take the store's place
    # at the back, after the old store (now the newest history chunk)
    chunks = chunks[1:] + chunks[:1]
    window = [p for chunk in chunks for p in chunk]
    out = table[:first] + window + table[first + n_chunks * per:]
    return np.asarray(out, dtype=np.int32)
