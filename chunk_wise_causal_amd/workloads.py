"""Seeded synthetic workloads for the chunk-wise causal attention path.

This module only lays out and draws inputs: shapes, the logical context
layout, positions, page placement and random numbers.  It contains none of
the method's arithmetic (no RoPE, no attention, no paging math), so both the
CPU oracle and the GPU path can be fed from it without sharing any code that
they are meant to check against each other.

Context layout ("Wave Forcing: Towards Speed-of-Light Streaming Video
Generation", §3.1, per-layer context order): logical tokens are

    anchor | history chunk 0 (oldest) ... | live store | slot 0 | ... | slot W-1

with no gaps.  The anchor, history and store are visible to every query
(segment slot -1); denoising slot j is segment slot j.  Queries are the W
slot chunks, in slot order.

Positions (t, h, w) = (latent frame, latent row, latent column).  Frame 0 is
the anchor (its first A tokens in row-major order); history chunks follow
oldest first, then the store, then slot W-1 down to slot 0: slot 0 is the
newest and noisiest chunk of the wavefront (same page, §3.1 and overview:
newer, noisier chunks read older, cleaner ones).

Random inputs mirror the pages' system tests, which run dummy weights and
measure cost, not quality (same page, §C.3): Q, K, V ~ N(0, 1).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "Workload", "make_workload", "small_config", "query_groups",
           "AlignedLayout", "initial_context", "round_inputs"]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic layer shape.  Token counts derive from the latent grid."""
    name: str
    dtype: str                 # "bf16" | "fp32"
    heads: int
    head_dim: int
    frame_rows: int
    frame_cols: int
    frames_per_chunk: int
    anchor_tokens: int         # first tokens of frame 0, row-major
    n_hist: int
    slots: int                 # W denoising slots
    page_size: int
    rope: Tuple[int, int, int]
    theta: float = 10000.0
    permute_pages: bool = True
    stale_frac: float = 0.0    # extra physical pages holding stale N(0, 4) data
    hot_frac: float = 0.0      # fraction of K token rows scaled by hot_factor
    hot_factor: float = 8.0
    seed: int = 0

    # ---- derived sizes ---------------------------------------------------
    @property
    def chunk(self) -> int:
        return self.frames_per_chunk * self.frame_rows * self.frame_cols

    @property
    def prefix(self) -> int:
        """anchor + history + store tokens (visible to every slot)."""
        return self.anchor_tokens + self.n_hist * self.chunk + self.chunk

    @property
    def n_kv(self) -> int:
        return self.prefix + self.slots * self.chunk

    @property
    def n_q(self) -> int:
        return self.slots * self.chunk

    @property
    def n_logical_pages(self) -> int:
        return -(-self.n_kv // self.page_size)

    @property
    def n_stale_pages(self) -> int:
        return int(math.ceil(self.stale_frac * self.n_logical_pages - 1e-9))

    @property
    def n_pages(self) -> int:
        return self.n_logical_pages + self.n_stale_pages

    @property
    def store_start(self) -> int:
        return self.anchor_tokens + self.n_hist * self.chunk

    @property
    def tick_tokens(self) -> int:
        """Tokens published per round: the live store plus the W slots."""
        return self.n_kv - self.store_start

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def visible(self, s: int) -> int:
        """Number of keys a query of slot s sees (prefix + slots s..W-1)."""
        return self.prefix + (self.slots - s) * self.chunk

    def unmasked_flops(self) -> int:
        """2 matmuls x 2 flops x head_dim per visible (query, key) pair."""
        pairs = sum(self.chunk * self.visible(s) for s in range(self.slots))
        return 4 * self.heads * self.head_dim * pairs

    def publish_bytes(self, n_tok: Optional[int] = None) -> int:
        """Bytes a publish of n_tok tokens must move: read K, V; write K, V."""
        n = self.tick_tokens if n_tok is None else n_tok
        return 4 * n * self.heads * self.head_dim * self.elem_bytes

    def segments(self) -> List[Tuple[int, int, int]]:
        """(kv_start, kv_len, slot) in logical order."""
        segs = [(0, self.anchor_tokens, -1)]
        for k in range(self.n_hist):
            segs.append((self.anchor_tokens + k * self.chunk, self.chunk, -1))
        segs.append((self.store_start, self.chunk, -1))
        for j in range(self.slots):
            segs.append((self.prefix + j * self.chunk, self.chunk, j))
        return [s for s in segs if s[1] > 0]

    def q_slot_start(self) -> List[int]:
        return [j * self.chunk for j in range(self.slots + 1)]

    def positions(self) -> np.ndarray:
        """int32 [n_kv, 3] (t, h, w) for every logical token."""
        hw = self.frame_rows * self.frame_cols
        rows = np.arange(hw, dtype=np.int32) // self.frame_cols
        cols = np.arange(hw, dtype=np.int32) % self.frame_cols
        out = np.empty((self.n_kv, 3), dtype=np.int32)
        # anchor: frame 0, first anchor_tokens tokens
        a = self.anchor_tokens
        out[:a, 0] = 0
        out[:a, 1] = rows[np.arange(a) % hw]
        out[:a, 2] = cols[np.arange(a) % hw]
        fpc = self.frames_per_chunk
        # chunk order by age: history (oldest first), store, slot W-1 .. slot 0
        frame_of_chunk = {}
        f = 1
        for k in range(self.n_hist):
            frame_of_chunk[("hist", k)] = f
            f += fpc
        frame_of_chunk[("store", 0)] = f
        f += fpc
        for j in reversed(range(self.slots)):
            frame_of_chunk[("slot", j)] = f
            f += fpc
        starts = [(("hist", k), self.anchor_tokens + k * self.chunk) for k in range(self.n_hist)]
        starts.append((("store", 0), self.store_start))
        starts += [(("slot", j), self.prefix + j * self.chunk) for j in range(self.slots)]
        tok = np.arange(self.chunk, dtype=np.int32)
        for key, st in starts:
            out[st:st + self.chunk, 0] = frame_of_chunk[key] + tok // hw
            out[st:st + self.chunk, 1] = rows[tok % hw]
            out[st:st + self.chunk, 2] = cols[tok % hw]
        return out


def _cfg(**kw) -> Config:
    return Config(**kw)


# The five layer shapes the path is measured on.
CONFIGS = {
    1: _cfg(name="tiny fp32 (H2 D64, chunk 32, W=2)", dtype="fp32", heads=2,
            head_dim=64, frame_rows=4, frame_cols=8, frames_per_chunk=1,
            anchor_tokens=16, n_hist=1, slots=2, page_size=16,
            rope=(24, 20, 20), permute_pages=False, seed=1),
    2: _cfg(name="1.3B-like 4-step (H12 D128, chunk 4680, W=4)", dtype="bf16",
            heads=12, head_dim=128, frame_rows=30, frame_cols=52,
            frames_per_chunk=3, anchor_tokens=1560, n_hist=2, slots=4,
            page_size=256, rope=(44, 42, 42), seed=2),
    3: _cfg(name="1.3B-like 5-step (H12 D128, chunk 4680, W=5, stale pages)",
            dtype="bf16", heads=12, head_dim=128, frame_rows=30, frame_cols=52,
            frames_per_chunk=3, anchor_tokens=1560, n_hist=2, slots=5,
            page_size=128, rope=(44, 42, 42), stale_frac=0.10, seed=3),
    4: _cfg(name="14B-like 4-step (H40 D128, chunk 4680, W=4)", dtype="bf16",
            heads=40, head_dim=128, frame_rows=30, frame_cols=52,
            frames_per_chunk=3, anchor_tokens=1560, n_hist=2, slots=4,
            page_size=256, rope=(44, 42, 42), hot_frac=0.01, seed=4),
    5: _cfg(name="14B-like long context (H40 D128, chunk 10800, W=5)",
            dtype="bf16", heads=40, head_dim=128, frame_rows=45, frame_cols=80,
            frames_per_chunk=3, anchor_tokens=3600, n_hist=4, slots=5,
            page_size=256, rope=(44, 42, 42), seed=5),
}


def small_config(**overrides) -> Config:
    """A bf16 shape that the oracle finishes in seconds yet spans several
    attention tiles and ragged tails (defaults: H2 D128, chunk 64, W=3)."""
    base = dict(name="small bf16", dtype="bf16", heads=2, head_dim=128,
                frame_rows=4, frame_cols=8, frames_per_chunk=2,
                anchor_tokens=24, n_hist=1, slots=3, page_size=16,
                rope=(44, 42, 42), seed=11)
    base.update(overrides)
    return Config(**base)


@dataclasses.dataclass
class Workload:
    cfg: Config
    q: torch.Tensor            # [n_q, H, D] storage dtype, logical order
    k: torch.Tensor            # [n_kv, H, D] (before RoPE)
    v: torch.Tensor            # [n_kv, H, D]
    pos: np.ndarray            # int32 [n_kv, 3]
    page_table: np.ndarray     # int32 [n_logical_pages]
    stale_pages: np.ndarray    # int64 physical ids not in the table
    stale_k: Optional[torch.Tensor]  # [n_stale, H, ps, D] pool-layout contents
    stale_v: Optional[torch.Tensor]  # [n_stale, H, D, ps]
    hot_rows: np.ndarray       # K token rows scaled by hot_factor

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32


def make_workload(cfg: Config, seed: Optional[int] = None) -> Workload:
    """Draw one workload on the CPU.  Draw order is fixed: Q, K, V (float32
    N(0,1)), the hot K rows, the page permutation, the stale page contents;
    then everything is rounded to the storage type."""
    g = torch.Generator().manual_seed(cfg.seed if seed is None else seed)
    H, D = cfg.heads, cfg.head_dim
    q = torch.randn(cfg.n_q, H, D, generator=g)
    k = torch.randn(cfg.n_kv, H, D, generator=g)
    v = torch.randn(cfg.n_kv, H, D, generator=g)
    n_hot = int(round(cfg.hot_frac * cfg.n_kv))
    hot = np.zeros(0, dtype=np.int64)
    if n_hot:
        hot = torch.randperm(cfg.n_kv, generator=g)[:n_hot].numpy()
        k[torch.from_numpy(hot)] *= cfg.hot_factor
    if cfg.permute_pages:
        perm = torch.randperm(cfg.n_pages, generator=g).numpy()
    else:
        perm = np.arange(cfg.n_pages)
    table = perm[:cfg.n_logical_pages].astype(np.int32)
    stale = np.sort(perm[cfg.n_logical_pages:]).astype(np.int64)
    sk = sv = None
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    if len(stale):
        ps = cfg.page_size
        sk = (torch.randn(len(stale), H, ps, D, generator=g) * 2.0).to(td)
        sv = (torch.randn(len(stale), H, D, ps, generator=g) * 2.0).to(td)
    return Workload(cfg=cfg, q=q.to(td), k=k.to(td), v=v.to(td),
                    pos=cfg.positions(), page_table=table, stale_pages=stale,
                    stale_k=sk, stale_v=sv, hot_rows=hot)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bfloat16 tensor (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def query_groups(cfg: Config, seed: int = 0):
    """A seeded layout of query groups for the generic entry point, as
    (runs, groups) with runs (kv_start, kv_len) and groups (q_row_start,
    q_row_end, run_begin, run_end), over the cfg.n_q query rows:

      rows [0, C)       the store stage: the first chunk of rows stands in for
                        the store chunk's queries, over anchor | history |
                        store = [0, cfg.prefix)
      rows [C, 2C)      three random disjoint runs of random (unaligned)
                        lengths anywhere in [0, n_kv), listed out of order
      rows [2C, n_q)    (if any) the whole context, given as one run per
                        segment, so adjacent runs must be merged
    """
    rng = np.random.Generator(np.random.PCG64(10_000 + seed))
    C, n_kv = cfg.chunk, cfg.n_kv
    runs = [(0, cfg.prefix)]
    groups = [(0, C, 0, 1)]
    cuts = np.sort(rng.choice(np.arange(1, n_kv), size=5, replace=False))
    rnd = [(int(cuts[0]), int(cuts[1] - cuts[0])), (int(cuts[2]), int(cuts[3] - cuts[2])),
           (int(cuts[4]), int(n_kv - cuts[4]))]
    rnd = [rnd[i] for i in rng.permutation(3)]
    groups.append((C, min(2 * C, cfg.n_q), len(runs), len(runs) + 3))
    runs += rnd
    if cfg.n_q > 2 * C:
        segs = [(st, ln) for (st, ln, _) in cfg.segments()]
        groups.append((2 * C, cfg.n_q, len(runs), len(runs) + len(segs)))
        runs += segs
    return runs, groups


@dataclasses.dataclass(frozen=True)
class AlignedLayout:
    """The same context on page boundaries, for rotating the history by
    page-table edits: the anchor and every chunk start on a page, a chunk of
    C tokens occupies ceil(C / page_size) pages, and the tail of its last page
    is a gap no segment names.  Logical order is unchanged:

        anchor | history 0 (oldest) .. | store | slot 0 | .. | slot W-1

    The rotation window is history + store: n_hist + 1 chunks from
    window_start, chunk_stride tokens each.
    """
    cfg: Config

    @property
    def chunk_stride(self) -> int:
        ps = self.cfg.page_size
        return -(-self.cfg.chunk // ps) * ps

    @property
    def window_start(self) -> int:
        ps = self.cfg.page_size
        return -(-self.cfg.anchor_tokens // ps) * ps

    @property
    def window_chunks(self) -> int:
        return self.cfg.n_hist + 1

    def hist_start(self, k: int) -> int:
        return self.window_start + k * self.chunk_stride

    @property
    def store_start(self) -> int:
        return self.hist_start(self.cfg.n_hist)

    def slot_start(self, j: int) -> int:
        return self.store_start + (j + 1) * self.chunk_stride

    @property
    def span(self) -> int:
        """Logical tokens covered, gaps included (a whole number of pages)."""
        return self.slot_start(self.cfg.slots)

    @property
    def n_logical_pages(self) -> int:
        return self.span // self.cfg.page_size

    def segments(self) -> List[Tuple[int, int, int]]:
        c = self.cfg
        segs = [(0, c.anchor_tokens, -1)] if c.anchor_tokens else []
        segs += [(self.hist_start(k), c.chunk, -1) for k in range(c.n_hist)]
        segs.append((self.store_start, c.chunk, -1))
        segs += [(self.slot_start(j), c.chunk, j) for j in range(c.slots)]
        return segs


def round_inputs(cfg: Config, rnd: int, seed: int = 0):
    """Fresh inputs of streaming round `rnd` (seeded per round): K and V of
    the store chunk and the W slot chunks ([W+1, C, H, D], store first, then
    slot 0..W-1), the slot queries [W*C, H, D] and (t, h, w) positions
    [W+1, C, 3].  In round r the store holds latent frames after the r
    chunks completed before it (history starts at frame 1, after the anchor's
    frame 0); slot W-1 is the next chunk and slot 0 the newest."""
    g = torch.Generator().manual_seed(1_000_003 * (seed + 1) + rnd)
    H, D, C, W = cfg.heads, cfg.head_dim, cfg.chunk, cfg.slots
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    k = torch.randn(W + 1, C, H, D, generator=g).to(td)
    v = torch.randn(W + 1, C, H, D, generator=g).to(td)
    q = torch.randn(W * C, H, D, generator=g).to(td)
    hw = cfg.frame_rows * cfg.frame_cols
    tok = np.arange(C, dtype=np.int32)
    fpc = cfg.frames_per_chunk
    store_frame = 1 + (cfg.n_hist + rnd) * fpc
    pos = np.empty((W + 1, C, 3), dtype=np.int32)
    for c in range(W + 1):
        # c = 0: store; c = 1 + j: slot j, whose frame is store + (W - j) chunks
        f0 = store_frame + (0 if c == 0 else (W - (c - 1)) * fpc)
        pos[c, :, 0] = f0 + tok // hw
        pos[c, :, 1] = (tok % hw) // cfg.frame_cols
        pos[c, :, 2] = (tok % hw) % cfg.frame_cols
    return k, v, q, pos


def initial_context(cfg: Config, seed: int = 0):
    """The context resident before round 0: anchor K, V [A, H, D] with
    positions [A, 3] (frame 0), and the history chunks K, V [n_hist, C, H, D]
    with positions [n_hist, C, 3] (frames 1.., oldest first)."""
    g = torch.Generator().manual_seed(7_000_001 * (seed + 1))
    H, D, C, A = cfg.heads, cfg.head_dim, cfg.chunk, cfg.anchor_tokens
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ka = torch.randn(A, H, D, generator=g).to(td)
    va = torch.randn(A, H, D, generator=g).to(td)
    kh = torch.randn(cfg.n_hist, C, H, D, generator=g).to(td)
    vh = torch.randn(cfg.n_hist, C, H, D, generator=g).to(td)
    hw = cfg.frame_rows * cfg.frame_cols
    ta = np.arange(A, dtype=np.int32) % hw
    pa = np.stack([np.zeros(A, np.int32), ta // cfg.frame_cols, ta % cfg.frame_cols], axis=1)
    tok = np.arange(C, dtype=np.int32)
    ph = np.empty((cfg.n_hist, C, 3), dtype=np.int32)
    for k in range(cfg.n_hist):
        ph[k, :, 0] = 1 + k * cfg.frames_per_chunk + tok // hw
        ph[k, :, 1] = (tok % hw) // cfg.frame_cols
        ph[k, :, 2] = (tok % hw) % cfg.frame_cols
    return (ka, va, pa), (kh, vh, ph)
