"""GPU parity of wf_history_rotate against the CPU oracle, through the C ABI.

Streaming rounds on page-aligned layouts (chunks end inside a page, so the
gaps exist): set-up publishes the anchor and the history; each round
publishes the store and slot chunks, runs wf_chunk_attn and then rotates the
history by page-table edits.  Every round's attention is held to the usual
tolerance against tests._pipeline.oracle_stream, the table after each
rotation must equal the oracle's bit for bit, and so must both pools after
the last round.  Table-only rotations at the 14B-like and long-context
geometries and at the 16384-page limit are bit-exact, and n_chunks
rotations in a row give the table back.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import (AlignedLayout, CONFIGS, initial_context,
                                             round_inputs, small_config)
from oracle.history import rotate_history
from tests import _gpu as G
from tests._pipeline import oracle_stream

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


SHAPES = {
    # chunk 63 tokens on 16-token pages: one token of gap per chunk
    "bf16_ps16": small_config(frame_rows=3, frame_cols=7, frames_per_chunk=3, anchor_tokens=10,
                              n_hist=2, slots=3, page_size=16, seed=31),
    # chunk 200 on 64-token pages, three heads, ragged 256-row query tiles
    "bf16_ps64": small_config(heads=3, frame_rows=5, frame_cols=8, frames_per_chunk=5,
                              anchor_tokens=40, n_hist=3, slots=3, page_size=64, seed=32),
    "fp32_ps16": small_config(dtype="fp32", head_dim=64, rope=(24, 20, 20), frame_rows=3,
                              frame_cols=7, frames_per_chunk=2, anchor_tokens=10, n_hist=2,
                              slots=2, page_size=16, seed=33),
}


def _table(cfg, seed):
    lay = AlignedLayout(cfg)
    rng = np.random.default_rng(seed)
    return rng.permutation(lay.n_logical_pages + 3)[:lay.n_logical_pages].astype(np.int32)


def gpu_stream(cfg, table, n_rounds, seed=0):
    """The rounds of tests._pipeline.oracle_stream, step for step, on libwf."""
    lay = AlignedLayout(cfg)
    ps = cfg.page_size
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    pool = wf.KVPool.empty(int(table.max()) + 1, cfg.heads, ps, cfg.head_dim,
                           torch.from_numpy(table), dtype=td, device=G.DEV)
    for t in (pool.k_pages, pool.v_pages):
        if td == torch.bfloat16:
            t.view(torch.int16).fill_(0x7FC1)
        else:
            t.view(torch.int32).fill_(0x7FC00000)
    rp = (cfg.rope, cfg.theta)
    (ka, va, pa), (kh, vh, ph) = initial_context(cfg, seed)
    dev = lambda x: torch.from_numpy(x).to(G.DEV) if isinstance(x, np.ndarray) else x.to(G.DEV)
    if cfg.anchor_tokens:
        wf.wf_kv_publish(pool, dev(ka), dev(va), 0, pos=dev(pa), rope=rp)
    for k in range(cfg.n_hist):
        wf.wf_kv_publish(pool, dev(kh[k]), dev(vh[k]), lay.hist_start(k), pos=dev(ph[k]),
                         rope=rp)
    for r in range(n_rounds):
        k, v, q, pos = round_inputs(cfg, r, seed)
        starts = [lay.store_start] + [lay.slot_start(j) for j in range(cfg.slots)]
        for c, st in enumerate(starts):
            wf.wf_kv_publish(pool, dev(k[c]), dev(v[c]), st, pos=dev(np.ascontiguousarray(pos[c])),
                             rope=rp)
        qd = dev(q)
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((cfg.heads, cfg.n_q), float("nan"), device=G.DEV)
        wf.wf_chunk_attn(pool, lay.segments(), qd, cfg.q_slot_start(), 0, cfg.scale, out=out,
                         lse=lse)
        wf.wf_history_rotate(pool, lay.window_start, lay.chunk_stride, lay.window_chunks)
        torch.cuda.synchronize()
        yield out, lse, pool


@pytest.mark.parametrize("name", list(SHAPES))
def test_streaming_rounds_parity(name):
    cfg = SHAPES[name]
    table = _table(cfg, cfg.seed)
    print(f"\n[history] {name}: chunk {cfg.chunk}, stride {AlignedLayout(cfg).chunk_stride}",
          flush=True)
    n_rounds = 4
    for r, ((out, lse, pool), ref) in enumerate(zip(gpu_stream(cfg, table, n_rounds),
                                                    oracle_stream(cfg, table, n_rounds))):
        assert wf.wf_device_status() == 0
        assert np.array_equal(pool.page_table.cpu().numpy(), ref["table_after"]), r
        assert torch.isfinite(out.float()).all().item()
        mx, rr = G.err_stats(G.to_f64(out), ref["out"])
        print(f"[history] {name} round {r}: max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
        if cfg.dtype == "bf16":
            assert mx <= G.MAX_ABS and rr <= G.REL_RMS
        else:
            assert mx <= 1e-5
        np.testing.assert_allclose(G.to_f64(lse), ref["lse"], rtol=0,
                                   atol=G.lse_atol(cfg.dtype))
    # after the last round: both pools byte for byte (gaps and unused pages
    # keep the NaN fill on both sides)
    assert np.array_equal(G.bits(G.to_storage(pool.k_pages)), G.bits(ref["k_pool"]))
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(ref["v_pool"]))


@pytest.mark.parametrize("n_log,ps,start,stride,n", [
    (AlignedLayout(CONFIGS[4]).n_logical_pages, 256, AlignedLayout(CONFIGS[4]).window_start,
     AlignedLayout(CONFIGS[4]).chunk_stride, 3),
    (AlignedLayout(CONFIGS[5]).n_logical_pages, 256, AlignedLayout(CONFIGS[5]).window_start,
     AlignedLayout(CONFIGS[5]).chunk_stride, 5),
    (3000, 64, 64 * 5, 64 * 997, 3),            # 2991 entries: ragged over 1024 threads
    (16384 + 7, 16, 16 * 3, 16 * 4096, 4),      # the 16384-page limit
])
def test_table_rotation_bit_exact(n_log, ps, start, stride, n):
    rng = np.random.default_rng(n_log)
    table = rng.permutation(2 * n_log)[:n_log].astype(np.int32)
    dev = torch.from_numpy(table).to(G.DEV)
    pool = wf.KVPool(torch.empty(1, 1, ps, 64, dtype=torch.bfloat16, device=G.DEV),
                     torch.empty(1, 1, 64, ps, dtype=torch.bfloat16, device=G.DEV), dev)
    ref = table
    for i in range(n):
        wf.wf_history_rotate(pool, start, stride, n)
        ref = rotate_history(ref, ps, start, stride, n)
        got = dev.cpu().numpy()
        assert np.array_equal(got, ref), i
    assert np.array_equal(dev.cpu().numpy(), table)     # n rotations: identity
