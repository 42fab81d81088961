"""GPU parity of libwf against the CPU oracle (MI355X, through the C ABI).

publish: bit-exact, byte for byte over the whole pool (written rows, NaN
fill, stale pages).  attention: max-abs <= 2e-2 and relative RMS <= 5e-3
against the float64 oracle; LSE within the derived bound (4e-3 bf16, 1e-5
fp32).  Shapes span several query and
key tiles, ragged query tails, unaligned slot boundaries, every page-size
regime (smaller than, equal to and larger than a 64-key tile), head_dim 64
and 128, bf16 and fp32.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import CONFIGS, make_workload, small_config
from oracle.attention import chunk_attention
from tests import _gpu as G
from tests._pipeline import oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()          # fails loudly if libwf.so is missing


def medium(**kw):
    base = dict(name="medium", heads=3, frame_rows=10, frame_cols=13, frames_per_chunk=3,
                anchor_tokens=130, n_hist=2, slots=4, page_size=64, seed=21)
    base.update(kw)
    return small_config(**base)


SHAPES = {
    "tiny_fp32": CONFIGS[1],
    "small_ps16": small_config(),
    "small_d64_ps32": small_config(head_dim=64, rope=(24, 20, 20), page_size=32, seed=12),
    "medium_ps64": medium(),
    "medium_ps256_stale": medium(page_size=256, stale_frac=0.1, seed=22),
    "medium_ps128_hot": medium(page_size=128, hot_frac=0.01, seed=23),
    "medium_d64_ps1024": medium(head_dim=64, rope=(24, 20, 20), page_size=1024, seed=24),
    "fp32_d128_ps64": small_config(dtype="fp32", page_size=64, seed=13),
    "w1_dense": medium(slots=1, seed=25),
    "w6_ps16": small_config(slots=6, frames_per_chunk=1, seed=14),
    # chunk 360 = 256 + 104: a short partial last query tile in every slot
    "medium_packed_ps64": medium(frame_cols=12, seed=26),
    "medium_packed_w5_ps256": medium(frame_cols=12, slots=5, page_size=256, seed=27),
}


@pytest.fixture(scope="module", params=list(SHAPES), ids=list(SHAPES))
def case(request):
    cfg = SHAPES[request.param]
    print(f"\n[case] {request.param}: {cfg}", flush=True)
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    pool, q, dev = G.gpu_layer(wl)
    torch.cuda.synchronize()
    return wl, ref, pool, q, dev


def test_publish_bit_exact(case):
    wl, ref, pool, q, dev = case
    assert np.array_equal(G.bits(G.to_storage(pool.k_pages)), G.bits(ref["k_pool"]))
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(ref["v_pool"]))
    assert wf.wf_device_status() == 0


def test_attention_matches_oracle(case):
    wl, ref, pool, q, dev = case
    c = wl.cfg
    out, lse = G.attn(wl, pool, q)
    o_ref, l_ref = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                                   c.segments(), ref["q"], c.q_slot_start(), 0, c.scale, c.dtype)
    got = G.to_f64(out)
    assert np.isfinite(got).all()
    mx, rr = G.err_stats(got, o_ref)
    lse_err = float(np.abs(G.to_f64(lse) - l_ref).max())
    print(f"max-abs {mx:.3e} rel-rms {rr:.3e} lse {lse_err:.2e}", flush=True)
    G.record("attention", workload=c.name, dtype=c.dtype, heads=c.heads, head_dim=c.head_dim,
             page_size=c.page_size, rows=c.n_q, keys=c.n_kv, max_abs=mx, rel_rms=rr,
             lse_max=lse_err, all_elements=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    np.testing.assert_allclose(G.to_f64(lse), l_ref, rtol=0, atol=G.lse_atol(c.dtype))
    assert wf.wf_device_status() == 0


def test_publish_rotates_q_in_place(case):
    wl, ref, pool, q, dev = case
    c = wl.cfg
    n = min(c.n_q, 200)
    q_io = wl.q[:n].to(G.DEV).clone()
    scratch = G.gpu_pool(wl)
    wf.wf_kv_publish(scratch, dev["k"][:n], dev["v"][:n], 0, pos=dev["pos"][:n],
                     rope=(c.rope, c.theta), q=q_io)
    from oracle.publish import publish
    kp, vp = ref["k_pool"].copy(), ref["v_pool"].copy()
    _, q_rot = publish(kp, vp, wl.page_table, c.page_size, G.to_storage(wl.k[:n]),
                       G.to_storage(wl.v[:n]), wl.pos[:n], 0, c.dtype,
                       rope=(c.rope, c.theta), q=G.to_storage(wl.q[:n]))
    assert np.array_equal(G.bits(G.to_storage(q_io)), G.bits(q_rot))


def test_plain_scatter_and_unaligned_window():
    """rope = NULL copies K as is; a window starting mid-run and mid-page
    writes exactly its rows."""
    wl = make_workload(medium(page_size=128, seed=31))
    c = wl.cfg
    pool = G.gpu_pool(wl)
    k, v = wl.k.to(G.DEV), wl.v.to(G.DEV)
    dst, n = 203, 777
    wf.wf_kv_publish(pool, k[:n], v[:n], dst)
    from oracle.publish import publish
    from tests._pipeline import empty_pool
    kp, vp = empty_pool(wl)
    publish(kp, vp, wl.page_table, c.page_size, G.to_storage(wl.k[:n]), G.to_storage(wl.v[:n]),
            None, dst, c.dtype)
    assert np.array_equal(G.bits(G.to_storage(pool.k_pages)), G.bits(kp))
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(vp))


def _factor_table_tiles(pos, rope, head_dim, tile=64):
    """(tiles that fit the K blocks' factor table, tiles that do not): a
    64-token tile fits when sum over the axes of (pairs of the axis) x
    (position range of the axis) is at most the table's capacity, the LDS
    of 32 tokens' per-element factors less the tile's positions, header and
    row bases, in 8-byte (cos, sin) entries."""
    pairs = (rope[0] // 2, rope[1] // 2, head_dim // 2 - (rope[0] + rope[1]) // 2)
    cap = (tile // 2 * (head_dim // 2) * 8 - tile * 16 - 32 - (head_dim // 2) * 4) // 8
    fit = 0
    n_tiles = -(-len(pos) // tile)
    for b in range(n_tiles):
        p = pos[b * tile:(b + 1) * tile].astype(np.int64)
        need = sum(pr * (int(p[:, a].max()) - int(p[:, a].min()) + 1) for a, pr in enumerate(pairs))
        fit += need <= cap
    return fit, n_tiles - fit


@pytest.mark.parametrize(
    "kw",
    [dict(page_size=64, seed=51), dict(head_dim=64, rope=(24, 20, 20), page_size=32, seed=52),
     dict(dtype="fp32", page_size=64, seed=53)],
    ids=["bf16_d128_ps64", "bf16_d64_ps32", "fp32_d128_ps64"])
def test_publish_positions_beyond_the_factor_table(kw):
    """The first half of the tokens keep the frame grid (their K blocks
    rotate from the per-tile factor table), the second half take positions
    spread over +-50000 per axis (far more (pair, position) combinations per
    tile than the table holds: per-element factors).  One call; the pools
    and the rotated Q bit-exact against the oracle."""
    wl = make_workload(medium(**kw))
    c = wl.cfg
    n = c.n_kv
    rng = np.random.default_rng(c.seed)
    pos = rng.integers(-50000, 50000, size=(n, 3)).astype(np.int32)
    pos[: n // 2] = wl.pos[: n // 2]
    fit, spill = _factor_table_tiles(pos, c.rope, c.head_dim)
    assert fit > 0 and spill > 0
    g = torch.Generator().manual_seed(c.seed)
    q = torch.randn(n, c.heads, c.head_dim, generator=g).to(wl.torch_dtype)
    pool = G.gpu_pool(wl)
    q_io = q.to(G.DEV).clone()
    wf.wf_kv_publish(pool, wl.k.to(G.DEV), wl.v.to(G.DEV), 0, pos=torch.from_numpy(pos).to(G.DEV),
                     rope=(c.rope, c.theta), q=q_io)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    from oracle.publish import publish
    from tests._pipeline import empty_pool
    kp, vp = empty_pool(wl)
    _, q_rot = publish(kp, vp, wl.page_table, c.page_size, G.to_storage(wl.k), G.to_storage(wl.v),
                       pos, 0, c.dtype, rope=(c.rope, c.theta), q=G.to_storage(q))
    assert np.array_equal(G.bits(G.to_storage(pool.k_pages)), G.bits(kp))
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(vp))
    assert np.array_equal(G.bits(G.to_storage(q_io)), G.bits(q_rot))


@pytest.mark.parametrize("cols", [13, 12], ids=["chunk390", "chunk360_packed"])
def test_first_slot_share_equals_full_call(cols):
    """One slot per call equals that slot's rows of the full call, bit for
    bit (chunk 390 and 360: partial last query tiles of 134 and 104 rows)."""
    wl = make_workload(medium(frame_cols=cols, seed=32))
    c = wl.cfg
    pool, q, _ = G.gpu_layer(wl)
    full, lse_full = G.attn(wl, pool, q)
    qs = c.q_slot_start()
    for s in range(c.slots):
        r0, r1 = qs[s], qs[s + 1]
        part, lse_part = G.attn(wl, pool, q[r0:r1].contiguous(), q_slot_start=[0, r1 - r0],
                                first_slot=s)
        assert torch.equal(part, full[r0:r1])
        assert torch.equal(lse_part, lse_full[:, r0:r1])


def test_segments_with_gaps_and_any_order():
    """Segments laid out in reverse order with NaN gaps between them give the
    oracle's result for that layout."""
    cfg = medium(seed=33, page_size=64)
    wl = make_workload(cfg)
    c = wl.cfg
    ref = oracle_layer(wl)
    segs = c.segments()
    new_segs, cursor = [], 0
    for st, ln, slot in reversed(segs):
        new_segs.append((cursor, ln, slot))
        cursor += ln + 37
    n_log = -(-cursor // c.page_size)
    table = torch.randperm(n_log, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    pool = wf.KVPool.empty(n_log, c.heads, c.page_size, c.head_dim, table,
                           dtype=torch.bfloat16, device=G.DEV)
    pool.k_pages.view(torch.int16).fill_(0x7FC1)
    pool.v_pages.view(torch.int16).fill_(0x7FC1)
    k_rot = torch.from_numpy(ref["k_rot"].view(np.int16)).view(torch.bfloat16).to(G.DEV)
    v = wl.v.to(G.DEV)
    for (st, ln, _), (nst, _, _) in zip(reversed(segs), new_segs):
        wf.wf_kv_publish(pool, k_rot[st:st + ln], v[st:st + ln], nst)
    q = wl.q.to(G.DEV)
    out, _ = G.attn(wl, pool, q, segments=new_segs)
    o_ref, _ = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size, segs,
                               ref["q"], c.q_slot_start(), 0, c.scale, c.dtype)
    mx, rr = G.err_stats(G.to_f64(out), o_ref)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS


def test_degenerate_calls():
    """Edge cases of the slot layout: a publish of zero tokens leaves the pool
    untouched; slots with no rows (first, middle and last) and a slot of one
    row give the oracle's rows for the others and write nothing else; a call
    with no rows at all writes nothing."""
    cfg = medium(seed=34)
    wl = make_workload(cfg)
    c = wl.cfg
    ref = oracle_layer(wl)
    pool, q, _ = G.gpu_layer(wl)
    k_before, v_before = pool.k_pages.clone(), pool.v_pages.clone()
    wf.wf_kv_publish(pool, wl.k[:0].to(G.DEV), wl.v[:0].to(G.DEV), 0,
                     pos=torch.zeros((0, 3), dtype=torch.int32, device=G.DEV),
                     rope=(c.rope, c.theta))
    torch.cuda.synchronize()
    assert torch.equal(pool.k_pages.view(torch.int16), k_before.view(torch.int16))
    assert torch.equal(pool.v_pages.view(torch.int16), v_before.view(torch.int16))
    qs = c.q_slot_start()
    C = qs[1] - qs[0]
    # slot 0 empty, slot 1 one row, slot 2 empty, slot 3 its full chunk
    layouts = {
        "empty_first_one_row": [0, 0, 1, 1, 1 + C],
        "empty_last": [0, C, 2 * C, 3 * C, 3 * C],
        "no_rows": [0, 0, 0, 0, 0],
    }
    from oracle.attention import chunk_attention
    for name, lay in layouts.items():
        print(f"[case] {name}: q_slot_start {lay}", flush=True)
        n = lay[-1]
        rows = q[:max(n, 1)].contiguous()
        out, lse = G.attn(wl, pool, rows, q_slot_start=lay)
        assert wf.wf_device_status() == 0
        if n == 0:
            assert torch.isnan(out).all() and torch.isnan(lse).all()
            continue
        o_ref, l_ref = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                                       c.segments(), ref["q"][:n], lay, 0, c.scale, c.dtype)
        mx, rr = G.err_stats(G.to_f64(out[:n]), o_ref)
        assert mx <= G.MAX_ABS and rr <= G.REL_RMS, (name, mx, rr)
        np.testing.assert_allclose(G.to_f64(lse)[:, :n], l_ref, rtol=0,
                                   atol=G.lse_atol(c.dtype))
