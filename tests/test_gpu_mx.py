"""GPU parity of the 8-bit QK^T variant (wf_kv_publish_mx, wf_chunk_attn_mx)
against the CPU oracle (oracle/mx.py), through the C ABI on MI355X.

publish: the MXFP8 key codes and scales bit-exact against the oracle's
quantization of the oracle's RoPE'd keys, over the whole key pools (fill
included), and the V pool byte for byte.  attention: against the float64
attention on the decoded MXFP8 queries and keys, with the bfloat16 path's
bars (max-abs <= 2e-2, relative RMS <= 5e-3, LSE within 4e-3): the scores
themselves are exact products summed in float32, so what remains is the
same bfloat16 rounding of the probabilities.  The distance to the
unquantized attention is printed and loosely bounded.  Shapes cover every
page-size regime (16 < 64-key tile <= 64, 256), stale pages, hot keys,
ragged query tails and unaligned slot boundaries; the 14B-like shape runs
at full size on sampled rows.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import CONFIGS, make_workload, small_config
from oracle.attention import chunk_attention
from oracle.mx import mx_chunk_attention, mx_publish_keys
from tests import _gpu as G
from tests._pipeline import oracle_layer

pytestmark = pytest.mark.gpu

CODE_FILL, SCALE_FILL = 0x7F, 0x55     # never-written bytes: NaN codes, odd scales


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


def medium(**kw):
    base = dict(name="medium", heads=3, frame_rows=10, frame_cols=13, frames_per_chunk=3,
                anchor_tokens=130, n_hist=2, slots=4, page_size=64, seed=41)
    base.update(kw)
    return small_config(**base)


SHAPES = {
    "small_ps16": small_config(seed=42),
    "medium_ps64": medium(),
    "medium_ps256_stale": medium(page_size=256, stale_frac=0.1, seed=43),
    "medium_ps128_hot": medium(page_size=128, hot_frac=0.01, seed=44),
    "w1_dense_ps32": medium(slots=1, page_size=32, seed=45),
}


def gpu_mx_layer(wl):
    """wf_kv_publish_mx of the resident prefix, then of the round (the two
    calls of the bfloat16 pipeline)."""
    c = wl.cfg
    pool = G.gpu_pool(wl)
    keys = wf.MXKeys.empty(c.n_pages, c.heads, c.page_size, c.head_dim)
    keys.codes.fill_(CODE_FILL)
    keys.scales.fill_(SCALE_FILL)
    k, v = wl.k.to(G.DEV), wl.v.to(G.DEV)
    pos = torch.from_numpy(wl.pos).to(G.DEV)
    rp = (c.rope, c.theta)
    ss = c.store_start
    if ss:
        wf.wf_kv_publish_mx(pool, keys, k[:ss], v[:ss], 0, pos=pos[:ss], rope=rp)
    wf.wf_kv_publish_mx(pool, keys, k[ss:], v[ss:], ss, pos=pos[ss:], rope=rp)
    return pool, keys, wl.q.to(G.DEV)


def oracle_mx_keys(wl, ref):
    c = wl.cfg
    k8 = np.full((c.n_pages, c.heads, c.page_size, c.head_dim), CODE_FILL, np.uint8)
    k8s = np.full((c.n_pages, c.heads, c.page_size, c.head_dim // 32), SCALE_FILL, np.uint8)
    mx_publish_keys(k8, k8s, wl.page_table, c.page_size, ref["k_rot"], 0, c.dtype)
    return k8, k8s


@pytest.fixture(scope="module", params=list(SHAPES), ids=list(SHAPES))
def case(request):
    cfg = SHAPES[request.param]
    print(f"\n[mx] {request.param}: {cfg}", flush=True)
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    k8, k8s = oracle_mx_keys(wl, ref)
    pool, keys, q = gpu_mx_layer(wl)
    torch.cuda.synchronize()
    return wl, ref, k8, k8s, pool, keys, q


def test_publish_mx_positions_beyond_the_factor_table():
    """As the bfloat16 case: half the tokens on the frame grid (factor table),
    half with positions spread over +-50000 (per-element factors), one
    call; the 8-bit key codes, their scales and the V pool bit-exact."""
    wl = make_workload(medium(page_size=64, seed=54))
    c = wl.cfg
    n = c.n_kv
    rng = np.random.default_rng(c.seed)
    pos = rng.integers(-50000, 50000, size=(n, 3)).astype(np.int32)
    pos[: n // 2] = wl.pos[: n // 2]
    from tests.test_gpu_parity import _factor_table_tiles
    fit, spill = _factor_table_tiles(pos, c.rope, c.head_dim)
    assert fit > 0 and spill > 0
    pool = G.gpu_pool(wl)
    keys = wf.MXKeys.empty(c.n_pages, c.heads, c.page_size, c.head_dim)
    keys.codes.fill_(CODE_FILL)
    keys.scales.fill_(SCALE_FILL)
    wf.wf_kv_publish_mx(pool, keys, wl.k.to(G.DEV), wl.v.to(G.DEV), 0,
                        pos=torch.from_numpy(pos).to(G.DEV), rope=(c.rope, c.theta))
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    from oracle.publish import publish
    from tests._pipeline import empty_pool
    kp, vp = empty_pool(wl)
    k_rot, _ = publish(kp, vp, wl.page_table, c.page_size, G.to_storage(wl.k),
                       G.to_storage(wl.v), pos, 0, c.dtype, rope=(c.rope, c.theta))
    k8 = np.full((c.n_pages, c.heads, c.page_size, c.head_dim), CODE_FILL, np.uint8)
    k8s = np.full((c.n_pages, c.heads, c.page_size, c.head_dim // 32), SCALE_FILL, np.uint8)
    mx_publish_keys(k8, k8s, wl.page_table, c.page_size, k_rot, 0, c.dtype)
    assert np.array_equal(keys.codes.cpu().numpy(), k8)
    assert np.array_equal(keys.scales.cpu().numpy(), k8s)
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(vp))


def test_publish_mx_bit_exact(case):
    wl, ref, k8, k8s, pool, keys, q = case
    assert wf.wf_device_status() == 0
    assert np.array_equal(keys.codes.cpu().numpy(), k8)
    assert np.array_equal(keys.scales.cpu().numpy(), k8s)
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(ref["v_pool"]))


def test_attention_mx_parity(case):
    wl, ref, k8, k8s, pool, keys, q = case
    c = wl.cfg
    out = torch.full_like(q, float("nan"))
    lse = torch.full((c.heads, c.n_q), float("nan"), device=G.DEV)
    wf.wf_chunk_attn_mx(pool, keys, c.segments(), q, c.q_slot_start(), 0, c.scale, out=out,
                        lse=lse)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    o_ref, l_ref = mx_chunk_attention(k8, k8s, ref["v_pool"], wl.page_table, c.page_size,
                                      c.segments(), ref["q"], c.q_slot_start(), 0, c.scale)
    got = G.to_f64(out)
    assert np.isfinite(got).all()
    mx, rr = G.err_stats(got, o_ref)
    o16, _ = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                             c.segments(), ref["q"], c.q_slot_start(), 0, c.scale, c.dtype)
    qmx, qrr = G.err_stats(got, o16)
    print(f"[mx] parity max-abs {mx:.3e} rel-rms {rr:.3e}; vs unquantized max-abs {qmx:.3e} "
          f"rel-rms {qrr:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    np.testing.assert_allclose(G.to_f64(lse), l_ref, rtol=0, atol=G.lse_atol("bf16"))
    assert qrr < 0.1


@pytest.mark.timeout(900)
def test_full_size_14b_sampled():
    cfg = CONFIGS[4]
    print(f"\n[mx] full size: {cfg.name}", flush=True)
    wl = make_workload(cfg)
    pool, keys, q = gpu_mx_layer(wl)
    out = torch.empty_like(q)
    lse = torch.empty((cfg.heads, cfg.n_q), device=G.DEV)
    wf.wf_chunk_attn_mx(pool, keys, cfg.segments(), q, cfg.q_slot_start(), 0, cfg.scale,
                        out=out, lse=lse)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    assert torch.isfinite(out.float()).all().item()
    print("[mx] gpu done; oracle", flush=True)
    ref = oracle_layer(wl)
    k8, k8s = oracle_mx_keys(wl, ref)
    assert np.array_equal(keys.codes.cpu().numpy(), k8)
    assert np.array_equal(keys.scales.cpu().numpy(), k8s)
    rng = np.random.default_rng(4)
    qs = cfg.q_slot_start()
    rows = {}
    for g in range(cfg.slots):
        r0, r1 = qs[g], qs[g + 1]
        rows[g] = np.array(sorted(set(range(r0, r0 + 3)) | set(range(r1 - 3, r1)) |
                                  set(rng.integers(r0, r1, size=6).tolist())))
    heads = [0, 17, cfg.heads - 1]
    o_ref, l_ref = mx_chunk_attention(k8, k8s, ref["v_pool"], wl.page_table, cfg.page_size,
                                      cfg.segments(), ref["q"], qs, 0, cfg.scale, heads=heads,
                                      rows=rows)
    sel = np.concatenate(list(rows.values()))
    got = out[torch.from_numpy(sel).to(G.DEV)][:, heads].float().cpu().numpy().astype(np.float64)
    mx, rr = G.err_stats(got, o_ref[sel][:, heads])
    print(f"[mx] 14B-like sampled max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    np.testing.assert_allclose(G.to_f64(lse)[heads][:, sel], l_ref[heads][:, sel], rtol=0,
                               atol=G.lse_atol("bf16"))


def test_mx_segments_with_gaps_and_any_order():
    """Segments in reverse order with gaps of never-written bytes (NaN codes)
    between them: the 8-bit attention still reads only the named keys."""
    cfg = medium(seed=46, page_size=64)
    wl = make_workload(cfg)
    c = wl.cfg
    ref = oracle_layer(wl)
    segs = c.segments()
    new_segs, cursor = [], 0
    for st, ln, slot in reversed(segs):
        new_segs.append((cursor, ln, slot))
        cursor += ln + 37
    n_log = -(-cursor // c.page_size)
    table = torch.randperm(n_log, generator=torch.Generator().manual_seed(4)).to(torch.int32)
    pool = wf.KVPool.empty(n_log, c.heads, c.page_size, c.head_dim, table, device=G.DEV)
    pool.v_pages.view(torch.int16).fill_(0x7FC1)
    keys = wf.MXKeys.empty(n_log, c.heads, c.page_size, c.head_dim)
    keys.codes.fill_(CODE_FILL)
    keys.scales.fill_(SCALE_FILL)
    k_rot = torch.from_numpy(ref["k_rot"].view(np.int16)).view(torch.bfloat16).to(G.DEV)
    v = wl.v.to(G.DEV)
    k8 = np.full((n_log, c.heads, c.page_size, c.head_dim), CODE_FILL, np.uint8)
    k8s = np.full((n_log, c.heads, c.page_size, c.head_dim // 32), SCALE_FILL, np.uint8)
    vp = np.full((n_log, c.heads, c.head_dim, c.page_size), 0x7FC1, np.uint16)
    from oracle.publish import publish
    for (st, ln, _), (nst, _, _) in zip(reversed(segs), new_segs):
        wf.wf_kv_publish_mx(pool, keys, k_rot[st:st + ln], v[st:st + ln], nst)
        mx_publish_keys(k8, k8s, table.numpy(), c.page_size, ref["k_rot"][st:st + ln], nst, "bf16")
        publish(np.zeros((n_log, c.heads, c.page_size, c.head_dim), np.uint16), vp, table.numpy(),
                c.page_size, ref["k_rot"][st:st + ln], ref["v"][st:st + ln], None, nst, "bf16")
    q = wl.q.to(G.DEV)
    out = wf.wf_chunk_attn_mx(pool, keys, new_segs, q, c.q_slot_start(), 0, c.scale)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    assert np.array_equal(keys.codes.cpu().numpy(), k8)
    o_ref, _ = mx_chunk_attention(k8, k8s, vp, table.numpy(), c.page_size, new_segs, ref["q"],
                                  c.q_slot_start(), 0, c.scale)
    mx, rr = G.err_stats(G.to_f64(out), o_ref)
    print(f"[mx] gaps/any order: max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
