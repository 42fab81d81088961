"""GPU parity of wf_group_attn (query groups with explicit key runs) against
the CPU oracle, through the C ABI on MI355X.

Layouts from workloads.query_groups: the store stage (the store chunk's
queries over anchor | history | store), a group over three random unaligned
runs listed out of order, and a group over the whole context given as one
run per segment.  Same tolerances as wf_chunk_attn; rows outside every group
must stay untouched.  The slot rule written out as groups must give exactly
wf_chunk_attn's output (one kernel serves both).
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import CONFIGS, make_workload, query_groups, small_config
from oracle.attention import group_attention
from tests import _gpu as G
from tests._pipeline import oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


def medium(**kw):
    base = dict(name="medium", heads=3, frame_rows=10, frame_cols=13, frames_per_chunk=3,
                anchor_tokens=130, n_hist=2, slots=4, page_size=64, seed=21)
    base.update(kw)
    return small_config(**base)


SHAPES = {
    "tiny_fp32": CONFIGS[1],
    "small_ps16": small_config(),
    "medium_ps64": medium(),
    "medium_ps256_stale": medium(page_size=256, stale_frac=0.1, seed=22),
    "medium_d64_ps1024": medium(head_dim=64, rope=(24, 20, 20), page_size=1024, seed=24),
    "fp32_d128_ps64": small_config(dtype="fp32", page_size=64, seed=13),
}


@pytest.fixture(scope="module", params=list(SHAPES), ids=list(SHAPES))
def case(request):
    cfg = SHAPES[request.param]
    print(f"\n[case] {request.param}: {cfg}", flush=True)
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    pool, q, dev = G.gpu_layer(wl)
    torch.cuda.synchronize()
    return wl, ref, pool, q


@pytest.mark.parametrize("seed", [1, 2])
def test_group_attention_matches_oracle(case, seed):
    wl, ref, pool, q = case
    c = wl.cfg
    runs, groups = query_groups(c, seed=seed)
    extra = 7                                   # lse rows beyond the last group row
    lse = torch.full((c.heads, c.n_q + extra), float("nan"), device=G.DEV)
    out = torch.full_like(q, float("nan"))
    wf.wf_group_attn(pool, runs, groups, q, c.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = group_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                                   runs, groups, ref["q"], c.scale, c.dtype)
    got = G.to_f64(out)
    covered = np.zeros(c.n_q, dtype=bool)
    for (r0, r1, _, _) in groups:
        covered[r0:r1] = True
    assert np.isfinite(got[covered]).all() and np.isnan(got[~covered]).all()
    mx, rr = G.err_stats(got[covered], o_ref[covered])
    print(f"max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    l_got = G.to_f64(lse)
    np.testing.assert_allclose(l_got[:, :c.n_q][:, covered], l_ref[:, covered], rtol=0,
                               atol=G.lse_atol(c.dtype))
    assert np.isnan(l_got[:, c.n_q:]).all()
    assert wf.wf_device_status() == 0


def test_slot_rule_as_groups_equals_chunk_attn():
    wl = make_workload(medium(seed=26))
    pool, q, _ = G.gpu_layer(wl)
    c = wl.cfg
    runs, groups = [], []
    qss = c.q_slot_start()
    for s in range(c.slots):
        mine = [(st, ln) for (st, ln, sl) in c.segments() if sl < 0 or sl >= s]
        groups.append((qss[s], qss[s + 1], len(runs), len(runs) + len(mine)))
        runs += mine
    out_c, lse_c = G.attn(wl, pool, q)
    lse_g = torch.full_like(lse_c, float("nan"))
    out_g = torch.full_like(q, float("nan"))
    wf.wf_group_attn(pool, runs, groups, q, c.scale, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.int16), out_g.view(torch.int16))
    assert torch.equal(lse_c, lse_g)


def test_store_stage_alone_on_offset_rows():
    """One group whose rows start mid-buffer: only those rows are written."""
    wl = make_workload(medium(seed=27))
    ref = oracle_layer(wl)
    pool, q, _ = G.gpu_layer(wl)
    c = wl.cfg
    r0, r1 = 100, 100 + c.chunk
    runs, groups = [(0, c.prefix)], [(r0, r1, 0, 1)]
    out = torch.full_like(q, float("nan"))
    wf.wf_group_attn(pool, runs, groups, q, c.scale, out=out)
    torch.cuda.synchronize()
    o_ref, _ = group_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size, runs,
                               groups, ref["q"], c.scale, c.dtype)
    got = G.to_f64(out)
    assert np.isnan(got[:r0]).all() and np.isnan(got[r1:]).all()
    mx, rr = G.err_stats(got[r0:r1], o_ref[r0:r1])
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS


@pytest.mark.parametrize("cuts", [(1000,), (333, 1347), (64, 65, 1900)], ids=["2", "3", "4"])
def test_lse_merge_of_key_partitions(cuts):
    """Attention of all query rows over disjoint key ranges (unaligned cuts,
    one range a single key), merged on the host by e^LSE, against the
    oracle over the union: the LSE the kernel reports is the normalizer of
    the O it returns, so partial results combine (as a split of the keys
    across calls or devices would) within the single call's tolerances."""
    cfg = medium(page_size=64, seed=31)
    assert cuts[-1] < cfg.n_kv
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    pool, q, _ = G.gpu_layer(wl)
    c = wl.cfg
    print(f"\n[case] key partition at {cuts}: {cfg}", flush=True)
    edges = [0, *cuts, c.n_kv]
    outs, lses = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        out = torch.full_like(q, float("nan"))
        lse = torch.full((c.heads, c.n_q), float("nan"), device=G.DEV)
        wf.wf_group_attn(pool, [(a, b - a)], [(0, c.n_q, 0, 1)], q, c.scale, out=out, lse=lse)
        outs.append(G.to_f64(out))
        lses.append(G.to_f64(lse))
    torch.cuda.synchronize()
    lse = np.stack(lses)                              # [P, H, n]
    top = lse.max(axis=0)
    w = np.exp(lse - top)
    den = w.sum(axis=0)
    merged = sum(w[i].T[:, :, None] * outs[i] for i in range(len(outs))) / den.T[:, :, None]
    o_ref, l_ref = group_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                                   [(0, c.n_kv)], [(0, c.n_q, 0, 1)], ref["q"], c.scale, c.dtype)
    mx, rr = G.err_stats(merged, o_ref)
    dl = np.abs(top + np.log(den) - l_ref).max()
    print(f"merged: max-abs {mx:.3e} rel-rms {rr:.3e} lse {dl:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    assert dl <= G.lse_atol(c.dtype)
