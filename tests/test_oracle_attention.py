"""Pins for the oracle's chunk-wise causal attention (CPU only).

"Wave Forcing", §3.1 fixes: full attention within a chunk; slot s sees slot
j iff j >= s; anchor, history and store are seen by every slot.  Pins:
  - one slot (W = 1) reduces to dense attention: torch's fp64
    scaled_dot_product_attention on CPU and torch.logsumexp;
  - brute force with per-key visibility on tiny inputs (fp32 and bf16);
  - perturbing K/V of slots j < s leaves slot s bit-identical, while
    perturbing slot j >= s or the prefix changes it (non-vacuity);
  - physical page permutation invariance (exact);
  - softmax rows sum to 1; V == 1 gives O == 1; a dominant key wins;
  - the order of segments in logical space does not change the result.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd.workloads import CONFIGS, make_workload, small_config
from oracle.attention import chunk_attention, probabilities, visible_tokens
from oracle.brute import brute_attention
from oracle.publish import publish
from tests._pipeline import empty_pool, f64, oracle_layer, storage


def _attn(wl, ref, **kw):
    c = wl.cfg
    args = dict(k_pool=ref["k_pool"], v_pool=ref["v_pool"], page_table=wl.page_table,
                page_size=c.page_size, segments=c.segments(), q=ref["q"],
                q_slot_start=c.q_slot_start(), first_slot=0, scale=c.scale, dtype=c.dtype)
    args.update(kw)
    return chunk_attention(**args)


@pytest.mark.parametrize("prefix", [True, False])
def test_single_slot_is_dense_attention(prefix):
    cfg = small_config(slots=1, n_hist=1 if prefix else 0,
                       anchor_tokens=24 if prefix else 0)
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    segs = c.segments() if prefix else [(c.prefix, c.chunk, 0)]
    out, lse = _attn(wl, ref, segments=segs)
    toks = visible_tokens(segs, 0)
    q = torch.from_numpy(f64(ref["q"], c.dtype)).permute(1, 0, 2)      # [H, n, D]
    k = torch.from_numpy(f64(ref["k_rot"], c.dtype)[toks]).permute(1, 0, 2).contiguous()
    v = torch.from_numpy(f64(ref["v"], c.dtype)[toks]).permute(1, 0, 2).contiguous()
    o_ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=c.scale)
    np.testing.assert_allclose(out, o_ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    l_ref = torch.logsumexp(c.scale * torch.matmul(q, k.transpose(1, 2).contiguous()), dim=-1)
    np.testing.assert_allclose(lse, l_ref.numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("cfg", [CONFIGS[1], small_config()], ids=["tiny_fp32", "small_bf16"])
def test_matches_brute_force(cfg):
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    out, lse = _attn(wl, ref)
    bo, bl = brute_attention(f64(ref["q"], c.dtype), f64(ref["k_rot"], c.dtype),
                             f64(ref["v"], c.dtype), c.segments(), c.q_slot_start(),
                             0, c.scale)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def _republish_with(wl, ref, tokens, k_new, v_new):
    c = wl.cfg
    kp, vp = ref["k_pool"].copy(), ref["v_pool"].copy()
    for t, L in enumerate(tokens):
        publish(kp, vp, wl.page_table, c.page_size, k_new[t:t + 1], v_new[t:t + 1],
                None, int(L), c.dtype)
    return kp, vp


@pytest.mark.parametrize("s", [1, 2])
def test_mask_perturbation_invariance(s):
    """Slot s output is bit-identical when K/V of every slot j < s change
    (even to NaN), and changes when any slot j >= s or the prefix does."""
    cfg = small_config()
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    out0, lse0 = _attn(wl, ref)
    rows = slice(c.q_slot_start()[s], c.q_slot_start()[s + 1])
    rng = np.random.default_rng(5)

    def perturbed(tokens, nan=False):
        n = len(tokens)
        shape = (n, c.heads, c.head_dim)
        if nan:
            kk = np.full(shape, 0x7FC1, np.uint16)
            vv = kk.copy()
        else:
            kk = storage(torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16), "bf16")
            vv = storage(torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16), "bf16")
        kp, vp = _republish_with(wl, ref, tokens, kk, vv)
        return _attn(wl, dict(ref, k_pool=kp, v_pool=vp))

    lower = np.concatenate([np.arange(c.prefix + j * c.chunk, c.prefix + (j + 1) * c.chunk)
                            for j in range(s)])
    for nan in (False, True):
        o, l = perturbed(lower, nan)
        assert np.array_equal(o[rows], out0[rows]) and np.array_equal(l[:, rows], lse0[:, rows])
    # non-vacuity: self, a cleaner slot (if any) and the prefix all matter
    cands = [np.arange(c.prefix + s * c.chunk, c.prefix + s * c.chunk + 3),
             np.arange(0, 3), np.arange(c.store_start, c.store_start + 3)]
    if s + 1 < c.slots:
        cands.append(np.arange(c.prefix + (s + 1) * c.chunk, c.prefix + (s + 1) * c.chunk + 3))
    for toks in cands:
        o, _ = perturbed(toks)
        assert not np.allclose(o[rows], out0[rows], atol=1e-6)


def test_page_permutation_invariance():
    cfg = small_config(stale_frac=0.2)
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    out0, lse0 = _attn(wl, ref)
    c = wl.cfg
    rng = np.random.default_rng(6)
    new_place = rng.permutation(c.n_pages)          # physical p -> new_place[p]
    kp = np.empty_like(ref["k_pool"])
    vp = np.empty_like(ref["v_pool"])
    kp[new_place] = ref["k_pool"]
    vp[new_place] = ref["v_pool"]
    table = new_place[wl.page_table].astype(np.int32)
    out1, lse1 = chunk_attention(kp, vp, table, c.page_size, c.segments(), ref["q"],
                                 c.q_slot_start(), 0, c.scale, c.dtype)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_rows_sum_to_one_and_constant_v():
    cfg = small_config()
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    for s in range(c.slots):
        r0, r1 = c.q_slot_start()[s], c.q_slot_start()[s + 1]
        p = probabilities(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size,
                          c.segments(), ref["q"][r0:r1, 1], s, 1, c.scale, c.dtype)
        assert p.shape[1] == c.visible(s)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    vp = np.full_like(ref["v_pool"], 0x3F80)        # bf16 1.0 everywhere
    out, _ = _attn(wl, dict(ref, v_pool=vp))
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_dominant_key_wins():
    """One key with a far larger logit than all others takes the output."""
    cfg = small_config()
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    s, h = 1, 0
    i = c.q_slot_start()[s] + 5
    target = c.prefix + 2 * c.chunk + 7              # a token of slot 2 >= s
    kk = f64(ref["k_rot"][target:target + 1], "bf16")
    kk[0, h] = 400.0 * f64(ref["q"][i:i + 1, h], "bf16")[0] / np.sqrt(c.head_dim)
    kb = storage(torch.from_numpy(kk.astype(np.float32)).to(torch.bfloat16), "bf16")
    kp, vp = _republish_with(wl, ref, [target], kb, ref["v"][target:target + 1])
    out, _ = _attn(wl, dict(ref, k_pool=kp, v_pool=vp))
    np.testing.assert_allclose(out[i, h], f64(ref["v"][target, h], "bf16"), rtol=0, atol=1e-9)


def test_context_order_invariance():
    """Moving the segments around in logical space (slots first, prefix
    last, with gaps) gives the same attention up to float64 rounding."""
    cfg = small_config()
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    segs = c.segments()
    # new placement: reverse segment order, 16 tokens of gap between them
    new_segs, cursor = [], 0
    for st, ln, slot in reversed(segs):
        new_segs.append((cursor, ln, slot))
        cursor += ln + 16
    n_log = -(-cursor // c.page_size)
    kp = np.full((n_log, c.heads, c.page_size, c.head_dim), 0x7FC1, np.uint16)
    vp = np.full((n_log, c.heads, c.head_dim, c.page_size), 0x7FC1, np.uint16)
    table = np.arange(n_log, dtype=np.int32)
    for (st, ln, _), (nst, _, _) in zip(reversed(segs), new_segs):
        publish(kp, vp, table, c.page_size, ref["k_rot"][st:st + ln], ref["v"][st:st + ln],
                None, nst, c.dtype)
    out1, lse1 = chunk_attention(kp, vp, table, c.page_size, new_segs, ref["q"],
                                 c.q_slot_start(), 0, c.scale, c.dtype)
    out0, lse0 = _attn(wl, ref)
    np.testing.assert_allclose(out1, out0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-12)


def test_first_slot_share_equals_full_call():
    """Computing one slot's rows alone (first_slot = s, one group) gives the
    same rows as the call over all slots."""
    cfg = small_config()
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    out0, _ = _attn(wl, ref)
    s = 2
    r0, r1 = c.q_slot_start()[s], c.q_slot_start()[s + 1]
    out1, _ = _attn(wl, ref, q=ref["q"][r0:r1], q_slot_start=[0, r1 - r0], first_slot=s)
    assert np.array_equal(out1, out0[r0:r1])


def test_hot_rows_config_draws():
    cfg = small_config(hot_frac=0.05)
    wl = make_workload(cfg)
    assert len(wl.hot_rows) == round(0.05 * cfg.n_kv)
    big = np.abs(wl.k.float().numpy()).max(axis=(1, 2))
    assert big[wl.hot_rows].mean() > 4 * np.delete(big, wl.hot_rows).mean()


# ---- generic query groups (store stage, explicit key runs) -----------------

from chunk_wise_causal_amd.workloads import query_groups
from oracle.attention import group_attention, run_tokens
from oracle.brute import brute_group_attention


def _gattn(wl, ref, runs, groups):
    c = wl.cfg
    return group_attention(ref["k_pool"], ref["v_pool"], wl.page_table, c.page_size, runs,
                           groups, ref["q"], c.scale, c.dtype)


@pytest.mark.parametrize("cfg", [CONFIGS[1], small_config(slots=2)], ids=["tiny_fp32", "small_bf16"])
def test_group_attention_matches_brute_force(cfg):
    wl = make_workload(cfg)
    ref = oracle_layer(wl)
    c = wl.cfg
    runs, groups = query_groups(c, seed=1)
    out, lse = _gattn(wl, ref, runs, groups)
    bo, bl = brute_group_attention(f64(ref["q"], c.dtype), f64(ref["k_rot"], c.dtype),
                                   f64(ref["v"], c.dtype), runs, groups, c.scale)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_store_stage_is_dense_attention_over_the_prefix():
    """The store chunk's queries see anchor | history | store: dense
    attention (torch fp64 SDPA on CPU) over exactly those keys."""
    wl = make_workload(small_config())
    ref = oracle_layer(wl)
    c = wl.cfg
    runs, groups = [(0, c.prefix)], [(0, c.chunk, 0, 1)]
    out, lse = _gattn(wl, ref, runs, groups)
    q = torch.from_numpy(f64(ref["q"], c.dtype)[:c.chunk]).permute(1, 0, 2)
    k = torch.from_numpy(f64(ref["k_rot"], c.dtype)[:c.prefix]).permute(1, 0, 2).contiguous()
    v = torch.from_numpy(f64(ref["v"], c.dtype)[:c.prefix]).permute(1, 0, 2).contiguous()
    o_ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=c.scale)
    np.testing.assert_allclose(out[:c.chunk], o_ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    assert np.isnan(out[c.chunk:]).all() and np.isnan(lse[:, c.chunk:]).all()


def test_slot_rule_as_groups_reproduces_chunk_attention():
    """wf_chunk_attn's visibility written out as explicit runs per slot
    gives the same numbers through the group definition."""
    wl = make_workload(small_config())
    ref = oracle_layer(wl)
    c = wl.cfg
    runs, groups = [], []
    qss = c.q_slot_start()
    for s in range(c.slots):
        mine = [(st, ln) for (st, ln, sl) in c.segments() if sl < 0 or sl >= s]
        groups.append((qss[s], qss[s + 1], len(runs), len(runs) + len(mine)))
        runs += mine
    out, lse = _gattn(wl, ref, runs, groups)
    o2, l2 = _attn(wl, ref)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)


def test_run_tokens_is_the_union():
    assert list(run_tokens([(5, 2), (0, 3)])) == [0, 1, 2, 5, 6]


def _merge(parts):
    """Merge (out, lse) results over disjoint key sets by their natural-log
    LSE: weights e^lse, shifted by the row maximum."""
    lse = np.stack([p[1] for p in parts])            # [P, H, n]
    top = np.max(lse, axis=0)
    w = np.exp(lse - top)                            # [P, H, n]
    den = w.sum(axis=0)
    num = sum(w[i].T[:, :, None] * parts[i][0] for i in range(len(parts)))
    return num / den.T[:, :, None], top + np.log(den)


@pytest.mark.parametrize("cuts", [(1,), (37, 200), (64, 65, 201)], ids=["1", "2", "3"])
def test_lse_merges_key_partitions(cuts):
    """The LSE is the natural-log normalizer: attention over disjoint key
    sets, merged by e^LSE, gives attention over their union (an LSE in log2
    units or one that leaves out the scale fails this)."""
    wl = make_workload(small_config(slots=2, seed=5))
    ref = oracle_layer(wl)
    c = wl.cfg
    rows = (0, c.n_q)
    full = _gattn(wl, ref, [(0, c.n_kv)], [(*rows, 0, 1)])
    edges = [0, *cuts, c.n_kv]
    parts = [_gattn(wl, ref, [(a, b - a)], [(*rows, 0, 1)]) for a, b in zip(edges[:-1], edges[1:])]
    out, lse = _merge(parts)
    np.testing.assert_allclose(out, full[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, full[1], rtol=0, atol=1e-12)
