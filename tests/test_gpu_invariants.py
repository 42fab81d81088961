"""Properties of the GPU attention that the pages fix, checked bit for bit
("Wave Forcing", §3.1 and §4.2):
  - perturbing K/V of slots j < s (to noise or NaN) leaves slot s's output
    bit-identical; perturbing slot s itself or the prefix changes it;
  - a physical page permutation gives a bit-identical output;
  - NaN in unmapped pages and page tails never reaches the output;
  - V == 1 gives O == 1; repeated runs are bit-identical.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import make_workload, small_config
from tests import _gpu as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


def cfg(**kw):
    base = dict(heads=3, frame_rows=10, frame_cols=13, frames_per_chunk=3, anchor_tokens=130,
                n_hist=2, slots=4, page_size=64, stale_frac=0.15, seed=41)
    base.update(kw)
    return small_config(**base)


@pytest.mark.parametrize("ps", [16, 64, 256])
def test_mask_perturbation_bit_identical(ps):
    wl = make_workload(cfg(page_size=ps))
    c = wl.cfg
    pool, q, dev = G.gpu_layer(wl)
    out0, lse0 = G.attn(wl, pool, q)
    qs = c.q_slot_start()
    for s in range(1, c.slots):
        lo = c.prefix
        hi = c.prefix + s * c.chunk
        for fill in ("noise", "nan"):
            pert = G.gpu_pool(wl)
            pert.k_pages.copy_(pool.k_pages)
            pert.v_pages.copy_(pool.v_pages)
            n = hi - lo
            if fill == "nan":
                kk = torch.full((n, c.heads, c.head_dim), float("nan"), dtype=torch.bfloat16,
                                device=G.DEV)
                vv = kk.clone()
            else:
                kk = torch.randn(n, c.heads, c.head_dim, device=G.DEV).to(torch.bfloat16)
                vv = torch.randn(n, c.heads, c.head_dim, device=G.DEV).to(torch.bfloat16)
            wf.wf_kv_publish(pert, kk, vv, lo)
            out1, lse1 = G.attn(wl, pert, q)
            r0, r1 = qs[s], qs[s + 1]
            assert torch.equal(out1[r0:], out0[r0:]), (s, fill)
            assert torch.equal(lse1[:, r0:], lse0[:, r0:]), (s, fill)
            if fill == "noise":
                # slots below s do see the change (non-vacuity)
                assert not torch.equal(out1[:qs[s]], out0[:qs[s]])
    # non-vacuity: the prefix and each slot's own chunk matter
    for lo, n in ((0, 5), (c.store_start, 5)) + tuple((c.prefix + s * c.chunk, 5)
                                                       for s in range(c.slots)):
        pert = G.gpu_pool(wl)
        pert.k_pages.copy_(pool.k_pages)
        pert.v_pages.copy_(pool.v_pages)
        kk = torch.randn(n, c.heads, c.head_dim, device=G.DEV).to(torch.bfloat16)
        wf.wf_kv_publish(pert, kk, kk.clone(), lo)
        out1, _ = G.attn(wl, pert, q)
        s_max = c.slots if lo < c.prefix else (lo - c.prefix) // c.chunk + 1
        for s in range(s_max):
            assert not torch.equal(out1[qs[s]:qs[s + 1]], out0[qs[s]:qs[s + 1]]), (lo, s)


def test_page_permutation_bit_identical():
    wl = make_workload(cfg(page_size=64))
    c = wl.cfg
    pool, q, _ = G.gpu_layer(wl)
    out0, lse0 = G.attn(wl, pool, q)
    perm = torch.randperm(c.n_pages, generator=torch.Generator().manual_seed(9))
    k2 = torch.empty_like(pool.k_pages)
    v2 = torch.empty_like(pool.v_pages)
    k2[perm.to(G.DEV)] = pool.k_pages
    v2[perm.to(G.DEV)] = pool.v_pages
    table = perm[torch.from_numpy(wl.page_table).long()].to(torch.int32).to(G.DEV)
    out1, lse1 = G.attn(wl, wf.KVPool(k2, v2, table), q)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_nan_outside_visible_set_never_read():
    """The pool is NaN-filled before publishing and the stale pages hold
    N(0, 4): no output may be non-finite, and outputs equal those of a
    zero-filled pool bit for bit."""
    wl = make_workload(cfg(page_size=256, stale_frac=0.3))
    pool_nan, q, _ = G.gpu_layer(wl, fill="nan")
    pool_zero, _, _ = G.gpu_layer(wl, fill="zero")
    o1, l1 = G.attn(wl, pool_nan, q)
    o2, l2 = G.attn(wl, pool_zero, q)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_constant_v_gives_one():
    wl = make_workload(cfg(page_size=64))
    pool, q, _ = G.gpu_layer(wl)
    pool.v_pages.fill_(1.0)
    out, _ = G.attn(wl, pool, q)
    assert (out.float() - 1.0).abs().max().item() <= 4e-3


def test_deterministic():
    wl = make_workload(cfg(page_size=64))
    pool, q, _ = G.gpu_layer(wl)
    o1, l1 = G.attn(wl, pool, q)
    o2, l2 = G.attn(wl, pool, q)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("ps", [64, 256])
def test_repeatable_across_calls_and_grid_shapes(ps):
    """The same rows computed by differently shaped launches (all slots in
    one call, one slot per call) and by repeated calls agree bit for bit.
    A write-after-read race between waves on an LDS slot shows up here as a
    run-to-run or launch-to-launch difference."""
    wl = make_workload(cfg(page_size=ps, stale_frac=0.0, seed=43))
    c = wl.cfg
    pool, q, _ = G.gpu_layer(wl)
    ref, ref_lse = G.attn(wl, pool, q)
    qs = c.q_slot_start()
    for rep in range(4):
        out, lse = G.attn(wl, pool, q)
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), rep
        for s in range(c.slots):
            r0, r1 = qs[s], qs[s + 1]
            part, lse_p = G.attn(wl, pool, q[r0:r1].contiguous(), q_slot_start=[0, r1 - r0],
                                 first_slot=s)
            assert torch.equal(part, ref[r0:r1]), (rep, s)
            assert torch.equal(lse_p, ref_lse[:, r0:r1]), (rep, s)
