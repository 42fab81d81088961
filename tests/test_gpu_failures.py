"""Device data the host cannot check: page-table entries outside the pool.

Every kernel that reads the page table bounds-checks each entry and never
touches memory through a bad one.  Publish skips the rows, attention reads
zeros for the tile, and the QKV publish skips the tokens. Each raises
WF_STATUS_BAD_PAGE in the device status word.  The condition is set up from
the host, with tables that name pages past the end of the pool or
negative ones.  Every kernel still runs to completion.  Afterwards the same
calls on a good table are exact again and leave the status clear.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import make_workload, small_config
from oracle.attention import chunk_attention
from tests import _gpu as G
from tests._pipeline import oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()
    wf.wf_device_status(clear=True)


@pytest.mark.parametrize("ps", [16, 64])
def test_bad_entries_raise_status_and_read_nothing(ps):
    cfg = small_config(page_size=ps, seed=61)
    wl = make_workload(cfg)
    c = wl.cfg
    print(f"\n[bad-page] ps={ps}", flush=True)
    good = torch.from_numpy(wl.page_table.copy())
    bad = good.clone()
    bad[1] = c.n_pages + 5          # past the end of the pool
    bad[-2] = -3                    # negative
    k, v = wl.k.to(G.DEV), wl.v.to(G.DEV)
    pos = torch.from_numpy(wl.pos).to(G.DEV)
    rope = (c.rope, c.theta)
    q = wl.q.to(G.DEV)
    H, D = c.heads, c.head_dim

    def run(table):
        pool = wf.KVPool.empty(c.n_pages, H, ps, D, table, device=G.DEV, fill=0.0)
        keys = wf.MXKeys.empty(c.n_pages, H, ps, D)
        keys.codes.zero_()
        keys.scales.zero_()
        wf.wf_kv_publish(pool, k, v, 0, pos=pos, rope=rope)
        st_pub = wf.wf_device_status(clear=True)
        out = wf.wf_chunk_attn(pool, c.segments(), q, c.q_slot_start(), 0, c.scale)
        st_att = wf.wf_device_status(clear=True)
        wf.wf_kv_publish_mx(pool, keys, k, v, 0, pos=pos, rope=rope)
        st_pub_mx = wf.wf_device_status(clear=True)
        out_mx = wf.wf_chunk_attn_mx(pool, keys, c.segments(), q, c.q_slot_start(), 0, c.scale)
        st_att_mx = wf.wf_device_status(clear=True)
        hid = 128
        g = torch.Generator().manual_seed(5)
        x = torch.randn(c.n_kv, hid, generator=g).to(torch.bfloat16).to(G.DEV)
        w = (torch.randn(3 * H * D, hid, generator=g) / 16).to(torch.bfloat16).to(G.DEV)
        wf.wf_qkv_publish(pool, x, w, 0, pos=pos, rope=rope)
        st_qkv = wf.wf_device_status(clear=True)
        return (st_pub, st_att, st_pub_mx, st_att_mx, st_qkv), out, pool

    sts, _, _ = run(bad)
    assert sts == (wf.WF_STATUS_BAD_PAGE,) * 5, sts
    sts, out, _ = run(good)
    assert sts == (0,) * 5, sts
    ref = oracle_layer(wl, fill="zero")
    o_ref, _ = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, ps, c.segments(),
                               ref["q"], c.q_slot_start(), 0, c.scale, c.dtype)
    mx, rr = G.err_stats(G.to_f64(out), o_ref)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
