"""The five layer shapes at full size, in the launch configuration the
benchmark times (one wf_kv_publish for the resident prefix, one for the
round's store + slots, one wf_chunk_attn over all slots).

publish: the whole pool bit-exact against the oracle.  attention: every
output element of sampled query rows (first and last rows of every slot,
which sit in its first and ragged last query tile, plus random rows) for
sampled heads, against the float64 oracle computed row by row; plus
properties at full size (finite outputs, LSE agreement).
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from chunk_wise_causal_amd.workloads import CONFIGS, make_workload
from oracle.attention import chunk_attention
from tests import _gpu as G
from tests._pipeline import oracle_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


def _sample(cfg, rng):
    qs = cfg.q_slot_start()
    rows = {}
    for g in range(cfg.slots):
        r0, r1 = qs[g], qs[g + 1]
        pick = set(range(r0, min(r1, r0 + 4))) | set(range(max(r0, r1 - 4), r1))
        pick |= set(rng.integers(r0, r1, size=8).tolist())
        rows[g] = np.array(sorted(pick))
    H = cfg.heads
    heads = sorted(set([0, 1, H // 2, H - 1] + rng.integers(0, H, size=2).tolist()))
    return rows, heads


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_full_size_config(idx):
    cfg = CONFIGS[idx]
    print(f"\n[full] cfg{idx}: {cfg.name}", flush=True)
    wl = make_workload(cfg)
    pool, q, _ = G.gpu_layer(wl)
    out, lse = G.attn(wl, pool, q)
    assert wf.wf_device_status() == 0
    print("[full] gpu done; oracle publish", flush=True)
    ref = oracle_layer(wl)
    assert np.array_equal(G.bits(G.to_storage(pool.k_pages)), G.bits(ref["k_pool"]))
    assert np.array_equal(G.bits(G.to_storage(pool.v_pages)), G.bits(ref["v_pool"]))
    del pool
    assert torch.isfinite(out.float()).all().item()
    rng = np.random.default_rng(idx)
    rows, heads = _sample(cfg, rng)
    print(f"[full] oracle attention on {sum(len(r) for r in rows.values())} rows x "
          f"{len(heads)} heads", flush=True)
    o_ref, l_ref = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, cfg.page_size,
                                   cfg.segments(), ref["q"], cfg.q_slot_start(), 0, cfg.scale,
                                   cfg.dtype, heads=heads, rows=rows)
    sel = np.concatenate(list(rows.values()))
    got = out[torch.from_numpy(sel).to(G.DEV)][:, heads].float().cpu().numpy().astype(np.float64)
    ref_o = o_ref[sel][:, heads]
    mx, rr = G.err_stats(got, ref_o)
    print(f"[full] cfg{idx} max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    np.testing.assert_allclose(G.to_f64(lse)[heads][:, sel], l_ref[heads][:, sel],
                               rtol=0, atol=G.lse_atol(cfg.dtype))
