"""The five layer shapes at full size, in the launch configuration the
benchmark times (one wf_kv_publish for the resident prefix, one for the
round's store + slots, one wf_chunk_attn over all slots).

publish: the whole pool bit-exact against the oracle.  attention: every
output element of one whole head (all rows of every slot), and of sampled
query rows (first and last rows of every slot, which sit in its first and
ragged last query tile, plus random rows) for sampled heads, against the
float64 oracle; plus properties at full size (finite outputs, LSE
agreement).  The figures of every configuration are appended to the parity
record (tests/_gpu.py: record).
"""
import time

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
    # one whole head, every row of every slot
    hf = int(rng.integers(0, cfg.heads))
    print(f"[full] oracle attention, head {hf}, all {cfg.n_q} rows", flush=True)
    t0 = time.perf_counter()
    o_h, l_h = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, cfg.page_size,
                               cfg.segments(), ref["q"], cfg.q_slot_start(), 0, cfg.scale,
                               cfg.dtype, heads=[hf])
    t_head = time.perf_counter() - t0
    got_h = out[:, hf].float().cpu().numpy().astype(np.float64)
    mx_h, rr_h = G.err_stats(got_h, o_h[:, hf])
    lse_h = float(np.abs(G.to_f64(lse)[hf] - l_h[hf]).max())
    print(f"[full] cfg{idx} head {hf}: max-abs {mx_h:.3e} rel-rms {rr_h:.3e} "
          f"lse {lse_h:.2e} ({t_head:.1f} s)", flush=True)
    print(f"[full] oracle attention on {sum(len(r) for r in rows.values())} rows x "
          f"{len(heads)} heads", flush=True)
    o_ref, l_ref = chunk_attention(ref["k_pool"], ref["v_pool"], wl.page_table, cfg.page_size,
                                   cfg.segments(), ref["q"], cfg.q_slot_start(), 0, cfg.scale,
                                   cfg.dtype, heads=heads, rows=rows)
    sel = np.concatenate(list(rows.values()))
    got = out[torch.from_numpy(sel).to(G.DEV)][:, heads].float().cpu().numpy().astype(np.float64)
    ref_o = o_ref[sel][:, heads]
    mx, rr = G.err_stats(got, ref_o)
    lse_s = float(np.abs(G.to_f64(lse)[heads][:, sel] - l_ref[heads][:, sel]).max())
    print(f"[full] cfg{idx} sampled: max-abs {mx:.3e} rel-rms {rr:.3e}", flush=True)
    G.record("full_size_attention", config=idx, workload=cfg.name,
             whole_head=dict(head=hf, rows=cfg.n_q, max_abs=mx_h, rel_rms=rr_h, lse_max=lse_h,
                             oracle_s=round(t_head, 2)),
             sampled=dict(heads=heads, rows=int(len(sel)), max_abs=mx, rel_rms=rr,
                          lse_max=lse_s),
             bars=dict(max_abs=G.MAX_ABS, rel_rms=G.REL_RMS, lse=G.lse_atol(cfg.dtype)),
             publish="bit-exact over the whole pool")
    assert mx_h <= G.MAX_ABS and rr_h <= G.REL_RMS
    assert mx <= G.MAX_ABS and rr <= G.REL_RMS
    assert lse_h <= G.lse_atol(cfg.dtype) and lse_s <= G.lse_atol(cfg.dtype)
