#!/usr/bin/env python3
"""Benchmark of the chunk-wise causal attention layer tick on one MI355X.

One step = one round of the hot path on one layer: wf_kv_publish of the live
store and the W slot chunks (3D RoPE on K + paged scatter of K and V), then
wf_chunk_attn of the W query chunks over the pool (anchor | history | store |
slots j >= s), back to back on one stream.  Inputs are synthetic and resident
in HBM before the timed region; the resident prefix (anchor + history) is
published once before timing.

    python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]
                    [--no-long-tick]

Prints one JSON line.  `value` is the unmasked attention TFLOP/s of the
whole step (publish included in the time); `roofline` describes the
attention kernel (MFMA-bound), measured with HIP events on the launch
stream; `cpu_baseline` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
METRIC = "chunk-causal attn TFLOP/s (unmasked) & % bf16 MFMA peak; layer tick ms"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-tick", action="store_true",
                    help="skip the long-context layer tick reported beside the headline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only plain device copies of a known size (for counter scaling)")
    return ap.parse_args()


def device_inputs(cfg, torch, wf):
    """Synthetic inputs of the configuration's shape, drawn on the device
    (same distributions as chunk_wise_causal_amd.workloads, other values)."""
    from chunk_wise_causal_amd.workloads import Config  # noqa: F401  (shape source)
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(1000 + cfg.seed)
    gc = torch.Generator().manual_seed(1000 + cfg.seed)
    H, D = cfg.heads, cfg.head_dim
    td = torch.bfloat16
    q = torch.randn(cfg.n_q, H, D, device=dev, generator=g).to(td)
    k = torch.randn(cfg.n_kv, H, D, device=dev, generator=g)
    n_hot = int(round(cfg.hot_frac * cfg.n_kv))
    if n_hot:
        k[torch.randperm(cfg.n_kv, generator=gc)[:n_hot].to(dev)] *= cfg.hot_factor
    k = k.to(td)
    v = torch.randn(cfg.n_kv, H, D, device=dev, generator=g).to(td)
    perm = torch.randperm(cfg.n_pages, generator=gc) if cfg.permute_pages else torch.arange(cfg.n_pages)
    table = perm[:cfg.n_logical_pages].to(torch.int32)
    pool = wf.KVPool.empty(cfg.n_pages, H, cfg.page_size, D, table, dtype=td, device=dev)
    pool.k_pages.normal_(0.0, 2.0, generator=g)     # stale contents
    pool.v_pages.normal_(0.0, 2.0, generator=g)
    pos = torch.from_numpy(cfg.positions()).to(dev)
    return q, k, v, pos, pool


def copy_calibration(torch):
    """Plain copies of exactly 1 GiB each: the bytes a FETCH_SIZE / WRITE_SIZE
    counter reports for them give the scale from counter units to bytes."""
    n = 1 << 29                      # 2^29 bf16 = 1 GiB
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "copies": 3}))


def traffic_from_profiles(kernel_src_hash: str):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_bf16_14b_4step_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("attn_bf16.hip", "attn_core.h", "wf_internal.h"):
        with open(os.path.join(ROOT, "chunk_wise_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


_ORACLE = {}    # the sample's oracle inputs, set before the worker pool forks


def _oracle_worker_init():
    """One BLAS thread per worker: the pool supplies the parallelism."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_item(item):
    """Attention of one (head, slot, row block) of the sample with the CPU
    oracle as it stands; returns the item and its unmasked flops."""
    from oracle.attention import chunk_attention
    h, g, r0, r1, flops = item
    d = _ORACLE
    chunk_attention(d["k"], d["v"], d["table"], d["ps"], d["segs"], d["q"][r0:r1], [0, r1 - r0],
                    d["first"] + g, d["scale"], d["dtype"], heads=[h])
    return flops


def cpu_cores() -> tuple:
    """(workers, affinity): the CPUs this process may run on, capped by the
    thread share the environment declares (OMP_NUM_THREADS), if any."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    cap = int(env) if env.isdigit() and int(env) > 0 else aff
    return max(1, min(aff, cap)), aff


def cpu_baseline(cfg, seconds: float):
    """Time the CPU oracle (as it stands) on a bounded sample of the same
    workload, on the host's cores: a process pool (one BLAS thread per
    worker) over (head, slot, 1024-row block) items of a copy of the
    configuration with at most 8 heads, head by head, until `seconds` have
    passed; plus the oracle publish of the copy.  Both are scaled to one full
    step.  Runs before the process touches the GPU (the pool forks)."""
    import dataclasses
    import multiprocessing
    from chunk_wise_causal_amd.workloads import make_workload
    from tests._pipeline import oracle_layer  # test glue: oracle-only pipeline
    workers, aff = cpu_cores()
    small = dataclasses.replace(cfg, heads=min(cfg.heads, 8))
    wl = make_workload(small)
    t0 = time.perf_counter()
    ref = oracle_layer(wl)
    t_pub_all = time.perf_counter() - t0
    c = wl.cfg
    qss = c.q_slot_start()
    vis = [c.visible(g) for g in range(c.slots)]
    items = [(h, g, r0, min(qss[g + 1], r0 + 1024),
              4 * c.head_dim * (min(qss[g + 1], r0 + 1024) - r0) * vis[g])
             for h in range(c.heads) for g in range(c.slots) for r0 in range(qss[g], qss[g + 1], 1024)]
    _ORACLE.update(k=ref["k_pool"], v=ref["v_pool"], table=wl.page_table, ps=c.page_size,
                   segs=c.segments(), q=ref["q"], first=0, scale=c.scale, dtype=c.dtype)
    done_flops, done_items = 0, 0
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers, initializer=_oracle_worker_init) as pool:
        t0 = time.perf_counter()
        pending, nxt = [], 0
        while nxt < len(items) or pending:
            # keep every worker busy until the budget is spent, then drain
            while nxt < len(items) and len(pending) < 2 * workers and \
                    time.perf_counter() - t0 < seconds:
                pending.append(pool.apply_async(_oracle_item, (items[nxt],)))
                nxt += 1
            if not pending:
                break
            done_flops += pending.pop(0).get()
            done_items += 1
        t_attn = time.perf_counter() - t0
    rate = done_flops / t_attn                           # unmasked flop/s of the oracle
    attn_full = cfg.unmasked_flops() / rate
    # publish: the oracle published all n_kv tokens of the copy's heads
    pub_full = t_pub_all * (cfg.tick_tokens / c.n_kv) * (cfg.heads / c.heads)
    step = attn_full + pub_full
    return {
        "value": cfg.unmasked_flops() / step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on {workers} worker processes (one BLAS thread each; "
                   f"{aff} CPUs in the affinity set): attention of {done_items} (head, slot, "
                   f"1024-row block) items of a {c.heads}-head copy of the workload "
                   f"({done_flops:.3e} unmasked flops in {t_attn:.1f} s), publish of {c.n_kv} "
                   f"tokens x {c.heads} heads ({t_pub_all:.1f} s, one process), scaled by flops "
                   f"and bytes to one full step ({step:.0f} s)"),
        "affinity_cpus": int(aff),
        "step_s_extrapolated": step,
    }


def time_mx_variant(cfg, torch, wf, q, k, v, pos, pool, out, steps: int):
    """The 8-bit QK^T variant on the same inputs: wf_kv_publish_mx of the
    round, then wf_chunk_attn_mx, timed per step with HIP events on the
    launch stream.  TFLOP/s count the same unmasked FLOPs; half of them (QK^T)
    run at the FP8 rate, so the matching peak is 2 / (1/5000 + 1/2500)
    TFLOP/s."""
    keys = wf.MXKeys.empty(cfg.n_pages, cfg.heads, cfg.page_size, cfg.head_dim)
    rope = (cfg.rope, cfg.theta)
    ss = cfg.store_start
    stream = torch.cuda.current_stream()
    wf.wf_kv_publish_mx(pool, keys, k[:ss], v[:ss], 0, pos=pos[:ss], rope=rope, stream=stream)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        wf.wf_kv_publish_mx(pool, keys, k[ss:], v[ss:], ss, pos=pos[ss:], rope=rope,
                            stream=stream)
        if ev:
            ev[1].record(stream)
        wf.wf_chunk_attn_mx(pool, keys, cfg.segments(), q, cfg.q_slot_start(), 0, cfg.scale,
                            out=out, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    pub = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    att = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    tf = cfg.unmasked_flops() / (att * 1e-3) / 1e12
    mixed_peak = 2.0 / (1.0 / 5000.0 + 1.0 / PEAK_BF16_TFLOPS)
    return {"attn_ms_p50": round(att, 4), "attn_tflops": round(tf, 2),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "frac_fp8_bf16_peak": round(tf / mixed_peak, 4), "fp8_bf16_peak": round(mixed_peak, 1),
            "publish_ms_p50": round(pub, 4),
            "kernel": "attn_fwd_mx<128, true>",
            "format": "MXFP8 (E4M3, E8M0 per 32 features) Q and K; bf16 P V"}


def time_qkv_publish(cfg, torch, wf, pos, steps: int):
    """The QKV projection of the round's tokens (hidden = heads x head_dim)
    with the publish fused into its epilogue (wf_qkv_publish), against the
    unfused order: the same projection by torch's GEMM, then wf_kv_publish.
    Synthetic bf16 hidden states and weights drawn on the device."""
    H, D = cfg.heads, cfg.head_dim
    hid, n, ss = H * D, cfg.tick_tokens, cfg.store_start
    g = torch.Generator(device="cuda").manual_seed(cfg.seed + 7)
    x = torch.randn(n, hid, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * hid, hid, device="cuda", generator=g) / hid ** 0.5).to(torch.bfloat16)
    b = (torch.randn(3 * hid, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    table = torch.randperm(cfg.n_logical_pages, device="cuda", generator=g).to(torch.int32)
    qpool = wf.KVPool.empty(cfg.n_logical_pages, H, cfg.page_size, D, table)
    q_out = torch.empty(n, H, D, dtype=torch.bfloat16, device="cuda")
    rope = (cfg.rope, cfg.theta)
    p = pos[ss:]
    stream = torch.cuda.current_stream()

    def fused():
        wf.wf_qkv_publish(qpool, x, w, ss, pos=p, rope=rope, bias=b, q_out=q_out, stream=stream)

    def unfused():
        # Q rotated in place inside the projection's output (both calls take
        # a row stride, so no copy is needed on either side)
        qkv = torch.nn.functional.linear(x, w, b).view(n, 3, H, D)
        wf.wf_kv_publish(qpool, qkv[:, 1], qkv[:, 2], ss, pos=p, rope=rope, q=qkv[:, 0],
                         stream=stream)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    f_ms, u_ms = timed(fused), timed(unfused)
    assert wf.wf_device_status() == 0
    flops = 2.0 * n * hid * 3 * hid
    tf = flops / (f_ms * 1e-3) / 1e12
    return {"tokens": n, "hidden": hid, "fused_ms_p50": round(f_ms, 4),
            "fused_tflops": round(tf, 2), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "unfused_ms_p50": round(u_ms, 4), "kernel": "qkv_gemm_publish",
            "unfused": "torch linear (library GEMM) + wf_kv_publish"}


def time_publish_flushed(cfg, torch, wf, pool, k_t, v_t, pos_t, steps: int):
    """The round's publish alone with the caches flushed before every launch
    (a 512 MB device buffer is overwritten, more than the 4 MB L2 of each XCD
    and the 256 MB MALL), so its reads and writes go to HBM: HIP events on
    the launch stream around the publish only."""
    stream = torch.cuda.current_stream()
    rope = (cfg.rope, cfg.theta)
    flush = torch.empty(256 << 20, dtype=torch.bfloat16, device="cuda")
    ms = []
    for i in range(steps + 2):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        wf.wf_kv_publish(pool, k_t, v_t, cfg.store_start, pos=pos_t, rope=rope, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    del flush
    med = float(np.median(ms))
    gbps = cfg.publish_bytes() / (med * 1e-3) / 1e9
    return {"ms_p50": round(med, 4), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "flush": "512 MB device buffer overwritten before each launch"}


def copy_ceiling(torch, nbytes: int, steps: int):
    """A measured HBM ceiling beside the spec peak: a plain device copy
    (torch copy_) that reads and writes the publish's byte count (half read,
    half written), HIP events around each copy, median."""
    n = nbytes // 4
    a = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(steps + 3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    med = float(np.median(ms))
    return round(4 * n / (med * 1e-3) / 1e9, 1)


def time_layer_tick(cfg, torch, wf, steps: int, warmup: int):
    """One layer tick of another configuration, timed like the headline:
    the round's publish then the attention on one stream, HIP events around
    each, inputs resident in HBM.  Its buffers are freed afterwards."""
    q, k, v, pos, pool = device_inputs(cfg, torch, wf)
    out = torch.empty_like(q)
    ss, rope = cfg.store_start, (cfg.rope, cfg.theta)
    wf.wf_kv_publish(pool, k[:ss], v[:ss], 0, pos=pos[:ss], rope=rope)
    stream = torch.cuda.current_stream()
    segs, qss = cfg.segments(), cfg.q_slot_start()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        wf.wf_kv_publish(pool, k[ss:], v[ss:], ss, pos=pos[ss:], rope=rope, stream=stream)
        if ev:
            ev[1].record(stream)
        wf.wf_chunk_attn(pool, segs, q, qss, 0, cfg.scale, out=out, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    pub = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    att = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    tick = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    tf = cfg.unmasked_flops() / (att * 1e-3) / 1e12
    gbps = cfg.publish_bytes() / (pub * 1e-3) / 1e9
    del q, k, v, pos, pool, out
    torch.cuda.empty_cache()
    return {"workload": f"layer tick: {cfg.name}", "n_q": cfg.n_q, "n_kv": cfg.n_kv,
            "unmasked_flops": cfg.unmasked_flops(), "steps": steps,
            "tick_ms_p50": round(tick, 4), "attn_ms_p50": round(att, 4),
            "attn_tflops": round(tf, 2), "attn_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "publish_ms_p50": round(pub, 4), "publish_GBps": round(gbps, 1),
            "publish_frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def time_history_rotate(cfg, torch, wf, reps: int = 200):
    """End-of-round history rotation (wf_history_rotate) on the page-aligned
    placement of the same context: average launch duration over `reps`
    rotations, HIP events on the launch stream."""
    from chunk_wise_causal_amd.workloads import AlignedLayout
    lay = AlignedLayout(cfg)
    table = torch.randperm(lay.n_logical_pages, dtype=torch.int32, device="cuda")
    pool = wf.KVPool(torch.empty(1, 1, cfg.page_size, cfg.head_dim, dtype=torch.bfloat16,
                                 device="cuda"),
                     torch.empty(1, 1, cfg.head_dim, cfg.page_size, dtype=torch.bfloat16,
                                 device="cuda"), table)
    stream = torch.cuda.current_stream()
    for _ in range(10):
        wf.wf_history_rotate(pool, lay.window_start, lay.chunk_stride, lay.window_chunks,
                             stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        wf.wf_history_rotate(pool, lay.window_start, lay.chunk_stride, lay.window_chunks,
                             stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    window = lay.window_chunks * lay.chunk_stride // cfg.page_size
    return {"us_per_rotation": round(e0.elapsed_time(e1) * 1e3 / reps, 3),
            "window_pages": window, "table_pages": lay.n_logical_pages,
            "chunk_pages": lay.chunk_stride // cfg.page_size,
            "layout": "page-aligned placement of the same context"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from chunk_wise_causal_amd.workloads import CONFIGS
    cfg = CONFIGS[args.config]
    # the oracle's worker pool forks: run it before the process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, args.cpu_seconds)
    from chunk_wise_causal_amd import wf
    wf.lib()
    q, k, v, pos, pool = device_inputs(cfg, torch, wf)
    out = torch.empty_like(q)
    segs = cfg.segments()
    qss = cfg.q_slot_start()
    ss = cfg.store_start
    rope = (cfg.rope, cfg.theta)
    # resident prefix (anchor + history), published once before the round
    wf.wf_kv_publish(pool, k[:ss], v[:ss], 0, pos=pos[:ss], rope=rope)
    k_t, v_t, pos_t = k[ss:], v[ss:], pos[ss:]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        wf.wf_kv_publish(pool, k_t, v_t, ss, pos=pos_t, rope=rope, stream=stream)
        if ev:
            ev[1].record(stream)
        wf.wf_chunk_attn(pool, segs, q, qss, 0, cfg.scale, out=out, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pub_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    tick_ms = [e[0].elapsed_time(e[2]) for e in evs]
    assert wf.wf_device_status() == 0
    ms_step = wall * 1e3 / args.steps
    flops = cfg.unmasked_flops()
    attn_avg = float(np.mean(attn_ms))
    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    pub_bytes = cfg.publish_bytes()
    pub_avg = float(np.mean(pub_ms))
    pub_gbps = pub_bytes / (pub_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q/K/V ~ N(0,1) bf16 drawn on device, seeded; random-permuted pages",
        "config": {"workload": f"layer tick: {cfg.name}",
                   "heads": cfg.heads, "head_dim": cfg.head_dim, "chunk": cfg.chunk,
                   "anchor": cfg.anchor_tokens, "history_chunks": cfg.n_hist,
                   "slots": cfg.slots, "n_q": cfg.n_q, "n_kv": cfg.n_kv,
                   "page_size": cfg.page_size, "unmasked_flops": flops,
                   "publish_tokens": cfg.tick_tokens, "publish_bytes": pub_bytes},
        "tick_ms_p50": round(float(np.median(tick_ms)), 4),
        "attn_ms_p50": round(float(np.median(attn_ms)), 4),
        "attn_ms_p10_p90": [round(float(np.percentile(attn_ms, 10)), 4),
                            round(float(np.percentile(attn_ms, 90)), 4)],
        "attn_tflops": round(attn_tflops, 2),
        "publish_ms_p50": round(float(np.median(pub_ms)), 4),
        "publish_GBps": round(pub_gbps, 1),
        "publish_frac_hbm_peak": round(pub_gbps / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profiles(kernel_source_hash()),
                     "kernel": "attn_fwd_bf16<128, true>"},
        "cpu_baseline": None,
    }
    res["publish_flushed"] = time_publish_flushed(cfg, torch, wf, pool, k_t, v_t, pos_t,
                                                  args.steps)
    copy_gbps = copy_ceiling(torch, pub_bytes, args.steps)
    res["measured_ceilings"] = {
        "copy_GBps": copy_gbps, "copy_frac_hbm_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
        "publish_over_copy": round(pub_gbps / copy_gbps, 4),
        "copy": "device copy (torch copy_) reading and writing the publish's byte count"}
    res["history_rotate"] = time_history_rotate(cfg, torch, wf)
    res["mx_variant"] = time_mx_variant(cfg, torch, wf, q, k, v, pos, pool, out, args.steps)
    res["qkv_publish"] = time_qkv_publish(cfg, torch, wf, pos, args.steps)
    if args.config == 4 and not args.no_long_tick:
        # the long-context layer tick (14B-like, chunk 10800, W=5) beside the
        # headline: fewer steps, each about 85 ms
        del q, k, v, pos, pool, out, k_t, v_t, pos_t
        torch.cuda.empty_cache()
        res["long_context_tick"] = time_layer_tick(CONFIGS[5], torch, wf,
                                                   steps=max(3, args.steps // 2), warmup=2)
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
