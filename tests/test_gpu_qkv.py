"""GPU parity of wf_qkv_publish (the QKV projection with the publish fused
into its epilogue) against the CPU oracle (oracle/qkv.py), through the C ABI.

The projection accumulates in float32 in the kernel's own order, so a value
lying within float32 rounding of a bfloat16 rounding boundary can round to
the other neighbour than the float64 oracle's single rounding; the rotation
carries such a one-unit difference into at most two units.  The bar: every
element of the pools and of Q within 2 bfloat16 units in the last place of
the oracle, plus the float32 accumulation error bound of the projection
(hidden * 2^-24 * sum |x w|, which dominates for outputs near zero), plus,
for rotated features, 2^-7 of the rotated pair's norm (a one-unit input
change moves a rotation output by up to 2^-8 of it); untouched pool bytes
identical; at least 99 % of all elements bit-identical.  Shapes: ragged token tiles, unaligned publish windows,
page sizes 16 / 64 / 256, with and without bias, Q output and RoPE; the
14B-like projection (hidden 5120, 40 heads) on a full chunk with sampled
tokens.
"""
import numpy as np
import pytest
import torch

from chunk_wise_causal_amd import wf
from oracle.numerics import bf16_to_f32
from oracle.publish import publish
from oracle.qkv import qkv_project, qkv_publish
from tests import _gpu as G
from tests._pipeline import NAN_BF16, storage

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wf.lib()


def close_bf16(got: np.ndarray, ref: np.ndarray, rotated: bool = False, acc_err=None):
    """(all within the bound, fraction bit-identical).  Bound: 2 units in
    the last place of the element, plus the float32 accumulation error bound
    acc_err of the projection (for rotated features, that of both elements
    of the pair); for rotated features (pairs along the last axis) also 2^-7
    of the pair's norm, since a one-unit change of a rotation input moves
    both outputs by up to 2^-8 of the norm, which can be many units of an
    output near zero."""
    g = bf16_to_f32(got).astype(np.float64)
    r = bf16_to_f32(ref).astype(np.float64)
    same = got == ref
    nan_ok = np.isnan(g) == np.isnan(r)
    mag = np.maximum(np.abs(g), np.abs(r))
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    bound = 2 * np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    if rotated:
        rr = np.nan_to_num(r)
        pn = np.sqrt(rr[..., 0::2] ** 2 + rr[..., 1::2] ** 2)
        bound = bound + 2.0 ** -7 * np.repeat(pn, 2, axis=-1)
    if acc_err is not None:
        a = np.nan_to_num(acc_err)
        if rotated:
            a = np.repeat(a[..., 0::2] + a[..., 1::2], 2, axis=-1)
        bound = bound + a
    within = same | (np.abs(g - r) <= bound)
    valid = ~np.isnan(r)
    if not within[valid].all():
        i = np.argwhere(~within & valid)[0]
        print("[qkv] worst", tuple(i), g[tuple(i)], r[tuple(i)], flush=True)
    return bool(nan_ok.all() and within[valid].all()), float(same.mean())


def acc_bound(x, w, b, H):
    """float32 accumulation error bound of the projection, per token and
    feature: hidden * 2^-24 * (sum_k |x_k w_k| + |b|), as (q, k, v) [n, H, D]."""
    ax = np.abs(bf16_to_f32(storage(x, "bf16")).astype(np.float64))
    aw = np.abs(bf16_to_f32(storage(w, "bf16")).astype(np.float64))
    a = ax @ aw.T
    if b is not None:
        a = a + np.abs(bf16_to_f32(storage(b, "bf16")).astype(np.float64))[None, :]
    a = a * x.shape[1] * 2.0 ** -24
    n, hd = x.shape[0], H * 128
    return tuple(a[:, i * hd:(i + 1) * hd].reshape(n, H, 128) for i in range(3))


CASES = {
    # H, hidden, n_tok, ps, dst, bias, q_out, rope
    "ps16_ragged_bias_q": (2, 256, 200, 16, 37, True, True, True),
    "ps64_plain": (2, 192, 130, 64, 64, False, False, False),
    "ps256_h3": (3, 384, 700, 256, 1000, True, True, True),
    "ps64_one_tile_no_q": (1, 64, 17, 64, 5, True, False, True),
    "ps32_wide_positions": (2, 128, 300, 32, 64, True, True, "wide"),
    "ps16_denormal_outputs": (1, 64, 80, 16, 0, False, True, "denormal"),
    # bias at an address 2 bytes past an 8-byte boundary: the kernel's
    # element-wise bias path
    "ps64_h3_bias_unaligned": (3, 256, 300, 64, 0, "unaligned", True, True),
}


def draw(H, hidden, n, seed, wide=False):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, hidden, generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * H * 128, hidden, generator=g) / hidden ** 0.5).to(torch.bfloat16)
    b = (torch.randn(3 * H * 128, generator=g) * 0.1).to(torch.bfloat16)
    if wide == "denormal":
        # every output is one hidden state times 1 + 2^-7: x is a bfloat16
        # denormal m * 2^-133, so the float32 product m (1 + 2^-7) 2^-133 is
        # exact and its rounding to bfloat16 happens in the denormal range
        # (m = 64 is a tie); the rotation then multiplies denormals
        m = torch.randint(1, 128, (n, hidden), generator=g).to(torch.float64)
        x = (m * 2.0 ** -133).to(torch.bfloat16)
        w = torch.zeros(3 * H * 128, hidden, dtype=torch.float64)
        w[torch.arange(3 * H * 128), torch.arange(3 * H * 128) % hidden] = 1 + 2.0 ** -7
        w = w.to(torch.bfloat16)
    if wide == "wide":
        # positions spread over +-50000 per axis: far more (pair, position)
        # combinations per 256-token block than the kernel's factor table holds
        pos = torch.randint(-50000, 50000, (n, 3), generator=g).to(torch.int32)
    else:
        pos = torch.stack([torch.arange(n) // 40, torch.arange(n) % 40 // 8, torch.arange(n) % 8],
                          1).to(torch.int32)
    return x, w, b, pos


@pytest.mark.parametrize("name", list(CASES))
def test_qkv_publish_parity(name):
    H, hidden, n, ps, dst, use_bias, use_q, use_rope = CASES[name]
    print(f"\n[qkv] {name}", flush=True)
    wide = use_rope if isinstance(use_rope, str) else False
    x, w, b, pos = draw(H, hidden, n, seed=sum(map(ord, name)), wide=wide)
    n_log = (dst + n + ps - 1) // ps + 1
    rng = np.random.default_rng(7)
    table = rng.permutation(n_log + 2)[:n_log].astype(np.int32)
    n_pages = n_log + 2
    rope = ((44, 42, 42), 1e4) if use_rope else None
    # oracle
    kp = np.full((n_pages, H, ps, 128), NAN_BF16, np.uint16)
    vp = np.full((n_pages, H, 128, ps), NAN_BF16, np.uint16)
    q_ref = qkv_publish(kp, vp, table, ps, storage(x, "bf16"), storage(w, "bf16"), H, 128,
                        pos.numpy(), dst, rope, bias=storage(b, "bf16") if use_bias else None)
    # GPU
    pool = wf.KVPool.empty(n_pages, H, ps, 128, torch.from_numpy(table), device=G.DEV)
    pool.k_pages.view(torch.int16).fill_(int(NAN_BF16))     # 0x7FC1: the oracle's NaN fill
    pool.v_pages.view(torch.int16).fill_(int(NAN_BF16))
    q_out = torch.full((n, H, 128), float("nan"), dtype=torch.bfloat16, device=G.DEV) if use_q else None
    bias = None
    if use_bias == "unaligned":
        store = torch.empty(b.numel() + 1, dtype=torch.bfloat16, device=G.DEV)
        store[1:] = b.to(G.DEV)
        bias = store[1:]
        assert bias.data_ptr() % 8 == 2
    elif use_bias:
        bias = b.to(G.DEV)
    wf.wf_qkv_publish(pool, x.to(G.DEV), w.to(G.DEV), dst, pos=pos.to(G.DEV) if use_rope else None,
                      rope=rope, bias=bias, q_out=q_out)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    kg, vg = G.to_storage(pool.k_pages), G.to_storage(pool.v_pages)
    # every byte outside the published rows keeps the fill, on both sides
    toks = np.arange(dst, dst + n)
    pages, rows = table[toks // ps], toks % ps
    mk = np.ones(kp.shape, bool); mk[pages, :, rows, :] = False
    mv = np.ones(vp.shape, bool); mv[pages, :, :, rows] = False
    assert np.array_equal(kg[mk], kp[mk]) and np.array_equal(vg[mv], vp[mv])
    ea_q, ea_k, ea_v = acc_bound(x, w, b if use_bias else None, H)
    checks = [("k", kg[pages, :, rows, :], kp[pages, :, rows, :], ea_k),
              ("v", vg[pages, :, :, rows], vp[pages, :, :, rows], ea_v)]
    if use_q:
        checks.append(("q", G.to_storage(q_out), q_ref, ea_q))
    for what, got, ref, ea in checks:
        ok, frac = close_bf16(got, ref, rotated=use_rope and what != "v", acc_err=ea)
        print(f"[qkv] {name} {what}: bit-identical {frac:.5f}", flush=True)
        assert ok and frac >= 0.99, (what, frac)


@pytest.mark.timeout(600)
def test_qkv_publish_14b_chunk_sampled():
    """hidden 5120, 40 heads, one 4680-token chunk on 256-token pages at an
    unaligned start; tokens sampled for the oracle."""
    H, hidden, n, ps, dst = 40, 5120, 4680, 256, 10920
    x, w, b, pos = draw(H, hidden, n, seed=5)
    n_log = (dst + n + ps - 1) // ps
    table = np.random.default_rng(8).permutation(n_log).astype(np.int32)
    pool = wf.KVPool.empty(n_log, H, ps, 128, torch.from_numpy(table), device=G.DEV)
    q_out = torch.empty((n, H, 128), dtype=torch.bfloat16, device=G.DEV)
    rope = ((44, 42, 42), 1e4)
    wf.wf_qkv_publish(pool, x.to(G.DEV), w.to(G.DEV), dst, pos=pos.to(G.DEV), rope=rope,
                      bias=b.to(G.DEV), q_out=q_out)
    torch.cuda.synchronize()
    assert wf.wf_device_status() == 0
    rng = np.random.default_rng(9)
    sel = np.unique(np.concatenate([[0, 1, 127, 128, n - 1], rng.integers(0, n, 40)]))
    xs, ws, bs = storage(x, "bf16"), storage(w, "bf16"), storage(b, "bf16")
    q, k, v = qkv_project(xs[sel], ws, H, 128, bias=bs)
    ea_q, ea_k, ea_v = acc_bound(x[torch.from_numpy(sel)], w, b, H)
    kp_g, vp_g = G.to_storage(pool.k_pages), G.to_storage(pool.v_pages)
    q_g = G.to_storage(q_out)
    fracs = []
    for i, t in enumerate(sel):
        kp = np.zeros((n_log, H, ps, 128), np.uint16)
        vp = np.zeros((n_log, H, 128, ps), np.uint16)
        k_rot, q_rot = publish(kp, vp, table, ps, k[i:i + 1], v[i:i + 1], pos.numpy()[t:t + 1],
                               dst + int(t), "bf16", rope=rope, q=q[i:i + 1])
        L = dst + int(t)
        page, row = table[L // ps], L % ps
        for got, ref, rot, ea in ((kp_g[page, :, row, :], k_rot[0], True, ea_k[i]),
                                  (vp_g[page, :, :, row], v[i], False, ea_v[i]),
                                  (q_g[t], q_rot[0], True, ea_q[i])):
            ok, frac = close_bf16(got, ref, rotated=rot, acc_err=ea)
            assert ok, t
            fracs.append(frac)
    print(f"[qkv] 14B-like chunk: bit-identical {np.mean(fracs):.5f} over {len(sel)} tokens",
          flush=True)
    assert np.mean(fracs) >= 0.99
