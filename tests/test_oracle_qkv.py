"""Pins for the fused QKV-projection publish oracle (oracle/qkv.py).

The single rounding float64 -> bfloat16 (hand-worked values where a detour
through float32 would round twice; torch agreement where no double rounding
can occur); the projection against explicit per-element dot products
(math.fsum) on tiny inputs; the Q | K | V slice order with weights built
from identity blocks; and the publish composition (the pool holds RoPE of
the K slice and the V slice at the published rows).
"""
import math

import numpy as np
import torch

from oracle.numerics import bf16_to_f32
from oracle.publish import gather, publish
from oracle.qkv import f64_to_bf16, qkv_project, qkv_publish
from tests._pipeline import storage


def bits(v):
    return int(f64_to_bf16(np.array([v]))[0])


def test_single_rounding_by_hand():
    # just above the halfway point between 1 and 1 + 2^-7: rounds up once;
    # via float32 it would first land on the tie and then go to even (1.0)
    assert bits(1 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert bits(1 + 2 ** -8) == 0x3F80                 # exact tie: to even
    assert bits(1 + 3 * 2 ** -8) == 0x3F82             # exact tie: to even (up)
    assert bits(-2.0) == 0xC000 and bits(0.0) == 0x0000
    assert bits(2.0 ** -130) == 0x0008                 # subnormal, exact
    assert bits(3.0e38) == 0x7F62


def test_agrees_with_torch_without_double_rounding():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, 200_000)))
    a = a.astype(np.float32).astype(np.float64)        # float32 values: one rounding only
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(f64_to_bf16(a), ref.view(np.uint16))


def test_projection_brute_force():
    rng = np.random.default_rng(1)
    H, D, hid, n = 2, 4, 6, 3
    x = storage(torch.from_numpy(rng.standard_normal((n, hid)).astype(np.float32)).to(torch.bfloat16), "bf16")
    w = storage(torch.from_numpy(rng.standard_normal((3 * H * D, hid)).astype(np.float32)).to(torch.bfloat16), "bf16")
    b = storage(torch.from_numpy(rng.standard_normal(3 * H * D).astype(np.float32)).to(torch.bfloat16), "bf16")
    q, k, v = qkv_project(x, w, H, D, bias=b)
    xf, wf_, bf = (bf16_to_f32(a).astype(np.float64) for a in (x, w, b))
    for t in range(n):
        for f in range(3 * H * D):
            exact = math.fsum([xf[t, i] * wf_[f, i] for i in range(hid)] + [bf[f]])
            got = (q, k, v)[f // (H * D)][t, (f % (H * D)) // D, f % D]
            assert got == bits(exact), (t, f)


def test_slice_order():
    H, D = 2, 4
    rng = np.random.default_rng(2)
    x = storage(torch.from_numpy(rng.standard_normal((5, H * D)).astype(np.float32)).to(torch.bfloat16), "bf16")
    eye = np.eye(H * D)
    w = storage(torch.from_numpy(np.concatenate([eye, 2 * eye, -eye]).astype(np.float32)).to(torch.bfloat16), "bf16")
    q, k, v = qkv_project(x, w, H, D)
    xf = bf16_to_f32(x).reshape(5, H, D)
    assert np.array_equal(bf16_to_f32(q), xf)
    assert np.array_equal(bf16_to_f32(k), 2 * xf)
    assert np.array_equal(bf16_to_f32(v), -xf)


def test_publish_composition():
    H, D, hid, n, ps = 2, 128, 64, 40, 16
    rng = np.random.default_rng(3)
    x = storage(torch.from_numpy(rng.standard_normal((n, hid)).astype(np.float32)).to(torch.bfloat16), "bf16")
    w = storage(torch.from_numpy(rng.standard_normal((3 * H * D, hid)).astype(np.float32) * 0.1).to(torch.bfloat16), "bf16")
    pos = np.stack([np.arange(n) // 8, np.arange(n) % 8 // 4, np.arange(n) % 4], 1).astype(np.int32)
    table = np.array([3, 0, 4, 1, 2], dtype=np.int32)
    rope = ((44, 42, 42), 1e4)
    kp = np.zeros((5, H, ps, D), np.uint16); vp = np.zeros((5, H, D, ps), np.uint16)
    q_rot = qkv_publish(kp, vp, table, ps, x, w, H, D, pos, 7, rope)
    q, k, v = qkv_project(x, w, H, D)
    kp2 = np.zeros_like(kp); vp2 = np.zeros_like(vp)
    k_rot, q_rot2 = publish(kp2, vp2, table, ps, k, v, pos, 7, "bf16", rope=rope, q=q)
    assert np.array_equal(kp, kp2) and np.array_equal(vp, vp2) and np.array_equal(q_rot, q_rot2)
    kg, vg = gather(kp, vp, table, ps, np.arange(7, 7 + n))
    assert np.array_equal(kg, k_rot) and np.array_equal(vg, v)
