"""Pins for the MXFP8 oracle (oracle/mx.py).

E4M3 codes worked out by hand from the format's definition; agreement with
torch's own float8_e4m3fn conversion (round to nearest even) on in-range
values; saturation; the half-step error bound; block scale codes worked out
by hand (and the clipping case the rule implies); lossless round trips on
the grid; and the 8-bit attention against float64 attention on the decoded
values, by brute force.
"""
import math

import numpy as np
import pytest
import torch

from chunk_wise_causal_amd.workloads import small_config
from oracle.brute import brute_attention
from oracle.mx import (block_scale_code, e4m3_encode, e4m3_value, mx_chunk_attention,
                       mx_dequantize, mx_publish_keys, mx_quantize)
from oracle.publish import publish
from tests._pipeline import storage

HAND = [  # (value, code) from sign | exponent (bias 7) | mantissa
    (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01),
    (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07), (1.875, 0x3F), (0.0, 0x00), (-0.0, 0x80),
    (240.0, 0x77), (3.0, 0x44), (0.3125, 0x2A),
]


def test_hand_codes():
    vals = np.array([v for v, _ in HAND])
    codes = np.array([c for _, c in HAND], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(vals), codes)
    dec = e4m3_value(codes)
    assert np.array_equal(dec, vals) and np.array_equal(np.signbit(dec), np.signbit(vals))
    assert np.isnan(e4m3_value(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_ties_and_saturation():
    # halfway points go to the even mantissa
    y = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 232.0, 464.0])
    assert e4m3_value(e4m3_encode(y)).tolist() == [1.0, 1.25, 0.0, 2.0 ** -9, 224.0, 448.0]
    # beyond the largest finite value: saturation, never NaN
    assert e4m3_value(e4m3_encode(np.array([449.0, 1e6, -500.0, 479.0]))).tolist() == \
        [448.0, 448.0, -448.0, 448.0]


def test_agrees_with_torch_float8():
    rng = np.random.default_rng(0)
    y = rng.standard_normal(200_000) * np.exp2(rng.integers(-14, 9, 200_000))
    y = np.clip(y, -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(y), ref)


def test_half_step_error_bound():
    rng = np.random.default_rng(1)
    y = rng.uniform(-448, 448, 100_000) * np.exp2(rng.integers(-12, 1, 100_000))
    d = e4m3_value(e4m3_encode(y))
    _, ex = np.frexp(np.abs(y))
    step = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    assert (np.abs(d - y) <= step / 2).all()


def test_block_scale_codes():
    # floor(log2 amax) - 8 + 127
    assert block_scale_code(np.array([1.0, 448.0, 1.9, 0.5, 2.0 ** -130, 0.0,
                                      3.0e38])).tolist() == [119, 127, 119, 118, 0, 0, 246]
    # amax = 1.0 -> scale 2^-8: the block maximum lands on 256 exactly
    x = np.zeros((1, 32)); x[0, 3] = 1.0; x[0, 7] = -0.25
    c, s = mx_quantize(x)
    assert s.tolist() == [[119]] and e4m3_value(c[0, 3]) == 256.0
    assert np.array_equal(mx_dequantize(c, s), x)
    # the rule clips: amax = 1.875 * 2^k maps to 480 > 448
    x[0, 3] = 1.875
    c, s = mx_quantize(x)
    assert e4m3_value(c[0, 3]) == 448.0 and mx_dequantize(c, s)[0, 3] == 1.75
    # an all-zero block: scale code 0, zero codes
    c, s = mx_quantize(np.zeros((2, 64)))
    assert (s == 0).all() and (c == 0).all()


def test_block_error_bound_and_independence():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * np.exp2(rng.integers(-5, 5, (50, 1)))
    c, s = mx_quantize(x)
    d = mx_dequantize(c, s)
    for b in range(4):
        blk = x[:, 32 * b:32 * b + 32]
        _, ex = np.frexp(np.abs(blk).max(axis=1))
        top = np.exp2(ex - 1.0)[:, None]          # 2^floor(log2 amax)
        # relative half step 2^-4 in the normal range; an absolute floor at
        # the block's smallest step below it; clipping only above 1.75 * top
        err = np.abs(d[:, 32 * b:32 * b + 32] - blk)
        bound = np.maximum(np.abs(blk) * 2.0 ** -4, top * 2.0 ** -18)
        clip = np.abs(blk) > 1.75 * top
        assert (err[~clip] <= bound[~clip]).all()
        assert (np.abs(d[:, 32 * b:32 * b + 32][clip]) == (1.75 * top * np.ones_like(blk))[clip]).all()
    # a block's codes depend on that block only
    x2 = x.copy(); x2[:, 32:64] *= 1000
    c2, s2 = mx_quantize(x2)
    assert np.array_equal(c2[:, :32], c[:, :32]) and np.array_equal(c2[:, 64:], c[:, 64:])


def test_grid_values_round_trip():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (40, 64)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38              # no NaN codes
    codes[:, 0] = 0x7E; codes[:, 32] = 0x7E          # each block's max is 448 -> scale 1
    x = e4m3_value(codes)
    c, s = mx_quantize(x)
    assert (s == 127).all() and np.array_equal(mx_dequantize(c, s), x)


def test_mx_attention_against_brute_force():
    """Publish keys through the MX pool, then the 8-bit attention equals
    float64 brute-force attention on the decoded keys and queries."""
    cfg = small_config(frame_rows=2, frame_cols=4, frames_per_chunk=2, anchor_tokens=8,
                       n_hist=1, slots=2, page_size=16, heads=2)
    rng = np.random.default_rng(4)
    n_kv, H, D, ps = cfg.n_kv, cfg.heads, cfg.head_dim, cfg.page_size
    npg = cfg.n_logical_pages
    table = rng.permutation(npg).astype(np.int32)
    g = torch.Generator().manual_seed(4)
    k = storage(torch.randn(n_kv, H, D, generator=g).to(torch.bfloat16), "bf16")
    v = storage(torch.randn(n_kv, H, D, generator=g).to(torch.bfloat16), "bf16")
    q = storage(torch.randn(cfg.n_q, H, D, generator=g).to(torch.bfloat16), "bf16")
    kp = np.zeros((npg, H, ps, D), np.uint16); vp = np.zeros((npg, H, D, ps), np.uint16)
    publish(kp, vp, table, ps, k, v, None, 0, "bf16")
    k8 = np.zeros((npg, H, ps, D), np.uint8); k8s = np.zeros((npg, H, ps, D // 32), np.uint8)
    mx_publish_keys(k8, k8s, table, ps, k, 0, "bf16")
    out, lse = mx_chunk_attention(k8, k8s, vp, table, ps, cfg.segments(), q, cfg.q_slot_start(),
                                  0, cfg.scale)
    from oracle.numerics import to_f32
    kd = mx_dequantize(*mx_quantize(to_f32(k, "bf16")))
    qd = mx_dequantize(*mx_quantize(to_f32(q, "bf16")))
    ref, ref_lse = brute_attention(qd, kd, to_f32(v, "bf16").astype(np.float64), cfg.segments(),
                                   cfg.q_slot_start(), 0, cfg.scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    # quantization moves the result, but not far, from the bf16 attention
    from oracle.attention import chunk_attention
    o16, _ = chunk_attention(kp, vp, table, ps, cfg.segments(), q, cfg.q_slot_start(), 0,
                             cfg.scale, "bf16")
    assert 0 < np.abs(out - o16).max() < 0.1
