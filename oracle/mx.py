"""MXFP8 keys and queries for the low-precision QK^T (oracle; test
infrastructure).

[WF] §5.5: across model scales the pages also run the pipeline with Sage
attention and 8-bit weights and activations (Sage + W8A8), i.e. an 8-bit
QK^T.  The pages do not fix a format.  The reading here is the one that the target's
matrix cores take natively: OCP microscaling, FP8 E4M3 elements with one
power-of-two scale (E8M0) per 32 consecutive features of a token's head
vector, for Q and K; P V stays bfloat16.

E4M3 (the OCP variant without infinities): sign, 4 exponent bits (bias 7),
3 mantissa bits.  Normal values (1 + m/8) * 2^(e-7) for e = 1..15 (e = 15,
m = 7 is NaN), subnormals m/8 * 2^-6; largest finite 448, smallest
subnormal 2^-9.

Block quantization (OCP MX): with amax the largest |v| of the 32 values,
the shared scale is X = 2^(floor(log2 amax) - 8) (8 is the exponent of
E4M3's largest power of two), stored as the biased exponent
floor(log2 amax) - 8 + 127 clamped to [0, 254] (0 when amax = 0).  Each
element is v / X rounded to the nearest E4M3 value, ties to even, and
saturated to +-448 (v / X can reach 2^9 - 1 ulp; values above 448 clip).
"""
from __future__ import annotations

import numpy as np

from .numerics import to_f32

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64 (NaN codes give NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each finite y (ties to even), saturating at
    +-448.  The sign of zero is kept."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # binade of a (the subnormal binade shares the step of 2^-6)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, -6)
    step = np.exp2(e - 3.0)
    v = np.round(a / step) * step            # numpy rounds halves to even
    v = np.minimum(v, E4M3_MAX)
    # encode the (exactly representable) v
    _, ev = np.frexp(np.where(v > 0, v, 1.0))
    ev = ev - 1
    sub = v < 2.0 ** -6
    code_sub = np.round(v / 2.0 ** -9)
    code_nrm = (ev + 7) * 8 + np.round((v / np.exp2(ev) - 1.0) * 8)
    code = np.where(sub, code_sub, code_nrm).astype(np.int64)
    code |= np.where(np.signbit(y), 0x80, 0)
    return code.astype(np.uint8)


def block_scale_code(amax: np.ndarray) -> np.ndarray:
    """E8M0 code of the shared scale for blocks with largest magnitude amax."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    code = np.clip(ex - 1 - 8 + 127, 0, 254)
    return np.where(amax > 0, code, 0).astype(np.uint8)


def mx_quantize(x: np.ndarray):
    """x [..., D] (float values; D a multiple of 32) -> (codes uint8 [..., D],
    scales uint8 [..., D // 32])."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // BLOCK, BLOCK)
    sc = block_scale_code(np.abs(blocks).max(axis=-1))
    scale = np.exp2(sc.astype(np.float64) - 127.0)[..., None]
    codes = e4m3_encode(blocks / scale)
    return codes.reshape(x.shape), sc


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of mx_quantize's encoding: float64 [..., D]."""
    v = e4m3_value(codes)
    blocks = v.reshape(*v.shape[:-1], v.shape[-1] // BLOCK, BLOCK)
    out = blocks * np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)[..., None]
    return out.reshape(v.shape)


def mx_publish_keys(k8_pool: np.ndarray, k8_scales: np.ndarray, page_table: np.ndarray,
                    page_size: int, k_storage: np.ndarray, dst_start: int, dtype: str):
    """Quantize keys (storage array [n, H, D], RoPE already applied) and write
    them to logical rows dst_start.. of the MX key pool, in place:
    k8_pool [num_pages][H][page_size][D] codes, k8_scales
    [num_pages][H][page_size][D // 32] scale codes."""
    codes, sc = mx_quantize(to_f32(k_storage, dtype))
    for t in range(k_storage.shape[0]):
        L = dst_start + t
        page = int(page_table[L // page_size])
        r = L % page_size
        k8_pool[page, :, r, :] = codes[t]
        k8_scales[page, :, r, :] = sc[t]


def mx_chunk_attention(k8_pool, k8_scales, v_pool, page_table, page_size: int, segments,
                       q: np.ndarray, q_slot_start, first_slot: int, scale: float,
                       heads=None, rows=None, block: int = 1024):
    """Chunk-wise causal attention with the 8-bit QK^T: scores from the
    MXFP8 keys of the pool and the MXFP8-quantized bfloat16 queries (both
    decoded exactly to float64), softmax and P V in float64 over the
    bfloat16 V pool.  Same rows/heads selection and outputs as
    oracle.attention.chunk_attention."""
    from .attention import visible_tokens

    n_rows, H, D = q.shape
    heads = range(H) if heads is None else list(heads)
    out = np.full((n_rows, H, D), np.nan)
    lse = np.full((H, n_rows), np.nan)
    table = np.asarray(page_table, dtype=np.int64)
    for g in range(len(q_slot_start) - 1):
        s = first_slot + g
        r0, r1 = q_slot_start[g], q_slot_start[g + 1]
        sel = np.arange(r0, r1) if rows is None else np.asarray(rows.get(g, []), dtype=np.int64)
        if len(sel) == 0:
            continue
        vis = visible_tokens(segments, s)
        pages, prow = table[vis // page_size], vis % page_size
        for h in heads:
            kh = mx_dequantize(k8_pool[pages, h, prow, :], k8_scales[pages, h, prow, :])
            vh = to_f32(v_pool[pages, h, :, prow], "bf16").astype(np.float64)
            for b in range(0, len(sel), block):
                idx = sel[b:b + block]
                c, sc = mx_quantize(to_f32(q[idx, h], "bf16"))
                qh = mx_dequantize(c, sc)
                z = scale * (qh @ kh.T)
                m = z.max(axis=1, keepdims=True)
                p = np.exp(z - m)
                l = p.sum(axis=1, keepdims=True)
                out[idx, h] = (p @ vh) / l
                lse[h, idx] = (m + np.log(l))[:, 0]
    return out, lse
