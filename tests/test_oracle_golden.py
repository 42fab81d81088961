"""Hand-worked examples of chunk-wise causal attention (CPU only).

tests/golden/attention_hand_examples.json holds tiny inputs whose outputs
follow by hand from the mask rule of "Wave Forcing: Towards Speed-of-Light
Streaming Video Generation", section 3.1 (each case carries its derivation).
They pin the oracle's visibility rule, its prefix handling and its paging
against numbers that do not come from the oracle: a reversed or shifted
mask, a dropped prefix segment or a wrong page lookup changes them.
"""
import json
import os

import numpy as np
import pytest

from oracle.attention import chunk_attention
from oracle.publish import publish

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "attention_hand_examples.json")) as f:
    GOLDEN = json.load(f)


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["name"] for c in GOLDEN["cases"]])
def test_hand_worked_attention(case):
    ps = GOLDEN["page_size"]
    table = np.array(GOLDEN["page_table"], dtype=np.int32)
    k = np.array(case["k"], dtype=np.float32)[:, None, :]     # [tokens, H=1, D]
    v = np.array(case["v"], dtype=np.float32)[:, None, :]
    q = np.array(case["q"], dtype=np.float32)[:, None, :]
    n, _, D = k.shape
    kp = np.full((len(table), 1, ps, D), np.nan, dtype=np.float32)
    vp = np.full((len(table), 1, D, ps), np.nan, dtype=np.float32)
    publish(kp, vp, table, ps, k, v, None, 0, "fp32")
    segs = [tuple(s) for s in GOLDEN["segments"]]
    out, lse = chunk_attention(kp, vp, table, ps, segs, q, GOLDEN["q_slot_start"], 0,
                               case["scale"], "fp32")
    np.testing.assert_allclose(out[:, 0, :], np.array(case["out"], dtype=np.float64),
                               rtol=0, atol=case["atol"])
    np.testing.assert_allclose(lse[0], np.array(case["lse"]), rtol=0, atol=case["atol"])
