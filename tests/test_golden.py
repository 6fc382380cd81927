"""Stored checker outputs for the small causal GQA workload still match the
checker run afresh on the same seeded inputs (CPU only)."""

import json
import os

import numpy as np

import oracle
from tiled_attention_03_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "causal_q32_h4kv2_d64.json")


def load_golden():
    with open(GOLDEN) as f:
        doc = json.load(f)
    out = np.array([[float(x) for x in row] for row in doc["out"]])
    lse = np.array([[[float(a), float(b)] for a, b in row] for row in doc["lse"]])
    return doc, out, lse


def test_inputs_are_the_recorded_ones():
    doc, _, _ = load_golden()
    q, k, v = inputs.make_prefill(inputs.CAUSAL_SMALL)
    for name, arr in (("q", q), ("k", k), ("v", v)):
        assert float(arr.astype(np.float64).sum()) == doc["input_checksums"][name]


def test_checker_reproduces_golden():
    doc, out_g, lse_g = load_golden()
    w = inputs.CAUSAL_SMALL
    q, k, v = inputs.make_prefill(w)
    out, lse = oracle.attention_forward(q, k, v, num_heads=w.num_heads,
                                        num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                        mode=w.mode, kv_len=w.kv_len, scale=w.scale)
    np.testing.assert_allclose(out[doc["out_rows"]], out_g, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_g, rtol=0, atol=1e-12)
    # row 0 sees key 0 only: out is V[0] of the head's KV head, log sum is 0
    d = w.head_dim
    for h in range(w.num_heads):
        kvh = h // w.group
        np.testing.assert_allclose(out_g[0, h * d:(h + 1) * d], v[0, kvh * d:(kvh + 1) * d],
                                   rtol=0, atol=1e-12)
    assert np.all(lse_g[0, :, 1] == 0.0)
