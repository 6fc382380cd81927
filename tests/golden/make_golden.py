"""Writes causal_q32_h4kv2_d64.json: float64 checker outputs for the small
causal GQA workload (32 rows, 4 query heads over 2 KV heads, head_dim 64,
scale 1/8), on the seeded inputs of ``tiled_attention_03_amd.inputs``.

Calls only the checker (``oracle``) and the input generator. The stored
values pin the checker against silent drift and serve the GPU parity test.
Run from the repository root: ``python tests/golden/make_golden.py``.
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tiled_attention_03_amd import inputs  # noqa: E402

OUT_ROWS = [0, 1, 2, 15, 30, 31]


def main():
    w = inputs.CAUSAL_SMALL
    q, k, v = inputs.make_prefill(w)
    out, lse = oracle.attention_forward(q, k, v, num_heads=w.num_heads,
                                        num_kv_heads=w.num_kv_heads,
                                        head_dim=w.head_dim, mode=w.mode,
                                        kv_len=w.kv_len, start_pos=w.start_pos,
                                        scale=w.scale)
    doc = {
        "what": "float64 checker output, causal self-attention q_seq=kv_len=32, "
                "num_heads=4, num_kv_heads=2, head_dim=64, scale=1/sqrt(64)",
        "source": "meganeura attention.wgsl (causal variant, GQA map, (max, log sum) "
                  "side output); values written by tests/golden/make_golden.py",
        "workload": w.name,
        "input_checksums": {"q": float(q.astype("float64").sum()),
                            "k": float(k.astype("float64").sum()),
                            "v": float(v.astype("float64").sum())},
        "out_rows": OUT_ROWS,
        "out": [[repr(float(x)) for x in out[r]] for r in OUT_ROWS],
        "lse": [[[repr(float(lse[i, h, 0])), repr(float(lse[i, h, 1]))]
                 for h in range(w.num_heads)] for i in range(w.q_seq)],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "causal_q32_h4kv2_d64.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
