"""Writes tests/golden/tiny_fp32_oracle.json: oracle outputs of the tiny fp32
layer (seeded inputs) at a few rows.  The pages print no worked GDLA example,
so this file is a regression fixture for the oracle itself: it is produced
only by the oracle, and a change to the oracle's arithmetic must regenerate it
and say why.  Run:  python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from attention_gdla_prefill_02_amd import configs, inputs  # noqa: E402
from oracle import gdla_ref as R  # noqa: E402

ROWS = [0, 1, 2, 63, 64, 127]


def main():
    w = configs.WORKLOADS["tiny_fp32"]
    s = w.shapes
    Wt = inputs.make_weights(s, configs.layer_seed(w, 0), "fp32", init=w.weight_init)
    x = inputs.make_x(w.B, w.L, s["d_model"], w.seed, "fp32")
    cfg = R.Cfg(**configs.cfg_dict(w, 0))
    out = R.gdla_layer(inputs.widen(x), {k: inputs.widen(v) for k, v in Wt.items()}, cfg, rows=ROWS)
    doc = {
        "what": "oracle y rows of the tiny fp32 GDLA layer (seeded inputs); regression fixture",
        "workload": "tiny_fp32", "rows": ROWS,
        "y": [[float(v) for v in r] for r in out["y"][0]],
        "cache_row0": [float(v) for v in out["cache"][0, 0]],
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32_oracle.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
