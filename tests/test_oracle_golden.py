"""The oracle still reproduces its own stored outputs (tests/golden), and the
input generator is deterministic and rounds to bf16 by round-to-nearest-even."""

import json
import os

import numpy as np
import torch

from attention_gdla_prefill_02_amd import configs, inputs
from oracle import gdla_ref as R

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_fp32_oracle.json")


def test_oracle_regression_fixture():
    doc = json.load(open(GOLD))
    w = configs.WORKLOADS["tiny_fp32"]
    s = w.shapes
    Wt = inputs.make_weights(s, configs.layer_seed(w, 0), "fp32", init=w.weight_init)
    x = inputs.make_x(w.B, w.L, s["d_model"], w.seed, "fp32")
    out = R.gdla_layer(inputs.widen(x), {k: inputs.widen(v) for k, v in Wt.items()},
                       R.Cfg(**configs.cfg_dict(w, 0)), rows=doc["rows"])
    np.testing.assert_allclose(out["y"][0], np.array(doc["y"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["cache"][0, 0], np.array(doc["cache_row0"]), rtol=0, atol=1e-13)


def test_inputs_deterministic_and_rne():
    s = configs.TINY_SHAPES
    a = inputs.make_weights(s, 5, "bf16")
    b = inputs.make_weights(s, 5, "bf16")
    for k in a:
        assert torch.equal(a[k], b[k])
    # RNE: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> rounds to even (1.0)
    t = inputs.to_storage(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]), "bf16")
    assert inputs.widen(t).tolist() == [1.0, 1.0 + 2.0 ** -6]
    x = inputs.make_x(2, 33, 16, 9, "bf16")
    assert x.shape == (2, 33, 16) and x.dtype == torch.bfloat16
    assert abs(float(x.float().std()) - 1.0) < 0.2


def test_decode_state_recipe():
    cache, lens = inputs.make_decode_state(3, 64, 16, 8, (10, 40), 3, "bf16")
    assert cache.shape == (3, 64, 24)
    for b in range(3):
        n = int(lens[b])
        assert 9 <= n <= 39
        z = inputs.widen(cache[b, :n, :16])
        np.testing.assert_allclose(np.sqrt((z ** 2).mean(1)), 1.0, atol=2e-2)
        assert float(cache[b, n:].abs().max()) == 0.0


def test_sampled_rows_include_boundaries():
    rows = inputs.sampled_rows(32768, 4096, 256, 7)
    for r in (0, 1, 4094, 4095, 4096, 4097, 32767):
        assert r in rows
    assert rows == sorted(set(rows)) and len(rows) >= 256
