"""YaRN parity: the HIP path with the long-context RoPE settings of the Motif 3
report (factor 64 over a native 4096, beta_fast 32, beta_slow 1, full-causal
layers only) against the fp64 oracle on the same bits, for prefill at short
and very long positions, the appended cache rows, decode against a cache
written with those rows, and the windowed layers that must ignore the
settings; both placements of YaRN's temperature ("rotary": m on cos and sin,
"logit": m^2 on the whole logit)."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, assert_close, host64, make_layer, oracle_cfg

pytestmark = pytest.mark.gpu

YARN = (64.0, 4096, 32.0, 1.0)


TEMPS = ["rotary", "logit"]


def yarn_oracle_cfg(shapes, window, temp="rotary"):
    return replace(oracle_cfg(shapes, window), yarn_factor=YARN[0], yarn_orig_len=YARN[1],
                   yarn_beta_fast=YARN[2], yarn_beta_slow=YARN[3], yarn_temperature=temp)


def run(shapes, dtype, B, L, window, seed, pos_offset=0, with_cache=False, yarn=YARN, temp="rotary"):
    print(f"[case] yarn={yarn} temperature={temp} shapes={shapes['d_model']}/{shapes['kv_rank']} dtype={dtype} "
          f"B={B} L={L} W={window} pos={pos_offset}", flush=True)
    Wd, W64 = make_layer(shapes, seed, dtype)
    xc = inputs.make_x(B, L, shapes["d_model"], seed, dtype)
    cfg = gdla.make_config(shapes, window, dtype, yarn=yarn, yarn_temperature=temp)
    cache = None
    if with_cache:
        cache = torch.full((B, pos_offset + L + 3, shapes["kv_rank"] + shapes["d_rope"]), 5.0,
                           dtype=xc.dtype, device="cuda")
    y = gdla.prefill(cfg, Wd, xc.to("cuda"), pos_offset=pos_offset, cache=cache)
    torch.cuda.synchronize()
    return xc, W64, host64(y), cache


@pytest.mark.parametrize("temp", TEMPS)
@pytest.mark.parametrize("pos_offset", [0, 250000])
def test_yarn_prefill_small(pos_offset, temp):
    B, L = 2, 300
    xc, W64, y, cache = run(SMALL, "bf16", B, L, 0, seed=41, pos_offset=pos_offset, with_cache=True, temp=temp)
    ref = R.gdla_layer(inputs.widen(xc), W64, yarn_oracle_cfg(SMALL, 0, temp), pos_offset=pos_offset)
    assert_close(y, ref["y"], "bf16", f"YaRN ({temp}) prefill y pos_offset={pos_offset}")
    rows = host64(cache)[:, pos_offset:pos_offset + L]
    assert_close(rows, ref["cache"], "bf16", "YaRN cache rows")
    plain = R.gdla_layer(inputs.widen(xc), W64, oracle_cfg(SMALL, 0), pos_offset=pos_offset)
    d = float(np.max(np.abs(plain["y"] - ref["y"])))
    print(f"[yarn] oracle |y_yarn - y_plain| max {d:.3e}", flush=True)
    assert d > 0.05, "the YaRN settings should change this layer's output"


@pytest.mark.parametrize("temp", TEMPS)
def test_yarn_ignored_on_windowed_layers(temp):
    _, _, y_yarn, _ = run(SMALL, "bf16", 2, 200, 64, seed=42, temp=temp)
    _, _, y_plain, _ = run(SMALL, "bf16", 2, 200, 64, seed=42, yarn=None)
    assert np.array_equal(y_yarn, y_plain), "a windowed layer must not apply YaRN"


@pytest.mark.parametrize("temp", TEMPS)
def test_yarn_prefill_tiny_fp32(temp):
    w = configs.WORKLOADS["tiny_fp32"]
    xc, W64, y, _ = run(w.shapes, "fp32", 1, w.L, 0, seed=43, pos_offset=100000, temp=temp)
    ref = R.gdla_layer(inputs.widen(xc), W64, yarn_oracle_cfg(w.shapes, 0, temp), pos_offset=100000)
    assert_close(y, ref["y"], "fp32", f"YaRN ({temp}) tiny fp32")


def test_yarn_prefill_motif_shapes_long_offset():
    xc, W64, y, _ = run(configs.MOTIF_SHAPES, "bf16", 1, 320, 0, seed=44, pos_offset=200000)
    ref = R.gdla_layer(inputs.widen(xc), W64, yarn_oracle_cfg(configs.MOTIF_SHAPES, 0), pos_offset=200000)
    assert_close(y, ref["y"], "bf16", "YaRN motif shapes L=320 at position 200000")


@pytest.mark.parametrize("temp", TEMPS)
def test_yarn_decode_small(temp):
    s = SMALL
    lens = [0, 1, 100, 4095, 4096, 9000, 20000, 29999]
    B, cap = len(lens), 30000
    print(f"[case] yarn ({temp}) decode B={B} cap={cap}", flush=True)
    Wd, W64 = make_layer(s, 45, "bf16")
    rng = np.random.Generator(np.random.PCG64(50))
    z = rng.standard_normal((B, cap, s["kv_rank"]))
    z /= np.sqrt((z ** 2).mean(-1, keepdims=True))
    rows = np.concatenate([z, rng.standard_normal((B, cap, s["d_rope"]))], -1)
    cache_c = inputs.to_storage(rows, "bf16")
    for b in range(B):
        cache_c[b, lens[b]:] = 0
    xc = inputs.make_x(B, 1, s["d_model"], 45, "bf16")[:, 0].contiguous()
    cache = cache_c.to("cuda")
    y = gdla.decode(gdla.make_config(s, 0, "bf16", yarn=YARN, yarn_temperature=temp), Wd, xc.to("cuda"), cache,
                    torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = R.gdla_decode(inputs.widen(xc), W64, yarn_oracle_cfg(s, 0, temp), inputs.widen(cache_c), np.array(lens))
    assert_close(host64(y), ref["y"], "bf16", f"YaRN ({temp}) decode y")
    got_rows = np.stack([host64(cache[b, lens[b]]) for b in range(B)])
    assert_close(got_rows, ref["new_rows"], "bf16", "YaRN appended rows")


@pytest.mark.parametrize("temp", TEMPS)
def test_yarn_prefill_then_decode(temp):
    B, L = 2, 150
    Wd, W64 = make_layer(SMALL, 46, "bf16")
    xc = inputs.make_x(B, L, SMALL["d_model"], 46, "bf16")
    x = xc.to("cuda")
    cfg = gdla.make_config(SMALL, 0, "bf16", yarn=YARN, yarn_temperature=temp)
    cache = torch.zeros((B, L + 2, SMALL["kv_rank"] + SMALL["d_rope"]), dtype=torch.bfloat16, device="cuda")
    gdla.prefill(cfg, Wd, x[:, :L - 1].contiguous(), cache=cache)
    cache_before = cache.cpu()
    yd = gdla.decode(cfg, Wd, x[:, L - 1].contiguous(), cache,
                     torch.full((B,), L - 1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = R.gdla_decode(inputs.widen(xc[:, L - 1]), W64, yarn_oracle_cfg(SMALL, 0, temp),
                        inputs.widen(cache_before), np.full(B, L - 1))
    assert_close(host64(yd), ref["y"], "bf16", f"YaRN ({temp}) decode on the prefill-written cache")
