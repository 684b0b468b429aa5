"""Backward parity: the HIP layer backward (forward recomputed from x) through
the C ABI against the oracle's fp64 gradients on the same bits, for dx and
every weight gradient, over several query and key tiles with ragged tails,
full and windowed masks, position offsets, YaRN, and the report's g = 4
shapes.  Tolerance: the bf16 path rounds dZ-derived products, dH, dS and the
transposed operands to bf16 before each MFMA; each rounding adds ~2e-3 of
relative error, so gradient tensors are held to rel-L2 <= 1.5e-2 and max-abs
<= 3e-2 of the tensor's largest magnitude (floored at 1e-3, for gradients
that are exactly zero in the reference, such as dQ with a window of 1)."""

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, errors, host64, make_layer, oracle_cfg

pytestmark = pytest.mark.gpu

GRAD_TOL = dict(rel_l2=1.5e-2, max_rel=3e-2)


def check(got, ref, what):
    ma, rl = errors(got, ref)
    scale = max(float(np.max(np.abs(ref))) if ref.size else 1.0, 1e-3)   # floor: exactly-zero references
    print(f"[grad] {what}: rel_l2={rl:.3e} max_abs={ma:.3e} (|ref| max {scale:.3e})", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert rl <= GRAD_TOL["rel_l2"], f"{what}: rel_l2 {rl:.3e}"
    assert ma <= GRAD_TOL["max_rel"] * scale, f"{what}: max_abs {ma:.3e} > {GRAD_TOL['max_rel']} x {scale:.3e}"


def run(shapes, B, L, window, seed, pos_offset=0, yarn=None, temp="rotary"):
    print(f"[case] backward shapes={shapes['d_model']}/{shapes['group']} B={B} L={L} W={window} "
          f"pos={pos_offset} yarn={yarn} temperature={temp}", flush=True)
    Wd, W64 = make_layer(shapes, seed, "bf16", gamma="random")
    xc = inputs.make_x(B, L, shapes["d_model"], seed, "bf16")
    dyc = inputs.make_x(B, L, shapes["d_model"], seed + 1000, "bf16")
    cfg = gdla.make_config(shapes, window, "bf16", yarn=yarn, yarn_temperature=temp)
    dx, grads = gdla.backward(cfg, Wd, xc.to("cuda"), dyc.to("cuda"), pos_offset=pos_offset)
    torch.cuda.synchronize()
    ocfg = oracle_cfg(shapes, window)
    if yarn:
        from dataclasses import replace
        ocfg = replace(ocfg, yarn_factor=yarn[0], yarn_orig_len=yarn[1], yarn_beta_fast=yarn[2],
                       yarn_beta_slow=yarn[3], yarn_temperature=temp)
    ref = R.gdla_layer_backward(inputs.widen(xc), W64, ocfg, inputs.widen(dyc), pos_offset=pos_offset)
    check(host64(dx), ref["dx"], "dx")
    for n in inputs.WEIGHT_NAMES:
        check(host64(grads[n]), ref[n], n)


@pytest.mark.parametrize("B,L,window", [(1, 64, 0), (2, 100, 0), (1, 300, 0), (2, 150, 40), (1, 257, 1)])
def test_backward_small(B, L, window):
    run(SMALL, B, L, window, seed=81 + L)


@pytest.mark.parametrize("B,L,window", [(2, 100, 0), (1, 257, 40)])
def test_backward_small_library_gemms(monkeypatch, B, L, window):
    """The gradient GEMMs on the library's own GEMM (GDLA_NO_HIPBLASLT), the
    fallback of the hipBLASLt path the other tests take."""
    monkeypatch.setenv("GDLA_NO_HIPBLASLT", "1")
    run(SMALL, B, L, window, seed=81 + L)


def test_backward_deterministic():
    """Two calls on the same inputs give the same bits (no atomics in any
    gradient reduction, hipBLASLt's included), at a length whose weight
    gradients reduce over 4,096 tokens."""
    Wd, _ = make_layer(SMALL, 90, "bf16", gamma="random")
    x = inputs.make_x(1, 4096, SMALL["d_model"], 90, "bf16").to("cuda")
    dy = inputs.make_x(1, 4096, SMALL["d_model"], 1090, "bf16").to("cuda")
    cfg = gdla.make_config(SMALL, 0, "bf16")
    dx1, g1 = gdla.backward(cfg, Wd, x, dy)
    dx2, g2 = gdla.backward(cfg, Wd, x, dy)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2)
    for n in inputs.WEIGHT_NAMES:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("temp", ["rotary", "logit"])
def test_backward_position_offset_and_yarn(temp):
    run(SMALL, 2, 130, 0, seed=82, pos_offset=70000, yarn=(64.0, 4096, 32.0, 1.0), temp=temp)


@pytest.mark.parametrize("window", [0, 64])
def test_backward_report_shapes_g4(window):
    s = dict(configs.REPORT_SHAPES, d_model=512, q_rank=256)
    run(s, 1, 160, window, seed=83)


def run_packed(shapes, lens, window, seed, pos=None, yarn=None):
    """The packed backward against the oracle's: sequences of `lens` (empty and
    one-token ones included) packed into one stream at positions `pos`."""
    T = int(sum(lens))
    print(f"[case] packed backward shapes={shapes['d_model']}/{shapes['group']} lens={lens} W={window} "
          f"pos={pos} yarn={yarn}", flush=True)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = [0] * len(lens) if pos is None else list(pos)
    Wd, W64 = make_layer(shapes, seed, "bf16", gamma="random")
    xc = inputs.make_x(1, T, shapes["d_model"], seed, "bf16")[0]
    dyc = inputs.make_x(1, T, shapes["d_model"], seed + 1000, "bf16")[0]
    cfg = gdla.make_config(shapes, window, "bf16", yarn=yarn)
    dx, grads = gdla.backward_packed(cfg, Wd, xc.to("cuda"), dyc.to("cuda"), torch.tensor(cu, device="cuda"),
                                     pos_offsets=torch.tensor(np.asarray(pos, np.int32), device="cuda"))
    torch.cuda.synchronize()
    ocfg = oracle_cfg(shapes, window)
    if yarn:
        from dataclasses import replace
        ocfg = replace(ocfg, yarn_factor=yarn[0], yarn_orig_len=yarn[1], yarn_beta_fast=yarn[2],
                       yarn_beta_slow=yarn[3])
    ref = R.gdla_layer_packed_backward(inputs.widen(xc), W64, ocfg, inputs.widen(dyc), cu, pos)
    check(host64(dx), ref["dx"], "packed dx")
    for n in inputs.WEIGHT_NAMES:
        check(host64(grads[n]), ref[n], "packed " + n)
    return dx, grads


@pytest.mark.parametrize("window", [0, 40])
def test_backward_packed_small(window):
    run_packed(SMALL, [37, 0, 130, 1, 64, 200, 33], window, seed=86, pos=[0, 5, 300, 7, 1000, 0, 64])


def test_backward_packed_report_shapes_g4():
    s = dict(configs.REPORT_SHAPES, d_model=512, q_rank=256)
    run_packed(s, [150, 97, 1, 129], 64, seed=87, pos=[0, 12, 3, 4000])


def test_backward_packed_yarn():
    run_packed(SMALL, [100, 161, 5], 0, seed=88, pos=[70000, 0, 250000], yarn=(64.0, 4096, 32.0, 1.0))


def test_backward_packed_equal_lengths_match_the_batch():
    """Equal lengths packed end to end give the batched backward's dx and
    weight gradients (the same per-sequence work, other work lists)."""
    B, L = 3, 96
    Wd, _ = make_layer(SMALL, 89, "bf16", gamma="random")
    xc = inputs.make_x(B, L, SMALL["d_model"], 89, "bf16")
    dyc = inputs.make_x(B, L, SMALL["d_model"], 1089, "bf16")
    cfg = gdla.make_config(SMALL, 50, "bf16")
    x, dy = xc.to("cuda"), dyc.to("cuda")
    dxb, gb = gdla.backward(cfg, Wd, x, dy)
    cu = torch.tensor([0, L, 2 * L, 3 * L], dtype=torch.int32, device="cuda")
    dxp, gp = gdla.backward_packed(cfg, Wd, x.reshape(B * L, -1).contiguous(), dy.reshape(B * L, -1).contiguous(), cu)
    torch.cuda.synchronize()
    check(host64(dxp), host64(dxb).reshape(B * L, -1), "packed vs batched dx")
    for n in inputs.WEIGHT_NAMES:
        check(host64(gp[n]), host64(gb[n]), "packed vs batched " + n)


def test_backward_motif_shapes():
    run(configs.MOTIF_SHAPES, 1, 200, 0, seed=84)


def test_backward_motif_shapes_l4096_dense():
    """Motif shapes at L = 4096 with a dense upstream gradient on every row:
    the dK/dV accumulation over 4096 query rows (128 query tiles per key
    block) and every weight gradient against the oracle's full backward."""
    run(configs.MOTIF_SHAPES, 1, 4096, 0, seed=85)


@pytest.mark.parametrize("layer", [0, 1])
def test_backward_hybrid_l32k_sparse_rows(layer):
    """Full size (Motif shapes, L = 32768, the block's full-causal layer and a
    W = 4096 layer): dy is nonzero only on sampled rows, so the oracle's
    row-restricted backward gives every gradient exactly (dx on all rows,
    through the keys and values; every weight gradient); the kernels run at
    full size, unaware of the sparsity."""
    import time
    w = configs.WORKLOADS["hybrid_l32k"]
    s = w.shapes
    win = w.windows[layer]
    rows = inputs.sampled_rows(w.L, win, 12, configs.layer_seed(w, layer))
    print(f"[case] backward hybrid_l32k layer {layer} W={win}, {len(rows)} rows with a gradient", flush=True)
    Wc = inputs.make_weights(s, configs.layer_seed(w, layer), "bf16")
    xc = inputs.make_x(w.B, w.L, s["d_model"], w.seed, "bf16")
    rng = np.random.Generator(np.random.PCG64(91 + layer))
    dy_rows = inputs.to_storage(rng.standard_normal((w.B, len(rows), s["d_model"]), dtype=np.float32), "bf16")
    dyc = torch.zeros((w.B, w.L, s["d_model"]), dtype=torch.bfloat16)
    dyc[:, rows] = dy_rows
    cfg = gdla.make_config(s, win, "bf16")
    dx, grads = gdla.backward(cfg, {k: v.to("cuda") for k, v in Wc.items()}, xc.to("cuda"), dyc.to("cuda"))
    torch.cuda.synchronize()
    t0 = time.time()
    ref = R.gdla_layer_backward(inputs.widen(xc), {k: inputs.widen(v) for k, v in Wc.items()},
                                oracle_cfg(s, win), inputs.widen(dy_rows), rows=rows)
    print(f"[workload] oracle backward (rows {len(rows)}) in {time.time() - t0:.1f} s", flush=True)
    check(host64(dx), ref["dx"], "dx")
    for n in inputs.WEIGHT_NAMES:
        check(host64(grads[n]), ref[n], n)
