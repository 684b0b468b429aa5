"""Prefill parity: the HIP path through the C ABI against the fp64 oracle on
the same seeded bits, element by element over every row (small and ragged
shapes, several tiles, edge cases), plus the tiny fp32 workload."""

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, assert_close, errors, host64, make_layer, oracle_cfg

pytestmark = pytest.mark.gpu


def run_layer(shapes, dtype, B, L, window, seed, pos_offset=0, init="fan_in", gamma="ones", with_cache=False):
    print(f"[case] shapes={shapes} dtype={dtype} B={B} L={L} W={window} seed={seed} pos={pos_offset}", flush=True)
    Wd, W64 = make_layer(shapes, seed, dtype, init=init, gamma=gamma)
    xc = inputs.make_x(B, L, shapes["d_model"], seed, dtype)
    x = xc.to("cuda")
    cfg = gdla.make_config(shapes, window, dtype)
    cache = None
    if with_cache:
        cache = torch.full((B, pos_offset + L + 5, shapes["kv_rank"] + shapes["d_rope"]), 7.0,
                           dtype=x.dtype, device="cuda")
    ws = gdla.alloc_workspace(gdla.prefill_workspace_size(cfg, B, L))
    y = gdla.prefill(cfg, Wd, x, pos_offset=pos_offset, cache=cache, workspace=ws)
    torch.cuda.synchronize()
    ref = R.gdla_layer(inputs.widen(xc), W64, oracle_cfg(shapes, window), pos_offset=pos_offset)
    return dict(y=host64(y), ref=ref, cfg=cfg, ws=ws, cache=cache, x=x, Wd=Wd)


SMALL_CASES = [
    (1, 1, 0), (2, 63, 0), (2, 200, 0), (1, 300, 100), (2, 257, 64), (1, 130, 1), (1, 100, 500), (1, 64, 0),
]


@pytest.mark.parametrize("B,L,window", SMALL_CASES)
def test_prefill_small_bf16(B, L, window):
    run_small(B, L, window)


@pytest.mark.parametrize("B,L,window", [(2, 257, 0), (1, 300, 100)])
def test_prefill_small_bf16_both_output_projections(out_proj, B, L, window):
    run_small(B, L, window)


def run_small(B, L, window):
    r = run_layer(SMALL, "bf16", B, L, window, seed=11)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"y B={B} L={L} W={window}")
    lay = gdla.prefill_layout(r["cfg"], B, L)
    nz = 2 * SMALL["group"] * SMALL["n_noise"] * SMALL["d_v"]
    z = r["ws"][lay["z"]:lay["z"] + B * L * nz].view(torch.bfloat16).reshape(B, L, -1)
    assert_close(host64(z), r["ref"]["Z"], "bf16", "Z")


def test_prefill_random_gains_and_offset_bf16():
    r = run_layer(SMALL, "bf16", 2, 150, 0, seed=12, pos_offset=1000, gamma="random", with_cache=True)
    assert_close(r["y"], r["ref"]["y"], "bf16", "y (random gains, pos_offset 1000)")
    cache = host64(r["cache"])
    assert_close(cache[:, 1000:1150], r["ref"]["cache"], "bf16", "cache rows")
    assert np.all(cache[:, :1000] == 7.0) and np.all(cache[:, 1150:] == 7.0), "cache rows outside the call were touched"


def test_prefill_tiny_fp32_workload():
    w = configs.WORKLOADS["tiny_fp32"]
    r = run_layer(w.shapes, "fp32", w.B, w.L, 0, seed=configs.layer_seed(w, 0), init=w.weight_init)
    assert_close(r["y"], r["ref"]["y"], "fp32", "tiny fp32 y")


@pytest.mark.parametrize("window,L", [(16, 128), (1, 37), (0, 1), (200, 77)])
def test_prefill_tiny_fp32_windows(window, L):
    w = configs.WORKLOADS["tiny_fp32"]
    r = run_layer(w.shapes, "fp32", 2, L, window, seed=5, init="fan_in", gamma="random")
    assert_close(r["y"], r["ref"]["y"], "fp32", f"tiny fp32 W={window} L={L}")


@pytest.fixture(params=["hipblaslt", "library"])
def out_proj(request, monkeypatch):
    """The bf16 output projection runs on hipBLASLt; GDLA_NO_HIPBLASLT selects
    the library's own GEMM, its fallback.  Both are checked."""
    if request.param == "library":
        monkeypatch.setenv("GDLA_NO_HIPBLASLT", "1")
    print(f"[case] output projection on {request.param}", flush=True)
    return request.param


def test_residual_variant_bf16(out_proj):
    Wd, _ = make_layer(SMALL, 13, "bf16")
    x = inputs.make_x(1, 96, SMALL["d_model"], 13, "bf16").to("cuda")
    cfg = gdla.make_config(SMALL, 0, "bf16")
    y = gdla.prefill(cfg, Wd, x)
    yr = gdla.prefill(cfg, Wd, x, residual=x)
    torch.cuda.synchronize()
    ref = (x.double() + y.double())
    ma, _ = errors(host64(yr), ref.cpu().numpy())
    assert ma <= 2.0 ** -7 * float(ref.abs().max()), ma


def test_determinism_bf16():
    Wd, _ = make_layer(SMALL, 14, "bf16")
    x = inputs.make_x(2, 333, SMALL["d_model"], 14, "bf16").to("cuda")
    cfg = gdla.make_config(SMALL, 70, "bf16")
    a = gdla.prefill(cfg, Wd, x)
    b = gdla.prefill(cfg, Wd, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_layer_deterministic_32k():
    """A 32K full-causal layer at the timed shapes, twice: the same bits, so
    no kernel on the path (hipBLASLt's stream-K output projection included)
    reduces in a run-dependent order."""
    s, T = configs.MOTIF_SHAPES, 32768
    print(f"[case] full layer twice, L={T}", flush=True)
    Wd = {k: v.to("cuda") for k, v in inputs.make_weights(s, 31, "bf16").items()}
    x = inputs.make_x(1, T, s["d_model"], 31, "bf16").to("cuda")
    cfg = gdla.make_config(s, 0, "bf16")
    ws = gdla.alloc_workspace(gdla.prefill_workspace_size(cfg, 1, T))
    y1 = gdla.prefill(cfg, Wd, x, residual=x, workspace=ws)
    y2 = gdla.prefill(cfg, Wd, x, residual=x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y1).all()
    assert torch.equal(y1, y2)


def _ws_view(ws, off, n, dtype, shape):
    esize = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * esize].view(dtype).reshape(shape)


def test_prefill_stages_compose_and_intermediates():
    """gdla_prefill_stages run one stage per call on one workspace gives gdla_prefill's
    y bit for bit, and the intermediates gdla_prefill_workspace_layout names hold
    what the oracle computes: lambda and the sigmoid gate (fp32), the RoPE'd
    queries, content keys and rotary key (fp16 in the bf16 configuration)."""
    B, L, window = 2, 200, 0
    Wd, W64 = make_layer(SMALL, 17, "bf16")
    xc = inputs.make_x(B, L, SMALL["d_model"], 17, "bf16")
    x = xc.to("cuda")
    cfg = gdla.make_config(SMALL, window, "bf16")
    y_all = gdla.prefill(cfg, Wd, x)
    ws = gdla.alloc_workspace(gdla.prefill_workspace_size(cfg, B, L))
    y = torch.empty_like(x)
    for st in (gdla.STAGE_DOWN, gdla.STAGE_PREP, gdla.STAGE_EXPAND, gdla.STAGE_QG, gdla.STAGE_ATTN, gdla.STAGE_OUT):
        gdla.prefill(cfg, Wd, x, y=y, workspace=ws, stages=st)
    torch.cuda.synchronize()
    assert torch.equal(y, y_all), "stage-by-stage calls must reproduce gdla_prefill"
    lay = gdla.prefill_layout(cfg, B, L)
    T, H, nS, nN = B * L, SMALL["group"] * SMALL["n_noise"] + SMALL["n_noise"], SMALL["group"] * SMALL["n_noise"], \
        SMALL["n_noise"]
    ocfg = oracle_cfg(SMALL, window)
    x64 = inputs.widen(xc)
    pos = np.arange(L, dtype=np.float64)
    refs = [R.project_tokens(x64[b], W64, ocfg, pos) for b in range(B)]
    lam = _ws_view(ws, lay["lam"], T * nS, torch.float32, (T, nS))
    gate = _ws_view(ws, lay["gate"], T * nS * 128, torch.float32, (T, nS * 128))
    q = _ws_view(ws, lay["q"], T * H * 192, torch.float16, (T, H, 192))
    kc = _ws_view(ws, lay["kc"], T * nN * 128, torch.float16, (T, nN, 128))
    kr = _ws_view(ws, lay["kr"], T * 64, torch.float16, (T, 64))
    assert_close(host64(lam), np.concatenate([r["lam"] for r in refs]), "bf16", "workspace lambda")
    assert_close(host64(gate), np.concatenate([r["gate"] for r in refs]), "bf16", "workspace gate")
    assert_close(host64(q), np.concatenate([r["q"] for r in refs]), "bf16", "workspace queries (fp16)")
    assert_close(host64(kr), np.concatenate([r["kr"] for r in refs]), "bf16", "workspace rotary key (fp16)")
    kc_ref = np.concatenate([R.latent_expand_from_norm(r["ckvn"], W64["w_ukv"], ocfg)[0] for r in refs])
    assert_close(host64(kc), kc_ref, "bf16", "workspace content keys (fp16)")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_latent_expand(dtype):
    shapes = SMALL if dtype == "bf16" else configs.TINY_SHAPES
    rng = np.random.Generator(np.random.PCG64(3))
    T = 333
    c = inputs.to_storage(rng.standard_normal((T, shapes["kv_rank"] + 64)) * 3.0, dtype)
    W = inputs.make_weights(shapes, 4, dtype, gamma="random")
    cfg = gdla.make_config(shapes, 0, dtype)
    k, v, cn = gdla.latent_expand(cfg, c.to("cuda"), W["g_kv"].to("cuda"), W["w_ukv"].to("cuda"))
    torch.cuda.synchronize()
    kr, vr, cnr = R.latent_expand(inputs.widen(c)[:, :shapes["kv_rank"]], inputs.widen(W["g_kv"]),
                                  inputs.widen(W["w_ukv"]), oracle_cfg(shapes))
    assert_close(host64(cn), cnr, dtype, "c_norm")
    assert_close(host64(k), kr, dtype, "k_nope")
    assert_close(host64(v), vr, dtype, "v")


def test_prefill_motif_shapes_bf16_short():
    """Full-size head/rank shapes of the large workloads at a short length."""
    r = run_layer(configs.MOTIF_SHAPES, "bf16", 1, 320, 0, seed=21)
    assert_close(r["y"], r["ref"]["y"], "bf16", "motif shapes L=320")
    r = run_layer(configs.MOTIF_SHAPES, "bf16", 1, 333, 128, seed=22)
    assert_close(r["y"], r["ref"]["y"], "bf16", "motif shapes L=333 W=128")
