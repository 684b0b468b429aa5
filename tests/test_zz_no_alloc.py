"""gdla_decode_noalloc (the decode step on the library's own device scratch,
for callers that cannot allocate) against gdla_decode with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller
batch and a windowed layer; outputs and appended cache rows must be the same
bits (same kernels, same inputs)."""

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from tests.helpers import make_layer

pytestmark = pytest.mark.gpu


def _state(shapes, B, cap, ctx, seed):
    cache_c, lens = inputs.make_decode_state(B, cap, shapes["kv_rank"], shapes["d_rope"], ctx, seed, "bf16")
    x = inputs.make_x(B, 1, shapes["d_model"], seed, "bf16")[:, 0].contiguous()
    return cache_c, lens, x


@pytest.mark.parametrize("shapes", [configs.MOTIF_SHAPES, configs.REPORT_SHAPES], ids=["motif", "report"])
def test_decode_noalloc_matches_decode(shapes):
    Wd, _ = make_layer(shapes, 501, "bf16")
    for B, cap, ctx, window, seed in ((64, 8192, (1024, 8192), 0, 502), (7, 6144, (1, 6144), 4096, 503)):
        print(f"[case] decode_noalloc B={B} cap={cap} W={window} heads={shapes['n_noise'] * (shapes['group'] + 1)}",
              flush=True)
        cache_c, lens, xc = _state(shapes, B, cap, ctx, seed)
        cfg = gdla.make_config(shapes, window, "bf16")
        assert gdla.decode_workspace_size(cfg, B) <= gdla.DECODE_NOALLOC_SCRATCH_BYTES
        x, lens_d = xc.to("cuda"), lens.to("cuda")
        cache_ref, cache_na = cache_c.to("cuda"), cache_c.to("cuda")
        y_ref = gdla.decode(cfg, Wd, x, cache_ref, lens_d)
        y_na = torch.full_like(y_ref, float("nan"))
        gdla.decode_noalloc(cfg, Wd, x, cache_na, lens_d, y=y_na)
        torch.cuda.synchronize()
        assert torch.isfinite(y_na).all()
        diff = (y_na.float() - y_ref.float()).abs().max().item()
        print(f"[parity] decode_noalloc vs decode B={B} W={window}: max_abs={diff:.3e}", flush=True)
        assert torch.equal(y_na, y_ref), "y differs from gdla_decode"
        assert torch.equal(cache_na, cache_ref), "cache differs from gdla_decode"
        del cache_ref, cache_na


def test_decode_noalloc_rejects_oversized_batch():
    s = configs.REPORT_SHAPES
    cfg = gdla.make_config(s, 0, "bf16")
    B = 512
    assert gdla.decode_workspace_size(cfg, B) > gdla.DECODE_NOALLOC_SCRATCH_BYTES
    Wd, _ = make_layer(s, 504, "bf16")
    x = torch.zeros((B, s["d_model"]), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 3.0)
    cache = torch.zeros((B, 64, s["kv_rank"] + s["d_rope"]), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(gdla.GdlaError, match="scratch holds"):
        gdla.decode_noalloc(cfg, Wd, x, cache, lens, y=y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a rejected call must launch nothing"
