"""The prefill attention's rescale path taken on every key tile.

The bf16 attention forms P against a running value and only checks each
query's row sum; past the bound (2^32 by default) the wave takes the tile's
max, raises the running value, rescales O and l and forms P again.  Random
inputs reach that branch only on a wave's first visible tile.  Here the
testing override GDLA_ATTN_SUM_LIMIT=1 sends every tile through it (mixed
lanes that raise and lanes that keep their value, on every step), and the
layer must still match the fp64 oracle to the bf16 bar: g = 3 and g = 4,
causal and windowed, a packed stream, and the backward, whose recomputed
forward stores the log-sum-exp built from that running value."""

import pytest

from attention_gdla_prefill_02_amd import configs
from tests import test_gpu_backward as bwd
from tests.helpers import SMALL, assert_close
from tests.test_gpu_packed import run_packed
from tests.test_gpu_prefill import run_layer

pytestmark = pytest.mark.gpu

SMALL4 = dict(SMALL, group=4)


@pytest.fixture
def every_tile(monkeypatch):
    monkeypatch.setenv("GDLA_ATTN_SUM_LIMIT", "1")
    print("[case] GDLA_ATTN_SUM_LIMIT=1: rescale on every tile", flush=True)


@pytest.mark.parametrize("name,B,L,window", [
    ("small", 2, 257, 0), ("small", 1, 300, 100), ("small", 2, 200, 1), ("small4", 1, 257, 64),
    ("motif", 1, 320, 0), ("motif", 1, 333, 128), ("report", 1, 512, 128)])
def test_prefill_rescale_every_tile(every_tile, name, B, L, window):
    shapes = {"small": SMALL, "small4": SMALL4, "motif": configs.MOTIF_SHAPES, "report": configs.REPORT_SHAPES}[name]
    r = run_layer(shapes, "bf16", B, L, window, seed=61 + L)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"y {name} B={B} L={L} W={window}, rescale on every tile")


@pytest.mark.parametrize("window", [0, 64])
def test_packed_prefill_rescale_every_tile(every_tile, window):
    lens, pos = [37, 0, 130, 1, 64, 200], [0, 5, 300, 7, 1000, 0]
    r = run_packed(SMALL, "bf16", lens, pos, window, seed=62)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"packed y W={window}, rescale on every tile")


@pytest.mark.parametrize("window", [0, 40])
def test_backward_rescale_every_tile(every_tile, window):
    bwd.run(SMALL, 2, 150, window, seed=63)
