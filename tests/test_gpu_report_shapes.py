"""Parity at the report's own layer shapes (group size 4: 64 signal + 16 noise
= 80 query heads, query rank 1024, sliding windows of 128): small shapes over
every row, the report shapes on short sequences over every row, the hybrid
32K block on sampled rows per layer, and batch-64 decode, dense and paged, on every sequence.
"""

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, assert_close, host64, make_layer, oracle_cfg
from tests.test_gpu_decode import run_batch_decode, run_decode
from tests.test_gpu_prefill import run_layer
from tests.test_gpu_workloads import _block_parity

pytestmark = pytest.mark.gpu

SMALL4 = dict(SMALL, group=4)   # 8 signal + 2 noise heads, five query heads per KV head


@pytest.mark.parametrize("B,L,window", [(1, 1, 0), (2, 200, 0), (1, 257, 128), (2, 300, 64), (1, 129, 128)])
def test_prefill_small_g4(B, L, window):
    r = run_layer(SMALL4, "bf16", B, L, window, seed=41)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"g=4 y B={B} L={L} W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_report_shapes_short(window):
    r = run_layer(configs.REPORT_SHAPES, "bf16", 1, 512, window, seed=42)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"report shapes y L=512 W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_decode_small_g4(window):
    lens = [0, 1, 127, 128, 129, 200, 299]
    y, ref, rows, untouched = run_decode(SMALL4, len(lens), 300, lens, window, seed=43)
    assert_close(y, ref["y"], "bf16", f"g=4 decode y W={window}")
    assert_close(rows, ref["new_rows"], "bf16", "g=4 appended cache rows")
    assert untouched


def test_decode_report_shapes():
    rng = np.random.Generator(np.random.PCG64(44))
    lens = [int(v) for v in rng.integers(1, 2047, size=6)] + [0, 2047]
    y, ref, _, untouched = run_decode(configs.REPORT_SHAPES, len(lens), 2048, lens, 128, seed=44)
    assert_close(y, ref["y"], "bf16", "decode y (report shapes, W=128)")
    assert untouched


def test_report_hybrid_l32k_sampled_rows():
    _block_parity("report_hybrid_l32k")


def test_report_decode_b64_all():
    """Batch 64 with a 32768-row cache at the report's shapes (80 query heads),
    every sequence against the oracle, full and W=128 layers, from the dense
    cache and from a shuffled NaN-filled pool of 64-row pages."""
    run_batch_decode("report_decode_b64", paged_too=True)
