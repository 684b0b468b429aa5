"""Decode parity: one new token per sequence against the compressed latent
cache, HIP path through the C ABI vs the oracle's plain (non-absorbed) decode
on the same bits; the appended cache rows; prefill -> decode consistency; the
batch-64 workload with a 32K-row cache on a seeded sample of sequences."""

import time

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, assert_close, host64, make_layer, oracle_cfg

pytestmark = pytest.mark.gpu


def run_decode(shapes, B, cap, lens, window, seed, check=None, cache_seed=None):
    print(f"[case] decode shapes={shapes['kv_rank']}/{shapes['n_noise']}x{shapes['group']} B={B} cap={cap} "
          f"W={window} seed={seed}", flush=True)
    Wd, W64 = make_layer(shapes, seed, "bf16")
    rng = np.random.Generator(np.random.PCG64(seed + 5))
    RLn = shapes["kv_rank"] + shapes["d_rope"]
    z = rng.standard_normal((B, cap, shapes["kv_rank"]))
    z /= np.sqrt((z ** 2).mean(-1, keepdims=True))
    rows = np.concatenate([z, rng.standard_normal((B, cap, shapes["d_rope"]))], -1)
    cache_c = inputs.to_storage(rows, "bf16")
    for b in range(B):
        cache_c[b, lens[b]:] = 0
    xc = inputs.make_x(B, 1, shapes["d_model"], seed, "bf16")[:, 0].contiguous()
    cache = cache_c.to("cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cfg = gdla.make_config(shapes, window, "bf16")
    y = gdla.decode(cfg, Wd, xc.to("cuda"), cache, lens_t)
    torch.cuda.synchronize()
    sel = list(range(B)) if check is None else check
    ref = R.gdla_decode(inputs.widen(xc[sel]), W64, oracle_cfg(shapes, window), inputs.widen(cache_c[sel]),
                        np.array(lens)[sel])
    got_rows = np.stack([host64(cache[b, lens[b]]) for b in sel])
    untouched = all(bool(torch.equal(cache[b, lens[b] + 1:].cpu(), cache_c[b, lens[b] + 1:])) and
                    bool(torch.equal(cache[b, :lens[b]].cpu(), cache_c[b, :lens[b]])) for b in sel)
    return host64(y)[sel], ref, got_rows, untouched


@pytest.mark.parametrize("window", [0, 64])
def test_decode_small(window):
    lens = [0, 1, 63, 64, 65, 100, 250, 299]
    y, ref, rows, untouched = run_decode(SMALL, len(lens), 300, lens, window, seed=31)
    assert_close(y, ref["y"], "bf16", f"decode y W={window}")
    assert_close(rows, ref["new_rows"], "bf16", "appended cache rows")
    assert untouched, "decode wrote cache rows other than cache_lens[b]"


def test_decode_motif_shapes():
    rng = np.random.Generator(np.random.PCG64(9))
    lens = [int(v) for v in rng.integers(1, 2047, size=6)] + [0, 2047]
    y, ref, rows, untouched = run_decode(configs.MOTIF_SHAPES, len(lens), 2048, lens, 0, seed=32)
    assert_close(y, ref["y"], "bf16", "decode y (motif shapes)")
    assert_close(rows, ref["new_rows"], "bf16", "appended rows (motif shapes)")
    assert untouched


def test_decode_motif_shapes_window():
    lens = [5000, 4095, 4096, 4097, 100, 7000]
    y, ref, _, _ = run_decode(configs.MOTIF_SHAPES, len(lens), 7168, lens, 4096, seed=33)
    assert_close(y, ref["y"], "bf16", "decode y (motif shapes, W=4096)")


@pytest.mark.parametrize("window", [0, 40])
def test_prefill_then_decode_matches_prefill(window):
    """prefill(L-1) writes the cache; decoding token L-1 against it matches the
    oracle's decode on those same cache bits, and agrees with prefill(L)'s last
    row up to the two paths' bf16 roundings (the cache itself is bf16)."""
    B, L = 3, 130
    Wd, W64 = make_layer(SMALL, 34, "bf16")
    xc = inputs.make_x(B, L, SMALL["d_model"], 34, "bf16")
    x = xc.to("cuda")
    cfg = gdla.make_config(SMALL, window, "bf16")
    cache = torch.zeros((B, L + 4, SMALL["kv_rank"] + SMALL["d_rope"]), dtype=torch.bfloat16, device="cuda")
    full = gdla.prefill(cfg, Wd, x)
    gdla.prefill(cfg, Wd, x[:, :L - 1].contiguous(), cache=cache)
    cache_before = cache.cpu()
    yd = gdla.decode(cfg, Wd, x[:, L - 1].contiguous(), cache,
                     torch.full((B,), L - 1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = R.gdla_decode(inputs.widen(xc[:, L - 1]), W64, oracle_cfg(SMALL, window), inputs.widen(cache_before),
                        np.full(B, L - 1))
    assert_close(host64(yd), ref["y"], "bf16", "decode on the prefill-written cache vs oracle")
    assert_close(host64(yd), host64(full[:, L - 1]), "bf16", "decode after prefill vs GPU prefill",
                 tol=dict(max_abs=2e-2, rel_l2=1e-2))


def oracle_decode_all(xc, W64, shapes, window, cache_c, lens, chunk=8):
    """The oracle's decode of every sequence of a batch, in chunks of `chunk`
    sequences (bounds the float64 copy of the cache)."""
    B = xc.shape[0]
    lens = np.asarray(lens)
    ys, rows = [], []
    t0 = time.time()
    for b0 in range(0, B, chunk):
        sel = list(range(b0, min(B, b0 + chunk)))
        cap = int(lens[sel].max()) + 1
        ref = R.gdla_decode(inputs.widen(xc[sel]), W64, oracle_cfg(shapes, window), inputs.widen(cache_c[sel, :cap]),
                            lens[sel])
        ys.append(ref["y"])
        rows.append(ref["new_rows"])
    print(f"[workload] oracle decode of {B} sequences (W={window}): {time.time() - t0:.1f} s", flush=True)
    return dict(y=np.concatenate(ys), new_rows=np.concatenate(rows))


def nan_pool(cache, lens, page_rows, seed):
    """The rows of a dense device cache [B, capacity, row] below cache_lens,
    moved into a shuffled pool of page_rows-row pages (inputs.page_table, with
    a page for each sequence's new row); every other pool row is NaN.
    Returns (pool, block_table on the device, block_table on the host)."""
    B, cap, RL = cache.shape
    ln = [int(v) for v in lens]
    bt, npages = inputs.page_table([n + 1 for n in ln], page_rows, seed)
    pool = torch.full((npages, page_rows, RL), float("nan"), dtype=cache.dtype, device=cache.device)
    src, dst = [], []
    for b, n in enumerate(ln):
        for j in range((n + page_rows) // page_rows):
            src.append(b * (cap // page_rows) + j)
            dst.append(int(bt[b, j]))
    pos = torch.arange(cap, device=cache.device)[None, :]
    masked = torch.where((pos < lens.to(cache.device)[:, None])[..., None], cache,
                         torch.tensor(float("nan"), dtype=cache.dtype, device=cache.device))
    pool[torch.tensor(dst, device=cache.device)] = masked.reshape(B * (cap // page_rows), page_rows, RL)[
        torch.tensor(src, device=cache.device)]
    del masked
    return pool, torch.from_numpy(bt).to(cache.device), bt


def check_batch(name, y, pool_or_cache, lens, ref, bt=None, page_rows=0):
    """y of every sequence and every appended row against the oracle."""
    assert_close(host64(y), ref["y"], "bf16", f"{name}: y of all {y.shape[0]} sequences")
    got = []
    for b, n in enumerate(int(v) for v in lens):
        if bt is None:
            got.append(host64(pool_or_cache[b, n]))
        else:
            pg, rr = R.paged_slot(bt, page_rows, b, n)
            got.append(host64(pool_or_cache[pg, rr]))
    assert_close(np.stack(got), ref["new_rows"], "bf16", f"{name}: appended rows")


def run_batch_decode(name, paged_too=False):
    """A batch-64 decode workload scored on all 64 sequences, full and
    windowed layers; with paged_too the same state is also decoded from a
    shuffled NaN-filled pool of 64-row pages and scored against the same
    oracle result."""
    w = configs.WORKLOADS[name]
    s = w.shapes
    cache_c, lens = inputs.make_decode_state(w.B, w.capacity, s["kv_rank"], s["d_rope"], w.ctx_range, w.seed, "bf16")
    Wd, W64 = make_layer(s, configs.layer_seed(w, 0), "bf16")
    xc = inputs.make_x(w.B, 1, s["d_model"], w.seed, "bf16")[:, 0].contiguous()
    page_rows = w.page_rows or 64
    for window in w.windows:
        print(f"[case] {name} W={window} (all {w.B} sequences{', dense and paged' if paged_too else ''})", flush=True)
        ref = oracle_decode_all(xc, W64, s, window, cache_c, lens.numpy())
        cfg = gdla.make_config(s, window, "bf16")
        lens_d = lens.to("cuda")
        if not w.page_rows:
            cache = cache_c.to("cuda")
            y = gdla.decode(cfg, Wd, xc.to("cuda"), cache, lens_d)
            torch.cuda.synchronize()
            check_batch(f"{name} dense W={window}", y, cache, lens, ref)
            if not paged_too:
                del cache
                continue
        else:
            cache = cache_c.to("cuda")
        pool, bt_d, bt = nan_pool(cache, lens, page_rows, w.seed)
        del cache
        y = gdla.decode_paged(cfg, Wd, xc.to("cuda"), pool, bt_d, lens_d)
        torch.cuda.synchronize()
        check_batch(f"{name} paged W={window}", y, pool, lens, ref, bt=bt, page_rows=page_rows)
        del pool


def test_decode_workload_b64_all():
    """Batch 64 with a 32768-row cache and contexts U{1024..32768} (the timed
    decode workload), every sequence against the oracle."""
    run_batch_decode("decode_b64")
