"""Packed variable-length prefill and the paged latent cache: the HIP path
through the C ABI against the fp64 oracle on the same bits -- mixed lengths
with empty, one-token and ragged sequences, several query blocks per
sequence, full and windowed masks, shuffled page pools whose unowned rows
hold NaN -- plus bitwise identities with the uniform-batch and dense-cache
entry points, and the packed block at full size on sampled rows."""

import time

import numpy as np
import pytest
import torch

from attention_gdla_prefill_02_amd import configs, gdla, inputs
from oracle import gdla_ref as R
from tests.helpers import SMALL, assert_close, host64, make_layer, oracle_cfg
from tests.test_gpu_decode import run_batch_decode

pytestmark = pytest.mark.gpu

MIX = [1, 63, 64, 65, 200, 0, 7, 130]
MIX_POS = [0, 1000, 5, 70, 0, 3, 4000, 31]


def _dt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def run_packed(shapes, dtype, lens, pos, window, seed, page_rows=32, fill=7.0, yarn=None):
    print(f"[case] packed shapes={shapes['d_model']}/{shapes['group']} dtype={dtype} lens={lens} pos={pos} "
          f"W={window} page_rows={page_rows} yarn={yarn}", flush=True)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Wd, W64 = make_layer(shapes, seed, dtype)
    xc = inputs.make_x(1, T, shapes["d_model"], seed, dtype)[0]
    RL = shapes["kv_rank"] + shapes["d_rope"]
    bt, npages = inputs.page_table([p + n for p, n in zip(pos, lens)], page_rows, seed)
    pages = torch.full((npages, page_rows, RL), fill, dtype=_dt(dtype), device="cuda")
    cfg = gdla.make_config(shapes, window, dtype, yarn=yarn)
    y = gdla.prefill_packed(cfg, Wd, xc.to("cuda"), _i32(cu), pos_offsets=_i32(pos), pages=pages,
                            block_table=_i32(bt))
    torch.cuda.synchronize()
    ocfg = oracle_cfg(shapes, window)
    if yarn:
        from dataclasses import replace
        ocfg = replace(ocfg, yarn_factor=yarn[0], yarn_orig_len=yarn[1], yarn_beta_fast=yarn[2],
                       yarn_beta_slow=yarn[3])
    ref = R.gdla_layer_packed(inputs.widen(xc), W64, ocfg, cu, pos)
    return dict(y=host64(y), ref=ref, pages=host64(pages), bt=bt, cu=cu, page_rows=page_rows)


def check_pages(r, lens, pos, dtype, fill=7.0):
    """Every token's row sits at its slot; every other pool row is untouched."""
    got = r["pages"]
    written = np.zeros(got.shape[:2], dtype=bool)
    rows, refs = [], []
    for b, n in enumerate(lens):
        for i in range(n):
            pg, rr = R.paged_slot(r["bt"], r["page_rows"], b, pos[b] + i)
            written[pg, rr] = True
            rows.append(got[pg, rr])
            refs.append(r["ref"]["cache"][r["cu"][b] + i])
    if rows:
        assert_close(np.stack(rows), np.stack(refs), dtype, "paged cache rows")
    rest = got[~written]
    assert np.all(rest == fill), "rows outside the call were touched"


@pytest.mark.parametrize("window", [0, 64, 1])
def test_packed_prefill_mixed_lengths(window):
    r = run_packed(SMALL, "bf16", MIX, MIX_POS, window, seed=61)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"packed y W={window}")
    check_pages(r, MIX, MIX_POS, "bf16")


def test_packed_prefill_many_sequences():
    lens = [1000] + [1] * 40 + [17] * 12 + [0, 0] + [129, 64]
    pos = [(37 * b) % 300 for b in range(len(lens))]
    r = run_packed(SMALL, "bf16", lens, pos, 0, seed=62, page_rows=64)
    assert_close(r["y"], r["ref"]["y"], "bf16", "packed y, 57 sequences")
    check_pages(r, lens, pos, "bf16")


@pytest.mark.parametrize("window", [0, 128])
def test_packed_prefill_report_shapes(window):
    lens = [33, 1, 95, 64, 0, 40]
    pos = [0, 9, 100, 7, 0, 1]
    r = run_packed(configs.REPORT_SHAPES, "bf16", lens, pos, window, seed=63)
    assert_close(r["y"], r["ref"]["y"], "bf16", f"packed y, report shapes W={window}")
    check_pages(r, lens, pos, "bf16")


@pytest.mark.parametrize("window", [0, 16])
def test_packed_prefill_tiny_fp32(window):
    lens = [5, 0, 40, 1, 77]
    pos = [3, 0, 0, 50, 11]
    r = run_packed(configs.TINY_SHAPES, "fp32", lens, pos, window, seed=64)
    assert_close(r["y"], r["ref"]["y"], "fp32", f"packed y, tiny fp32 W={window}")
    check_pages(r, lens, pos, "fp32")


def test_packed_prefill_yarn_long_positions():
    lens = [90, 1, 150]
    pos = [200000, 5, 131000]
    r = run_packed(SMALL, "bf16", lens, pos, 0, seed=65, yarn=(64.0, 4096, 32.0, 1.0))
    assert_close(r["y"], r["ref"]["y"], "bf16", "packed y with YaRN at long positions")
    check_pages(r, lens, pos, "bf16")


def test_packed_equal_lengths_match_uniform_bitwise():
    """Equal lengths packed end to end give the uniform-batch call's bits, and
    a paged cache with the in-order table holds the dense cache's bits."""
    B, L = 3, 100
    Wd, _ = make_layer(SMALL, 66, "bf16")
    x = inputs.make_x(B, L, SMALL["d_model"], 66, "bf16").to("cuda")
    RL = SMALL["kv_rank"] + SMALL["d_rope"]
    for window in (0, 40):
        cfg = gdla.make_config(SMALL, window, "bf16")
        dense = torch.zeros((B, 128, RL), dtype=torch.bfloat16, device="cuda")
        yu = gdla.prefill(cfg, Wd, x, pos_offset=20, cache=dense)
        pages = torch.zeros((B * 4, 32, RL), dtype=torch.bfloat16, device="cuda")
        bt = _i32(np.arange(B * 4).reshape(B, 4))
        yp = gdla.prefill_packed(cfg, Wd, x.reshape(B * L, -1), _i32([0, L, 2 * L, 3 * L]),
                                 pos_offsets=_i32([20] * B), pages=pages, block_table=bt)
        torch.cuda.synchronize()
        assert torch.equal(yu.reshape(B * L, -1), yp), f"packed != uniform, W={window}"
        assert torch.equal(dense, pages.reshape(B, 128, RL)), f"paged rows != dense rows, W={window}"


def _decode_state(shapes, lens, seed, page_rows, extra_pages=0):
    """Random normalized cache rows for positions < lens[b], written into a
    shuffled pool; every other pool row is NaN."""
    RL = shapes["kv_rank"] + shapes["d_rope"]
    rng = np.random.Generator(np.random.PCG64(seed))
    bt, npages = inputs.page_table([n + 1 for n in lens], page_rows, seed, max_pages=extra_pages)
    pool = np.full((npages, page_rows, RL), np.nan, dtype=np.float32)
    for b, n in enumerate(lens):
        for p in range(n):
            z = rng.standard_normal(shapes["kv_rank"])
            z /= np.sqrt(np.mean(z * z))
            pool[bt[b, p // page_rows], p % page_rows] = np.concatenate([z, rng.standard_normal(shapes["d_rope"])])
    return inputs.to_storage(pool, "bf16"), bt


@pytest.mark.parametrize("window,page_rows", [(0, 32), (64, 32), (0, 128), (100, 64)])
def test_paged_decode(window, page_rows):
    s = SMALL
    lens = [0, 1, 31, 32, 33, 100, 1000, 2047]
    print(f"[case] paged decode W={window} page_rows={page_rows} lens={lens}", flush=True)
    Wd, W64 = make_layer(s, 67, "bf16")
    pool_c, bt = _decode_state(s, lens, 68, page_rows)
    xc = inputs.make_x(len(lens), 1, s["d_model"], 67, "bf16")[:, 0].contiguous()
    pool = pool_c.to("cuda")
    y = gdla.decode_paged(gdla.make_config(s, window, "bf16"), Wd, xc.to("cuda"), pool, _i32(bt), _i32(lens))
    torch.cuda.synchronize()
    ref = R.gdla_decode_paged(inputs.widen(xc), W64, oracle_cfg(s, window), inputs.widen(pool_c), bt, page_rows,
                              np.array(lens))
    assert_close(host64(y), ref["y"], "bf16", f"paged decode y W={window} page_rows={page_rows}")
    got = host64(pool)
    before = inputs.widen(pool_c)
    new_rows = np.stack([got[pg, rr] for pg, rr in ref["slots"]])
    assert_close(new_rows, ref["new_rows"], "bf16", "appended rows")
    for pg, rr in ref["slots"]:
        got[pg, rr] = before[pg, rr]
    assert np.array_equal(got, before, equal_nan=True), "pool rows other than the appended ones changed"


def test_paged_decode_outside_the_table():
    """A position at or past page_rows * max_pages writes nothing and gives
    y = 0; the other sequences are unaffected."""
    s = SMALL
    page_rows = 32
    lens = [40, 127, 5]
    Wd, W64 = make_layer(s, 69, "bf16")
    pool_c, bt = _decode_state(s, [40, 60, 5], 70, page_rows)   # sequence 1 owns 2 pages: positions < 64 fit
    bt = bt[:, :2].copy()
    assert bt.shape[1] == 2
    xc = inputs.make_x(3, 1, s["d_model"], 69, "bf16")[:, 0].contiguous()
    pool = pool_c.to("cuda")
    y = gdla.decode_paged(gdla.make_config(s, 0, "bf16"), Wd, xc.to("cuda"), pool, _i32(bt), _i32(lens))
    torch.cuda.synchronize()
    y = host64(y)
    assert np.all(y[1] == 0.0), "a sequence outside its table must give y = 0"
    keep = [0, 2]
    ref = R.gdla_decode_paged(inputs.widen(xc[keep]), W64, oracle_cfg(s, 0), inputs.widen(pool_c), bt[keep],
                              page_rows, np.array([lens[b] for b in keep]))
    assert_close(y[keep], ref["y"], "bf16", "decode of the sequences inside their tables")
    got = host64(pool)
    for pg, rr in ref["slots"]:
        got[pg, rr] = inputs.widen(pool_c)[pg, rr]
    assert np.array_equal(got, inputs.widen(pool_c), equal_nan=True), "a row was written for the outside sequence"


def test_dense_decode_outside_capacity_gives_zero():
    s = SMALL
    Wd, _ = make_layer(s, 71, "bf16")
    cap = 64
    cache = torch.zeros((2, cap, s["kv_rank"] + s["d_rope"]), dtype=torch.bfloat16, device="cuda")
    cache[:, :10] = 0.5
    before = cache.clone()
    x = inputs.make_x(2, 1, s["d_model"], 71, "bf16")[:, 0].contiguous().to("cuda")
    y = gdla.decode(gdla.make_config(s, 0, "bf16"), Wd, x, cache, _i32([10, cap]))
    torch.cuda.synchronize()
    assert torch.all(y[1] == 0), "a position at the capacity must give y = 0"
    assert torch.equal(cache[1], before[1]), "nothing may be written for it"
    assert bool(torch.isfinite(y[0]).all())


def test_packed_prefill_then_paged_decode():
    """Prefill writes every sequence but its last token into the pool; decoding
    the last tokens against it gives the packed layer's last rows."""
    lens = [50, 1, 130, 64]
    Wd, W64 = make_layer(SMALL, 72, "bf16")
    T = sum(lens)
    xc = inputs.make_x(1, T, SMALL["d_model"], 72, "bf16")[0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    first = [n - 1 for n in lens]
    cu_first = np.concatenate([[0], np.cumsum(first)])
    idx_first = np.concatenate([np.arange(cu[b], cu[b + 1] - 1) for b in range(len(lens))])
    last = cu[1:] - 1
    RL = SMALL["kv_rank"] + SMALL["d_rope"]
    bt, npages = inputs.page_table(lens, 32, 72)
    for window in (0, 48):
        print(f"[case] packed prefill then paged decode W={window}", flush=True)
        cfg = gdla.make_config(SMALL, window, "bf16")
        pages = torch.full((npages, 32, RL), float("nan"), dtype=torch.bfloat16, device="cuda")
        x = xc.to("cuda")
        x_first = x[torch.from_numpy(idx_first).to("cuda")].contiguous()
        x_last = x[torch.from_numpy(last).to("cuda")].contiguous()
        gdla.prefill_packed(cfg, Wd, x_first, _i32(cu_first), pages=pages, block_table=_i32(bt))
        yd = gdla.decode_paged(cfg, Wd, x_last, pages, _i32(bt), _i32(first))
        torch.cuda.synchronize()
        ref = R.gdla_layer_packed(inputs.widen(xc), W64, oracle_cfg(SMALL, window), cu)
        assert_close(host64(yd), ref["y"][last], "bf16", f"decode after packed prefill W={window}")


def test_packed_hybrid_l32k_sampled_rows():
    """The packed block workload at full size: every layer on the GPU's own
    input to it, scored on sampled rows of three sequences (the longest, the
    shortest and one more) against the oracle run on those sequences alone."""
    w = configs.WORKLOADS["packed_hybrid_l32k"]
    s = w.shapes
    lens = inputs.packed_lengths(w.L, *w.len_range, w.seed)
    cu = np.concatenate([[0], np.cumsum(lens)])
    order = np.argsort(lens)
    picks = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})
    print(f"[workload] packed_hybrid_l32k: {len(lens)} sequences, scoring {[lens[b] for b in picks]}", flush=True)
    xc = inputs.make_x(1, w.L, s["d_model"], w.seed, "bf16")[0]
    x = xc.to("cuda")
    cu_d = _i32(cu)
    ws = gdla.alloc_workspace(gdla.prefill_packed_workspace_size(gdla.make_config(s, 0, "bf16"), len(lens), w.L))
    for l, win in enumerate(w.windows):
        Wc = inputs.make_weights(s, configs.layer_seed(w, l), "bf16")
        Wd = {k: v.to("cuda") for k, v in Wc.items()}
        cfg = gdla.make_config(s, win, "bf16")
        y = gdla.prefill_packed(cfg, Wd, x, cu_d, workspace=ws)
        torch.cuda.synchronize()
        if l in (0, 1):
            W64 = {k: inputs.widen(v) for k, v in Wc.items()}
            x_host = x.cpu()
            for b in picks:
                n = lens[b]
                rows = inputs.sampled_rows(n, win, w.sampled_rows, configs.layer_seed(w, l) + b)
                t0 = time.time()
                ref = R.gdla_layer(inputs.widen(x_host[cu[b]:cu[b + 1]])[None], W64, oracle_cfg(s, win), rows=rows)
                print(f"[workload] layer {l} W={win} sequence {b} (L={n}): oracle {len(rows)} rows "
                      f"in {time.time() - t0:.1f} s", flush=True)
                got = host64(y[torch.from_numpy(cu[b] + np.array(rows)).to("cuda")])
                assert_close(got, ref["y"][0], "bf16", f"packed block layer {l} sequence {b} ({len(rows)} rows)")
        x = gdla.prefill_packed(cfg, Wd, x, cu_d, residual=x, workspace=ws)
    assert bool(torch.isfinite(x).all())


def test_paged_decode_b64_all():
    """The timed paged decode workload (64 heads, 512-wide latent, contexts
    U{1024..32768}, 64-row pages in a shuffled pool whose unowned rows are
    NaN), every sequence against the oracle, full and W=4096 layers."""
    run_batch_decode("paged_decode_b64")
