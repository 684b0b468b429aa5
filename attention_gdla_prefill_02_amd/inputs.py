"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  It draws numbers and rounds them to the storage dtype; it holds none
of the GDLA arithmetic.

All draws use numpy's PCG64 in a fixed order.  bf16 storage is produced by
round-to-nearest-even from float32 (torch's CPU cast), and the float64 view the
oracle receives is the exact widening of those same bits.
"""

from __future__ import annotations

import math

import numpy as np
import torch

WEIGHT_NAMES = ("w_dq", "g_q", "w_dkv", "g_kv", "w_lambda", "w_uq", "w_ukv", "w_gate", "w_o")


def weight_shapes(s: dict) -> dict:
    """[out, in] shapes of every weight (gains are vectors)."""
    nS = s["group"] * s["n_noise"]
    H = nS + s["n_noise"]
    dqk = s["d_nope"] + s["d_rope"]
    return {
        "w_dq": (s["q_rank"], s["d_model"]),
        "g_q": (s["q_rank"],),
        "w_dkv": (s["kv_rank"] + s["d_rope"], s["d_model"]),
        "g_kv": (s["kv_rank"],),
        "w_lambda": (nS, s["d_model"]),
        "w_uq": (H * dqk, s["q_rank"]),
        "w_ukv": (s["n_noise"] * (s["d_nope"] + s["d_v"]), s["kv_rank"]),
        "w_gate": (nS * s["d_v"], s["q_rank"]),
        "w_o": (s["d_model"], nS * s["d_v"]),
    }


def _std(name: str, shape, init: str) -> float:
    if init == "std002":
        return 0.02
    # "fan_in": projections keep unit-scale activations (std = fan_in^-1/2);
    # the lambda and gate predictors use std 0.02.
    if name in ("w_lambda", "w_gate"):
        return 0.02
    return 1.0 / math.sqrt(shape[1])


def to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float array -> CPU tensor in the storage dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def widen(t: torch.Tensor) -> np.ndarray:
    """Exact float64 view of a CPU tensor's stored values."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def make_weights(shapes: dict, seed: int, dtype: str, init: str = "fan_in",
                 gamma: str = "ones") -> dict:
    """One layer's weights as CPU tensors in the storage dtype.
    gamma = "ones" (the workloads) or "random" (N(1, 0.1^2) gains)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shp in weight_shapes(shapes).items():
        if name in ("g_q", "g_kv"):
            a = np.ones(shp) if gamma == "ones" else 1.0 + 0.1 * rng.standard_normal(shp)
        else:
            a = rng.standard_normal(shp, dtype=np.float32) * np.float32(_std(name, shp, init))
        out[name] = to_storage(a, dtype)
    return out


def make_x(B: int, L: int, d_model: int, seed: int, dtype: str) -> torch.Tensor:
    """Activations x ~ N(0, 1), [B, L, d_model], drawn row by row so large
    inputs never materialize in float64."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    out = torch.empty((B, L, d_model), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    chunk = max(1, (1 << 24) // d_model)
    for b in range(B):
        for l0 in range(0, L, chunk):
            l1 = min(L, l0 + chunk)
            out[b, l0:l1] = to_storage(rng.standard_normal((l1 - l0, d_model), dtype=np.float32), dtype)
    return out


def make_decode_state(B: int, capacity: int, kv_rank: int, d_rope: int, ctx_range, seed: int,
                      dtype: str):
    """Synthetic decode state: context lengths c_b ~ U{lo..hi}; the cache holds
    c_b - 1 rows per sequence (the new token goes to row c_b - 1), each row
    [z / rms(z) | r] with z ~ N(0, I_kv_rank), r ~ N(0, I_d_rope).
    Rows at and beyond cache_lens are zero.  Returns (cache, cache_lens)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    lo, hi = ctx_range
    ctx = rng.integers(lo, hi + 1, size=B)
    lens = (ctx - 1).astype(np.int32)
    cache = torch.zeros((B, capacity, kv_rank + d_rope),
                        dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    for b in range(B):
        n = int(lens[b])
        z = rng.standard_normal((n, kv_rank), dtype=np.float32)
        z /= np.sqrt(np.mean(z * z, axis=1, keepdims=True))
        r = rng.standard_normal((n, d_rope), dtype=np.float32)
        cache[b, :n] = to_storage(np.concatenate([z, r], axis=1), dtype)
    return cache, torch.from_numpy(lens)


def sampled_rows(L: int, window: int, count: int, seed: int) -> list:
    """`count` seeded query rows plus the fixed boundary rows
    {0, 1, W-2, W-1, W, W+1, L-1} (those inside [0, L))."""
    rng = np.random.Generator(np.random.PCG64(seed + 15485863))
    rows = set(int(r) for r in rng.choice(L, size=min(count, L), replace=False))
    W = window if window > 0 else 4096
    for r in (0, 1, W - 2, W - 1, W, W + 1, L - 1):
        if 0 <= r < L:
            rows.add(r)
    return sorted(rows)


def packed_lengths(T: int, lo: int, hi: int, seed: int) -> list:
    """Sequence lengths ~ U{lo..hi} drawn until they cover T tokens; the last
    one is cut so that the lengths sum to exactly T."""
    rng = np.random.Generator(np.random.PCG64(seed + 32452843))
    out, total = [], 0
    while total < T:
        n = int(min(rng.integers(lo, hi + 1), T - total))
        out.append(n)
        total += n
    return out


def page_table(rows_needed, page_rows: int, seed: int, spare: int = 3, max_pages: int = 0):
    """A shuffled page pool for sequences that need rows_needed[b] rows each:
    every sequence gets ceil(rows / page_rows) distinct pages in random pool
    order, `spare` pages belong to nobody, and unused table entries are -1.
    Returns (block_table int32 [B, max_pages], num_pages)."""
    rng = np.random.Generator(np.random.PCG64(seed + 49979687))
    need = [(int(r) + page_rows - 1) // page_rows for r in rows_needed]
    mp = max(max_pages, max(need) if need else 1, 1)
    num_pages = sum(need) + spare
    order = rng.permutation(num_pages)
    bt = np.full((len(need), mp), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[k:k + n]
        k += n
    return bt, num_pages
