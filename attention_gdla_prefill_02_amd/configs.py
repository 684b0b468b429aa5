"""The synthetic GDLA workloads (shapes, dtypes, masks and seeds only).

Shapes follow the layer described in "Motif 3: Technical Report" (the
model-configuration paragraph: 16 KV heads, 192-dim query-key heads with a
64-dim rotary part, 128-dim values, a 512-dim KV latent) with the group size
g = 3 and query rank 1536 these workloads fix, and the sliding window of 4096
tokens from "Open-Source Frontier Models: Architecture and Benchmarks of
Rnj-1 and Motif-2", section 1.  This module holds no arithmetic of the method.
"""

from __future__ import annotations

from dataclasses import dataclass, field

# Layer shapes shared by the four large workloads.
MOTIF_SHAPES = dict(d_model=4096, q_rank=1536, kv_rank=512, n_noise=16, group=3,
                    d_nope=128, d_rope=64, d_v=128)
TINY_SHAPES = dict(d_model=256, q_rank=96, kv_rank=64, n_noise=2, group=2,
                   d_nope=32, d_rope=16, d_v=32)
# The report's own layer configuration (model-configuration paragraph of the
# report): group size 4 (64 signal + 16 noise = 80 query heads) and query rank
# 1024; its sliding-window layers use W = 128.
REPORT_SHAPES = dict(d_model=4096, q_rank=1024, kv_rank=512, n_noise=16, group=4,
                     d_nope=128, d_rope=64, d_v=128)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "block" | "packed" | "decode"
    shapes: dict
    dtype: str                # "fp32" | "bf16"
    B: int
    L: int = 0                # tokens per sequence (prefill / block)
    windows: tuple = (0,)     # per layer: 0 = full causal
    weight_init: str = "fan_in"   # "std002" (all N(0, 0.02^2)) | "fan_in"
    seed: int = 0
    ctx_range: tuple = ()     # decode: context lengths c_b ~ U{lo..hi}
    capacity: int = 0         # decode: cache rows per sequence
    len_range: tuple = ()     # packed: sequence lengths ~ U{lo..hi}, cut to sum to L
    page_rows: int = 0        # paged cache: rows per page (0 = dense cache)
    sampled_rows: int = 0     # >0: score this many seeded rows per layer
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_fp32": Workload(
        name="tiny_fp32", kind="prefill", shapes=TINY_SHAPES, dtype="fp32", B=1, L=128,
        windows=(0,), weight_init="std002", seed=0,
        note="tiny GDLA layer, fp32, full causal"),
    "prefill_b4_l4096": Workload(
        name="prefill_b4_l4096", kind="prefill", shapes=MOTIF_SHAPES, dtype="bf16", B=4,
        L=4096, windows=(0,), seed=1,
        note="GDLA prefill, bf16, full causal, B=4 L=4096"),
    "hybrid_l32k": Workload(
        name="hybrid_l32k", kind="block", shapes=MOTIF_SHAPES, dtype="bf16", B=1, L=32768,
        windows=(0, 4096, 4096, 4096), seed=2, sampled_rows=256,
        note="hybrid GDLA block (1 full + 3 x W=4096), bf16, B=1 L=32768"),
    "decode_b64": Workload(
        name="decode_b64", kind="decode", shapes=MOTIF_SHAPES, dtype="bf16", B=64,
        windows=(0, 4096), seed=3, ctx_range=(1024, 32768), capacity=32768,
        note="GDLA decode, bf16, batch 64, contexts U{1024..32768}"),
    "report_hybrid_l32k": Workload(
        name="report_hybrid_l32k", kind="block", shapes=REPORT_SHAPES, dtype="bf16", B=1, L=32768,
        windows=(0, 128, 128, 128), seed=5, sampled_rows=256,
        note="hybrid GDLA block at the report's shapes (g=4, q_rank 1024; 1 full + 3 x W=128), bf16, B=1 L=32768"),
    "report_decode_b64": Workload(
        name="report_decode_b64", kind="decode", shapes=REPORT_SHAPES, dtype="bf16", B=64,
        windows=(0, 128), seed=6, ctx_range=(1024, 32768), capacity=32768,
        note="GDLA decode at the report's shapes (g=4, 80 query heads), bf16, batch 64, contexts U{1024..32768}"),
    "packed_hybrid_l32k": Workload(
        name="packed_hybrid_l32k", kind="packed", shapes=MOTIF_SHAPES, dtype="bf16", B=1, L=32768,
        windows=(0, 4096, 4096, 4096), seed=7, len_range=(256, 8192), sampled_rows=64,
        note="hybrid GDLA block over complete sequences of U{256..8192} tokens packed into one "
             "stream of 32768, bf16"),
    "paged_decode_b64": Workload(
        name="paged_decode_b64", kind="decode", shapes=MOTIF_SHAPES, dtype="bf16", B=64,
        windows=(0, 4096), seed=8, ctx_range=(1024, 32768), capacity=32768, page_rows=64,
        note="GDLA decode, bf16, batch 64, contexts U{1024..32768}, paged cache of 64-row pages in "
             "shuffled pool order"),
    "hybrid_l256k": Workload(
        name="hybrid_l256k", kind="block", shapes=MOTIF_SHAPES, dtype="bf16", B=1,
        L=262144, windows=(0, 4096, 4096, 4096), seed=4, sampled_rows=256,
        note="long-context hybrid GDLA block, bf16, B=1 L=262144"),
}


def layer_seed(w: Workload, layer: int) -> int:
    """Independent seed per layer of a block."""
    return w.seed * 100 + layer


def cfg_dict(w: Workload, window: int = 0) -> dict:
    """Layer options in the field names of the C header's config struct."""
    return dict(w.shapes, window=int(window), rope_base=w.rope_base, rms_eps=w.rms_eps)
