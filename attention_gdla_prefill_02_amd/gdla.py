"""ctypes binding of libgdla.so (the C ABI in include/gdla.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and non-OK statuses raise GdlaError with the
library's detail string.  Every step of the layer runs in the library's HIP
kernels; there is no fallback.  torch is used for device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdla.so")

GDLA_OK, GDLA_ERR_INVALID_ARG, GDLA_ERR_UNSUPPORTED, GDLA_ERR_WORKSPACE, GDLA_ERR_HIP = range(5)
GDLA_BF16, GDLA_FP32 = 0, 1
STAGE_DOWN, STAGE_PREP, STAGE_EXPAND, STAGE_QG, STAGE_ATTN, STAGE_OUT, STAGE_ALL = 1, 2, 4, 8, 16, 32, 63
EXPORTED = ("gdla_prefill_workspace_size", "gdla_prefill", "gdla_prefill_stages", "gdla_prefill_workspace_layout",
            "gdla_decode_workspace_size", "gdla_decode", "gdla_latent_expand", "gdla_status_string",
            "gdla_last_error", "gdla_version", "gdla_prefill_packed_workspace_size", "gdla_prefill_packed",
            "gdla_decode_paged", "gdla_backward_workspace_size", "gdla_backward", "gdla_decode_noalloc",
            "gdla_backward_packed_workspace_size", "gdla_backward_packed")
# bytes of the library-owned device array gdla_decode_noalloc uses as its workspace
DECODE_NOALLOC_SCRATCH_BYTES = 128 << 20


class GdlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status
        self.detail = detail


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("q_rank", ctypes.c_int32), ("kv_rank", ctypes.c_int32),
                ("n_noise", ctypes.c_int32), ("group", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int),
                ("yarn_factor", ctypes.c_float), ("yarn_orig_len", ctypes.c_int32),
                ("yarn_beta_fast", ctypes.c_float), ("yarn_beta_slow", ctypes.c_float),
                ("yarn_temperature", ctypes.c_int32)]


WEIGHT_FIELDS = ("w_dq", "g_q", "w_dkv", "g_kv", "w_lambda", "w_uq", "w_ukv", "w_gate", "w_o")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class PrefillLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("down", "cqn", "ckvn", "kr", "lam", "rope", "q", "gate", "kc", "vt", "z")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class PagedCache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("page_rows", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdla.so once (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m attention_gdla_prefill_02_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(Config)
    wp = ctypes.POINTER(Weights)
    lib.gdla_prefill_workspace_size.argtypes = [cfgp, i32, i32]
    lib.gdla_prefill_workspace_size.restype = sz
    lib.gdla_prefill.argtypes = [cfgp, wp, i32, i32, i64, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.gdla_prefill.restype = ctypes.c_int
    lib.gdla_prefill_stages.argtypes = [cfgp, wp, i32, i32, i64, vp, vp, vp, vp, i32, vp, sz, vp, ctypes.c_uint32]
    lib.gdla_prefill_stages.restype = ctypes.c_int
    lib.gdla_prefill_workspace_layout.argtypes = [cfgp, i32, i32, ctypes.POINTER(PrefillLayout)]
    lib.gdla_prefill_workspace_layout.restype = ctypes.c_int
    lib.gdla_decode_workspace_size.argtypes = [cfgp, i32]
    lib.gdla_decode_workspace_size.restype = sz
    lib.gdla_decode.argtypes = [cfgp, wp, i32, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.gdla_decode.restype = ctypes.c_int
    lib.gdla_decode_noalloc.argtypes = [cfgp, wp, i32, vp, vp, vp, vp, i32, vp]
    lib.gdla_decode_noalloc.restype = ctypes.c_int
    pcp = ctypes.POINTER(PagedCache)
    lib.gdla_prefill_packed_workspace_size.argtypes = [cfgp, i32, i64]
    lib.gdla_prefill_packed_workspace_size.restype = sz
    lib.gdla_prefill_packed.argtypes = [cfgp, wp, i32, i64, vp, vp, vp, vp, vp, pcp, vp, sz, vp]
    lib.gdla_prefill_packed.restype = ctypes.c_int
    lib.gdla_decode_paged.argtypes = [cfgp, wp, i32, vp, vp, pcp, vp, vp, sz, vp]
    lib.gdla_decode_paged.restype = ctypes.c_int
    lib.gdla_backward_workspace_size.argtypes = [cfgp, i32, i32]
    lib.gdla_backward_workspace_size.restype = sz
    lib.gdla_backward.argtypes = [cfgp, wp, i32, i32, i64, vp, vp, vp, ctypes.POINTER(Grads), vp, sz, vp]
    lib.gdla_backward.restype = ctypes.c_int
    lib.gdla_backward_packed_workspace_size.argtypes = [cfgp, i32, i64]
    lib.gdla_backward_packed_workspace_size.restype = sz
    lib.gdla_backward_packed.argtypes = [cfgp, wp, i32, i64, vp, vp, vp, vp, vp, ctypes.POINTER(Grads), vp, sz, vp]
    lib.gdla_backward_packed.restype = ctypes.c_int
    lib.gdla_latent_expand.argtypes = [cfgp, i64, vp, i64, vp, vp, vp, vp, vp, vp]
    lib.gdla_latent_expand.restype = ctypes.c_int
    lib.gdla_status_string.argtypes = [ctypes.c_int]
    lib.gdla_status_string.restype = ctypes.c_char_p
    lib.gdla_last_error.argtypes = []
    lib.gdla_last_error.restype = ctypes.c_char_p
    lib.gdla_version.argtypes = []
    lib.gdla_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != GDLA_OK:
        lib = load()
        raise GdlaError(status, f"{lib.gdla_status_string(status).decode()}: {lib.gdla_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


YARN_TEMPERATURES = {"rotary": 0, "logit": 1}


def make_config(shapes: dict, window: int = 0, dtype: str = "bf16", rope_base: float = 10000.0,
                rms_eps: float = 1e-6, yarn=None, yarn_temperature: str = "rotary") -> Config:
    """yarn: None, or (factor, orig_len, beta_fast, beta_slow); the library
    applies it on full-causal layers (window <= 0) only.  yarn_temperature:
    "rotary" (m on cos and sin) or "logit" (m^2 on the whole logit)."""
    yf, yl, ybf, ybs = (0.0, 0, 0.0, 0.0) if not yarn else yarn
    return Config(shapes["d_model"], shapes["q_rank"], shapes["kv_rank"], shapes["n_noise"], shapes["group"],
                  shapes["d_nope"], shapes["d_rope"], shapes["d_v"], int(window), float(rope_base),
                  float(rms_eps), GDLA_BF16 if dtype == "bf16" else GDLA_FP32,
                  float(yf), int(yl), float(ybf), float(ybs), YARN_TEMPERATURES[yarn_temperature])


def weights_struct(W: dict) -> Weights:
    return Weights(*[W[n].data_ptr() for n in WEIGHT_FIELDS])


def torch_dtype(cfg: Config):
    return torch.bfloat16 if cfg.dtype == GDLA_BF16 else torch.float32


def prefill_workspace_size(cfg: Config, B: int, L: int) -> int:
    return int(load().gdla_prefill_workspace_size(ctypes.byref(cfg), B, L))


def prefill_layout(cfg: Config, B: int, L: int) -> dict:
    out = PrefillLayout()
    _check(load().gdla_prefill_workspace_layout(ctypes.byref(cfg), B, L, ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in PrefillLayout._fields_}


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def prefill(cfg: Config, W: dict, x: torch.Tensor, *, y: torch.Tensor | None = None, residual=None, pos_offset=0,
            cache=None, workspace=None, stream=None, stages: int = STAGE_ALL, wstruct=None) -> torch.Tensor:
    """One GDLA layer: x [B, L, d_model] -> y [B, L, d_model] (device tensors).
    `stages` restricts the call to a subset of the layer's kernels."""
    B, L, _ = x.shape
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(prefill_workspace_size(cfg, B, L), x.device)
    cap = 0 if cache is None else cache.shape[1]
    ws = wstruct if wstruct is not None else weights_struct(W)
    _check(load().gdla_prefill_stages(ctypes.byref(cfg), ctypes.byref(ws), B, L, int(pos_offset),
                                      _ptr(x), _ptr(y), _ptr(residual), _ptr(cache), cap, _ptr(workspace),
                                      workspace.numel(), _stream(stream), int(stages)))
    return y


def decode_workspace_size(cfg: Config, B: int) -> int:
    return int(load().gdla_decode_workspace_size(ctypes.byref(cfg), B))


def decode(cfg: Config, W: dict, x: torch.Tensor, cache: torch.Tensor, cache_lens: torch.Tensor, *, y=None,
           workspace=None, stream=None) -> torch.Tensor:
    """One decode step: x [B, d_model] -> y [B, d_model]; writes row cache_lens[b] of each sequence."""
    B = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_size(cfg, B), x.device)
    _check(load().gdla_decode(ctypes.byref(cfg), ctypes.byref(weights_struct(W)), B, _ptr(x), _ptr(y), _ptr(cache),
                              _ptr(cache_lens), cache.shape[1], _ptr(workspace), workspace.numel(), _stream(stream)))
    return y


def decode_noalloc(cfg: Config, W: dict, x: torch.Tensor, cache: torch.Tensor, cache_lens: torch.Tensor, *,
                   y: torch.Tensor, stream=None) -> torch.Tensor:
    """gdla_decode with the library's own device scratch as workspace: nothing
    is allocated, so y must be given."""
    _check(load().gdla_decode_noalloc(ctypes.byref(cfg), ctypes.byref(weights_struct(W)), x.shape[0], _ptr(x),
                                      _ptr(y), _ptr(cache), _ptr(cache_lens), cache.shape[1], _stream(stream)))
    return y


def paged_cache(pages: torch.Tensor, block_table: torch.Tensor) -> PagedCache:
    """pages [num_pages, page_rows, kv_rank + d_rope]; block_table int32 [sequences, max_pages]."""
    return PagedCache(pages.data_ptr(), block_table.data_ptr(), pages.shape[1], block_table.shape[1],
                      pages.shape[0])


def prefill_packed_workspace_size(cfg: Config, n_seq: int, T: int) -> int:
    return int(load().gdla_prefill_packed_workspace_size(ctypes.byref(cfg), n_seq, T))


def prefill_packed(cfg: Config, W: dict, x: torch.Tensor, cu_seqlens: torch.Tensor, *, pos_offsets=None,
                   y=None, residual=None, pages=None, block_table=None, workspace=None, stream=None,
                   wstruct=None) -> torch.Tensor:
    """One GDLA layer over packed sequences: x [T, d_model] -> y [T, d_model].
    cu_seqlens, pos_offsets: device int32; pages / block_table: optional paged cache."""
    T = x.shape[0]
    n = cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(prefill_packed_workspace_size(cfg, n, T), x.device)
    pc = None if pages is None else ctypes.byref(paged_cache(pages, block_table))
    ws = wstruct if wstruct is not None else weights_struct(W)
    _check(load().gdla_prefill_packed(ctypes.byref(cfg), ctypes.byref(ws), n, T, _ptr(cu_seqlens),
                                      _ptr(pos_offsets), _ptr(x), _ptr(y), _ptr(residual), pc, _ptr(workspace),
                                      workspace.numel(), _stream(stream)))
    return y


def decode_paged(cfg: Config, W: dict, x: torch.Tensor, pages: torch.Tensor, block_table: torch.Tensor,
                 cache_lens: torch.Tensor, *, y=None, workspace=None, stream=None) -> torch.Tensor:
    """One decode step against a paged cache: x [B, d_model] -> y [B, d_model]."""
    B = x.shape[0]
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_size(cfg, B), x.device)
    pc = paged_cache(pages, block_table)
    _check(load().gdla_decode_paged(ctypes.byref(cfg), ctypes.byref(weights_struct(W)), B, _ptr(x), _ptr(y),
                                    ctypes.byref(pc), _ptr(cache_lens), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return y


def backward_workspace_size(cfg: Config, B: int, L: int) -> int:
    return int(load().gdla_backward_workspace_size(ctypes.byref(cfg), B, L))


def backward(cfg: Config, W: dict, x: torch.Tensor, dy: torch.Tensor, *, pos_offset=0, dx=None, grads=None,
             workspace=None, stream=None, wstruct=None):
    """Backward of one layer: returns (dx [B, L, d_model], dict of fp32 weight gradients)."""
    B, L, _ = x.shape
    if dx is None:
        dx = torch.empty_like(x)
    if grads is None:
        grads = {n: torch.empty(W[n].shape, dtype=torch.float32, device=x.device) for n in WEIGHT_FIELDS}
    if workspace is None:
        workspace = alloc_workspace(backward_workspace_size(cfg, B, L), x.device)
    gs = Grads(*[grads[n].data_ptr() for n in WEIGHT_FIELDS])
    ws = wstruct if wstruct is not None else weights_struct(W)
    _check(load().gdla_backward(ctypes.byref(cfg), ctypes.byref(ws), B, L, int(pos_offset), _ptr(x), _ptr(dy),
                                _ptr(dx), ctypes.byref(gs), _ptr(workspace), workspace.numel(), _stream(stream)))
    return dx, grads


def backward_packed_workspace_size(cfg: Config, n_seq: int, T: int) -> int:
    return int(load().gdla_backward_packed_workspace_size(ctypes.byref(cfg), n_seq, T))


def backward_packed(cfg: Config, W: dict, x: torch.Tensor, dy: torch.Tensor, cu_seqlens: torch.Tensor, *,
                    pos_offsets=None, dx=None, grads=None, workspace=None, stream=None, wstruct=None):
    """Backward of the layer over a packed stream: x, dy [T, d_model] (cu_seqlens,
    pos_offsets: device int32) -> (dx [T, d_model], dict of fp32 weight gradients)."""
    T = x.shape[0]
    n = cu_seqlens.numel() - 1
    if dx is None:
        dx = torch.empty_like(x)
    if grads is None:
        grads = {k: torch.empty(W[k].shape, dtype=torch.float32, device=x.device) for k in WEIGHT_FIELDS}
    if workspace is None:
        workspace = alloc_workspace(backward_packed_workspace_size(cfg, n, T), x.device)
    gs = Grads(*[grads[k].data_ptr() for k in WEIGHT_FIELDS])
    ws = wstruct if wstruct is not None else weights_struct(W)
    _check(load().gdla_backward_packed(ctypes.byref(cfg), ctypes.byref(ws), n, T, _ptr(cu_seqlens),
                                       _ptr(pos_offsets), _ptr(x), _ptr(dy), _ptr(dx), ctypes.byref(gs),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return dx, grads


def latent_expand(cfg: Config, c_kv: torch.Tensor, g_kv: torch.Tensor, w_ukv: torch.Tensor, stream=None):
    """c_kv [T, ld] -> (k_nope [T, nN, d_nope], v [T, nN, d_v], c_norm [T, kv_rank])."""
    T = c_kv.shape[0]
    dt, dev = c_kv.dtype, c_kv.device
    k = torch.empty((T, cfg.n_noise, cfg.d_nope), dtype=dt, device=dev)
    v = torch.empty((T, cfg.n_noise, cfg.d_v), dtype=dt, device=dev)
    cn = torch.empty((T, cfg.kv_rank), dtype=dt, device=dev)
    _check(load().gdla_latent_expand(ctypes.byref(cfg), T, _ptr(c_kv), c_kv.stride(0), _ptr(g_kv), _ptr(w_ukv),
                                     _ptr(k), _ptr(v), _ptr(cn), _stream(stream)))
    return k, v, cn


def hybrid_block(cfgs: list, Ws: list, x: torch.Tensor, workspace=None, stream=None) -> list:
    """A block of layers joined by x_{l+1} = x_l + y_l (the residual add is fused
    into each layer's output projection).  Returns [x_1, ..., x_n]."""
    B, L, _ = x.shape
    if workspace is None:
        workspace = alloc_workspace(max(prefill_workspace_size(c, B, L) for c in cfgs), x.device)
    outs = []
    cur = x
    for cfg, W in zip(cfgs, Ws):
        nxt = torch.empty_like(x)
        prefill(cfg, W, cur, y=nxt, residual=cur, workspace=workspace, stream=stream)
        outs.append(nxt)
        cur = nxt
    return outs
