"""GDLA oracle: a plain fp64 CPU implementation of the Grouped Differential
Latent Attention forward pass (one layer), its single-token decode form, and
the latent expansion.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
smoke check and the benchmark's CPU-baseline leg may import this module.  It
shares no code with the HIP library and imports nothing from it; the HIP path
never calls it.

Sources (cited by page title and paragraph; the summary page of the technical
report has no headings, so its paragraphs are named by topic):

  [M3-arch]  "Motif 3: Technical Report", architecture paragraph: a block is a
             GDLA layer then a sparse MoE layer; hybrid schedule of one full
             causal layer followed by three sliding-window layers; GDLA has a
             query-dependent output gate.
  [M3-gdla]  same page, GDLA summary paragraph: one normalization and one
             up-projection of the compressed KV latent; signal and noise paths
             differ only along the expanded head dimension; compact MLA-style
             inference state.
  [M3-eq]    same page, GDLA definition paragraph: low-rank query down/up
             projection; joint KV down-projection giving the latent and a
             decoupled rotary key; normalize-and-expand into shared content
             key / value heads; RoPE on rotary parts only; g times more signal
             heads than noise heads; lambda_t = sigmoid(x_t W_lambda), one per
             signal head; D_t = H_S,t - lambda_t * Repeat_g(H_N,t); sigmoid
             gate from the normalized query latent before the output
             projection.
  [M3-cfg]   same page, model-configuration paragraph (head counts, 192-dim
             query-key heads with a 64-dim rotary part, 128-dim values).
  [OSM-1]    "Open-Source Frontier Models: Architecture and Benchmarks of
             Rnj-1 and Motif-2", section 1 (full vs sliding-window attention):
             softmax(Q K^T / sqrt(d_k)) V; a sliding window lets each token
             see W previous tokens.
  [OSM-2]    same page, section 2 (YaRN): RoPE as a block-diagonal rotation
             with theta_i = b^(-2(i-1)/d).
  [OSM-impl] same page, implementation section: frequencies duplicated as
             cat(freqs, freqs) and the rotate-half application
             x*cos + rotate_half(x)*sin.
  [OSM-yarn] same page, section 2 and the implementation section: YaRN
             scales each rotary frequency by 1, 1/s or a ramp between them,
             chosen by its wavelength against the native context length over
             beta_fast and beta_slow, and corrects the softmax temperature by
             m = 1 + 0.1 ln s, which the listing multiplies into cos and sin.
  [M3-ctx]   "Motif 3: Technical Report", long-context paragraph: the
             full-attention layers extend the native 4K context by a factor of
             64 with YaRN; the sliding-window layers keep plain RoPE.
  [M3-pack]  same page, long-context training paragraph: training batches
             hold complete sequences packed together, which are re-balanced
             across data-parallel ranks by a longest-processing-time greedy
             rule.
  [M3-train] "Motif 3: Technical Report", training-infrastructure paragraph:
             activations are recomputed for the backward pass (selective
             recomputation, full recomputation at the longest lengths).
  [OSM-page] "Open-Source Frontier Models: Architecture and Benchmarks of
             Rnj-1 and Motif-2", section 2, prefill sequence diagram: the
             attention step stores the normalized KV rows in the blocks of a
             PagedAttention cache.

Readings where the pages are silent (each listed in the design notes):
RMSNorm with a learned gain for both latents; eps = cfg rms_eps; rotate-half
RoPE with theta_i = base^(-2i/d_rope), i = 0..d_rope/2-1, positions
p = pos_offset + t; the rotary part is the last d_rope dims of each query head;
one rotary key per token shared by every head; softmax scale
1/sqrt(d_nope + d_rope); query heads 0..nS-1 are signal, nS..H-1 are noise;
signal head j and noise head j//g both use KV head j//g; window W means keys
s with t - W < s <= t (W <= 0 or W >= L: full causal); no biases; weights are
[out, in] (y = x W^T); W_UKV rows are all content-key heads then all value
heads.  YaRN (when cfg.yarn_factor > 1, full-causal layers only): the
frequency table of the listing in [OSM-yarn]; its temperature m = 1 + 0.1 ln s
either multiplies cos and sin (cfg.yarn_temperature "rotary", the listing, the
default: the rotary part of every logit scales by m^2) or the whole logit by
m^2 ("logit": the page's prose puts the temperature on the softmax logits,
garbled as sqrt(1 + 0.1 ln s), and [M3-ctx] names the DeepSeek form of YaRN,
which scales the softmax by the square of the same m).
Packed sequences ([M3-pack]): sequence b of a packed stream holds rows
cu[b] .. cu[b+1]-1, its positions restart at pos_offsets[b], and its tokens
attend only to earlier tokens of the same sequence -- each sequence is the
layer applied to it alone.  Paged cache ([OSM-page]): the rows of one sequence
are cut into blocks of page_rows positions; block j of sequence b lives in
pool page block_table[b][j], so position p is row p mod page_rows of page
block_table[b][p div page_rows].

Every function works in float64 on whatever it is given (inputs are widened
with np.asarray(..., float64)); nothing is rounded to bf16 here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Cfg:
    """Layer shape and options (field names follow the C header)."""

    d_model: int
    q_rank: int
    kv_rank: int
    n_noise: int      # number of noise heads = number of expanded KV heads
    group: int        # g: signal heads per noise head
    d_nope: int
    d_rope: int
    d_v: int
    window: int = 0   # <= 0: full causal
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    yarn_factor: float = 0.0     # s; <= 1: plain RoPE
    yarn_orig_len: int = 4096    # native context length
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    # where YaRN's temperature m = 1 + 0.1 ln s goes: "rotary" multiplies cos
    # and sin by m (the listing of [OSM-yarn]; with the decoupled rotary part
    # only the rotary term of each logit scales, by m^2); "logit" multiplies
    # the whole logit by m^2 and leaves cos and sin unscaled (the prose of
    # [OSM-yarn] applies the temperature to the softmax logits, and [M3-ctx]
    # names the DeepSeek form of YaRN)
    yarn_temperature: str = "rotary"

    @property
    def n_signal(self) -> int:
        return self.group * self.n_noise

    @property
    def n_heads(self) -> int:
        return self.n_signal + self.n_noise

    @property
    def d_qk(self) -> int:
        return self.d_nope + self.d_rope


def _with_window(cfg: Cfg, window):
    return replace(cfg, window=int(window))


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Elementary pieces
# --------------------------------------------------------------------------

def linear(x, w):
    """y = x W^T with W stored [out, in] (the layout reading).  A plain
    matrix product; the library routine is the step."""
    return _f64(x) @ _f64(w).T


def rms_norm(c, gamma, eps):
    """RMSNorm over the last axis: c / sqrt(mean(c^2) + eps) * gamma.
    [M3-gdla] and [M3-eq] say the latents are normalized; the norm's kind is
    the reading above."""
    c = _f64(c)
    rms = np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    return c / rms * _f64(gamma)


def sigmoid(z):
    """Logistic function 1 / (1 + e^-z) ([M3-eq]: lambda and the gate)."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def rope_inv_freq(d_rope, base):
    """theta_i = base^(-2i/d_rope), i = 0..d_rope/2-1 ([OSM-2], written
    0-based; the same table the implementation section builds from
    arange(0, d, 2) / d)."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d_rope)


def yarn_inv_freq(d_rope, base, s, orig_len, beta_fast, beta_slow):
    """YaRN frequencies ([OSM-yarn]).  With lambda_i = 2 pi / theta_i the
    wavelength of pair i, the short-wavelength bound orig_len / beta_fast and
    the long one orig_len / beta_slow, ramp_i is lambda_i's position between
    the two bounds clamped to [0, 1], and the frequency becomes
    (1 - ramp_i) theta_i + ramp_i theta_i / s: unchanged below the short
    bound, divided by s above the long one."""
    theta = rope_inv_freq(d_rope, base)
    wavelength = 2.0 * math.pi / theta
    short, long_ = orig_len / beta_fast, orig_len / beta_slow
    ramp = np.clip((wavelength - short) / (long_ - short), 0.0, 1.0)
    return (1.0 - ramp) * theta + ramp * theta / s


def yarn_mscale(s):
    """The listing's temperature correction m = 1 + 0.1 ln s ([OSM-yarn])."""
    return 1.0 + 0.1 * math.log(s)


def yarn_active(cfg: Cfg) -> bool:
    """YaRN applies on full-causal layers only ([M3-ctx])."""
    return cfg.yarn_factor > 1.0 and cfg.window <= 0


def rope_params(cfg: Cfg):
    """(base, yarn) for rope(): yarn is None for plain RoPE, else
    (s, orig_len, beta_fast, beta_slow, m) with m the cos/sin multiplier:
    yarn_mscale(s) for the "rotary" temperature, 1 for "logit"."""
    if yarn_active(cfg):
        m = yarn_mscale(cfg.yarn_factor) if cfg.yarn_temperature == "rotary" else 1.0
        return cfg.rope_base, (float(cfg.yarn_factor), float(cfg.yarn_orig_len),
                               float(cfg.yarn_beta_fast), float(cfg.yarn_beta_slow), m)
    return cfg.rope_base, None


def logit_scale(cfg: Cfg) -> float:
    """Multiplier of q . k in the softmax: 1/sqrt(d_qk) ([OSM-1]), times m^2
    on a YaRN layer with the "logit" temperature ([OSM-yarn])."""
    scale = 1.0 / math.sqrt(cfg.d_qk)
    if yarn_active(cfg) and cfg.yarn_temperature == "logit":
        scale *= yarn_mscale(cfg.yarn_factor) ** 2
    return scale


def _yarn_table(d, base, yarn):
    """(frequencies, cos/sin multiplier) of a rope() yarn argument: None, or
    (s, orig_len, beta_fast, beta_slow[, m]); m defaults to yarn_mscale(s)."""
    if yarn is None:
        return rope_inv_freq(d, base), 1.0
    s_, orig, bf, bs = yarn[:4]
    m = yarn[4] if len(yarn) > 4 else yarn_mscale(s_)
    return yarn_inv_freq(d, base, s_, orig, bf, bs), m


def rope(u, pos, base, yarn=None):
    """Rotate-half RoPE ([OSM-impl]) of u[..., T, d_rope] at positions pos[T].

    For each i < d_rope/2 the pair (u_i, u_{i+d/2}) is rotated by angle
    pos * theta_i:  u_i' = u_i cos - u_{i+d/2} sin,
                    u_{i+d/2}' = u_{i+d/2} cos + u_i sin.
    With yarn = (s, orig_len, beta_fast, beta_slow[, m]) the frequencies are
    YaRN's and cos, sin carry the factor m (default 1 + 0.1 ln s, [OSM-yarn]).
    """
    u = _f64(u)
    d = u.shape[-1]
    half = d // 2
    inv, m = _yarn_table(d, base, yarn)
    ang = _f64(pos)[:, None] * inv[None, :]      # [T, d/2]
    cos, sin = m * np.cos(ang), m * np.sin(ang)
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * cos - u2 * sin, u2 * cos + u1 * sin], axis=-1)


def kv_head_of(h, cfg: Cfg):
    """KV head used by query head h: j // g for signal head j, h - nS for
    noise head h ([M3-eq]: the expanded heads are shared by both paths; the
    pairing j -> j // g is the Repeat_g reading)."""
    return h // cfg.group if h < cfg.n_signal else h - cfg.n_signal


def attended_keys(t, window):
    """Keys position t may attend: max(0, t-W+1) .. t ([OSM-1]); W <= 0 is
    full causal ([M3-arch])."""
    lo = 0 if window <= 0 else max(0, t - window + 1)
    return lo, t + 1


# --------------------------------------------------------------------------
# Latent expansion ([M3-gdla], [M3-eq])
# --------------------------------------------------------------------------

def latent_expand(c_kv, g_kv, w_ukv, cfg: Cfg):
    """c_KVn = RMSNorm(c_KV); [K^C | V] = c_KVn W_UKV^T split into n_noise
    content-key heads [.., n_noise, d_nope] and value heads [.., n_noise, d_v].
    Returns (k_nope, v, c_norm)."""
    c_norm = rms_norm(c_kv, g_kv, cfg.rms_eps)
    kv = linear(c_norm, w_ukv)
    nk = cfg.n_noise * cfg.d_nope
    lead = kv.shape[:-1]
    k_nope = kv[..., :nk].reshape(*lead, cfg.n_noise, cfg.d_nope)
    v = kv[..., nk:].reshape(*lead, cfg.n_noise, cfg.d_v)
    return k_nope, v, c_norm


# --------------------------------------------------------------------------
# Per-token projections shared by prefill and decode ([M3-eq])
# --------------------------------------------------------------------------

def kv_tokens(x, W, cfg: Cfg, pos):
    """KV side of each token ([M3-eq], [M3-gdla]): the joint down-projection
    [c_KV | k_R] = x W_DKV^T, c_KVn = RMSNorm(c_KV), k_R <- RoPE(k_R, pos).
    x [T, d_model], pos [T].  Returns (ckvn [T, kv_rank], kr [T, d_rope])."""
    ckv_kr = linear(x, W["w_dkv"])
    ckvn = rms_norm(ckv_kr[:, :cfg.kv_rank], W["g_kv"], cfg.rms_eps)
    kr = rope(ckv_kr[:, cfg.kv_rank:], pos, *rope_params(cfg))
    return ckvn, kr


def query_tokens(x, W, cfg: Cfg, pos):
    """Query side of each token ([M3-eq]): c_Qn = RMSNorm(x W_DQ^T),
    q = c_Qn W_UQ^T with RoPE on the last d_rope dims of every head,
    lambda = sigmoid(x W_lambda^T), gate = sigmoid(c_Qn W_G^T).
    x [T, d_model], pos [T].  Returns dict cqn, q [T, H, d_qk], lam, gate."""
    T = x.shape[0]
    cqn = rms_norm(linear(x, W["w_dq"]), W["g_q"], cfg.rms_eps)
    q = linear(cqn, W["w_uq"]).reshape(T, cfg.n_heads, cfg.d_qk)
    q_rot = rope(np.transpose(q[:, :, cfg.d_nope:], (1, 0, 2)), pos, *rope_params(cfg))
    q = np.concatenate([q[:, :, :cfg.d_nope], np.transpose(q_rot, (1, 0, 2))], axis=-1)
    lam = sigmoid(linear(x, W["w_lambda"]))
    gate = sigmoid(linear(cqn, W["w_gate"]))
    return dict(cqn=cqn, q=q, lam=lam, gate=gate)


def project_tokens(x, W, cfg: Cfg, pos):
    """Both per-token halves: dict cqn, q, ckvn, kr, lam, gate."""
    x = _f64(x)
    ckvn, kr = kv_tokens(x, W, cfg, pos)
    out = query_tokens(x, W, cfg, pos)
    out.update(ckvn=ckvn, kr=kr)
    return out


def differential_gate_out(Hs, Hn, lam, gate, w_o, cfg: Cfg):
    """D_j = H_S,j - lambda_j * H_N,j//g; Z = gate * vec(D); y = Z W_O^T.
    Hs [R, nS, d_v], Hn [R, nN, d_v], lam [R, nS], gate [R, nS*d_v].
    ([M3-eq]; D's definition and the gate before the output projection.)"""
    rep = np.repeat(Hn, cfg.group, axis=1)                 # Repeat_g: j -> j//g
    D = Hs - lam[:, :, None] * rep
    Z = gate * D.reshape(D.shape[0], -1)
    y = linear(Z, w_o)
    return y, Z, D


# --------------------------------------------------------------------------
# Prefill: one GDLA layer over [B, L] tokens
# --------------------------------------------------------------------------

def _consecutive_runs(rows, max_len):
    """Split a sorted row list into runs of consecutive positions (at most
    max_len long); each run shares one key range.  Pure iteration order: every
    row is still computed on its own."""
    runs, cur = [], []
    for r in rows:
        if cur and (r != cur[-1] + 1 or len(cur) == max_len):
            runs.append(cur)
            cur = []
        cur.append(r)
    if cur:
        runs.append(cur)
    return runs


def attention_heads(q, kc, kr, v, rows, cfg: Cfg, scale=None):
    """Per-head causal / sliding-window softmax attention ([OSM-1], [M3-eq]).

    q [R, H, d_qk] for query positions `rows`; kc [L, nN, d_nope]; kr [L, d_rope]
    (one rotary key per token, shared by all heads); v [L, nN, d_v].
    H[r, h] = sum_{s in A(t)} softmax_s(scale q_h . [k^C_n,s | k_R,s]) v_n,s
    with n = kv_head_of(h), A(t) = attended_keys(t, window), scale =
    logit_scale(cfg) unless given.
    """
    if scale is None:
        scale = logit_scale(cfg)
    out = np.zeros((len(rows), cfg.n_heads, cfg.d_v))
    index = {t: i for i, t in enumerate(rows)}
    runs = _consecutive_runs(rows, 128)
    for n in range(cfg.n_noise):
        heads = [h for h in range(cfg.n_heads) if kv_head_of(h, cfg) == n]
        k = np.concatenate([kc[:, n, :], kr], axis=-1)                 # [L, d_qk], KV head n
        for run in runs:
            lo_run = attended_keys(run[0], cfg.window)[0]
            hi_run = run[-1] + 1
            spos = np.arange(lo_run, hi_run)
            tpos = np.array(run)
            lo_t = np.array([attended_keys(t, cfg.window)[0] for t in run])
            allowed = (spos[None, :] <= tpos[:, None]) & (spos[None, :] >= lo_t[:, None])
            idx = [index[t] for t in run]
            R_, G_ = len(run), len(heads)
            qg = q[idx][:, heads, :].reshape(R_ * G_, cfg.d_qk)           # rows (t, head)
            s = ((qg @ k[lo_run:hi_run].T) * scale).reshape(R_, G_, -1)  # [run, heads, S]
            s = np.where(allowed[:, None, :], s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=-1, keepdims=True)
            o = w.reshape(R_ * G_, -1) @ v[lo_run:hi_run, n, :]
            out[np.ix_(idx, heads)] = o.reshape(R_, G_, cfg.d_v)
    return out


def gdla_layer(x, W, cfg: Cfg, pos_offset=0, rows=None, lam_override=None):
    """One GDLA layer, [M3-eq] steps in order.

    x      [B, L, d_model]
    W      dict of weights (names as in the C header)
    rows   optional sorted list of query positions to evaluate (the same for
           every sequence); keys and values are still built for every position
    lam_override  optional constant replacing lambda (special-case checks)

    Returns dict: y [B, R, d_model], Z [B, R, nS*d_v], H [B, R, H, d_v]
    (per-head attention outputs before the difference), cache
    [B, L, kv_rank + d_rope] (normalized latent | RoPE'd rotary key),
    lam [B, R, nS], and the row list used.
    """
    x = _f64(x)
    B, L, _ = x.shape
    R = list(range(L)) if rows is None else sorted(int(r) for r in rows)
    pos = pos_offset + np.arange(L, dtype=np.float64)
    ys, Zs, Hs_all, caches, lams = [], [], [], [], []
    for b in range(B):
        # keys and values for every position; the query path only for rows R
        ckvn, kr = kv_tokens(x[b], W, cfg, pos)
        kc, v, _ = latent_expand_from_norm(ckvn, W["w_ukv"], cfg)
        qp = query_tokens(x[b, R], W, cfg, pos[R])
        Hh = attention_heads(qp["q"], kc, kr, v, R, cfg)
        lam = qp["lam"]
        if lam_override is not None:
            lam = np.full_like(lam, float(lam_override))
        y, Z, _ = differential_gate_out(Hh[:, :cfg.n_signal], Hh[:, cfg.n_signal:],
                                        lam, qp["gate"], W["w_o"], cfg)
        ys.append(y)
        Zs.append(Z)
        Hs_all.append(Hh)
        lams.append(lam)
        caches.append(np.concatenate([ckvn, kr], axis=-1))
    return dict(y=np.stack(ys), Z=np.stack(Zs), H=np.stack(Hs_all),
                cache=np.stack(caches), lam=np.stack(lams), rows=R)


def latent_expand_from_norm(ckvn, w_ukv, cfg: Cfg):
    """[K^C | V] = c_KVn W_UKV^T for an already-normalized latent (the cache
    holds normalized rows, so decode expands without renormalizing)."""
    kv = linear(ckvn, w_ukv)
    nk = cfg.n_noise * cfg.d_nope
    lead = kv.shape[:-1]
    return (kv[..., :nk].reshape(*lead, cfg.n_noise, cfg.d_nope),
            kv[..., nk:].reshape(*lead, cfg.n_noise, cfg.d_v), ckvn)


# --------------------------------------------------------------------------
# Decode: one new token per sequence against the compressed cache
# --------------------------------------------------------------------------

def gdla_decode(x_new, W, cfg: Cfg, cache, cache_lens):
    """One decode step ([M3-gdla]: only the normalized latent and rotary key
    are kept per position).

    x_new       [B, d_model]  the new token of each sequence
    cache       [B, capacity, kv_rank + d_rope] rows [c_KVn | RoPE(k_R)]
    cache_lens  [B] tokens already cached; the new token sits at that position

    The new token's row is appended first, then every attended cached row is
    expanded plainly (k^C = W_UK,n c, v = W_UV,n c) and steps 7-10 run for
    the one query.  Returns dict y [B, d_model], Z [B, nS*d_v], new_rows
    [B, kv_rank + d_rope].
    """
    x_new = _f64(x_new)
    cache = _f64(cache)
    B = x_new.shape[0]
    ys, Zs, rows_out = [], [], []
    for b in range(B):
        p_b = int(cache_lens[b])
        pr = project_tokens(x_new[b:b + 1], W, cfg, np.array([p_b], dtype=np.float64))
        new_row = np.concatenate([pr["ckvn"][0], pr["kr"][0]])
        lo, hi = attended_keys(p_b, cfg.window)
        rows = np.array(cache[b, lo:hi])
        rows[hi - 1 - lo] = new_row                      # the appended row
        kc, v, _ = latent_expand_from_norm(rows[:, :cfg.kv_rank], W["w_ukv"], cfg)
        kr = rows[:, cfg.kv_rank:]
        # keys are indexed relative to lo, so the query sits at hi-1-lo
        Hh = attention_heads(pr["q"], kc, kr, v, [hi - 1 - lo],
                             _with_window(cfg, 0), scale=logit_scale(cfg))[0]
        y, Z, _ = differential_gate_out(Hh[None, :cfg.n_signal], Hh[None, cfg.n_signal:],
                                        pr["lam"], pr["gate"], W["w_o"], cfg)
        ys.append(y[0])
        Zs.append(Z[0])
        rows_out.append(new_row)
    return dict(y=np.stack(ys), Z=np.stack(Zs), new_rows=np.stack(rows_out))


# --------------------------------------------------------------------------
# Packed variable-length prefill ([M3-pack]) and the paged cache ([OSM-page])
# --------------------------------------------------------------------------

def packed_segments(cu_seqlens):
    """[(start, end)] row ranges of the packed sequences: sequence b holds rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 of the stream."""
    cu = [int(c) for c in cu_seqlens]
    return [(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]


def gdla_layer_packed(x, W, cfg: Cfg, cu_seqlens, pos_offsets=None):
    """One GDLA layer over complete sequences packed end to end.

    x            [T, d_model], the sequences one after another
    cu_seqlens   [n+1] row offsets (cu[0] = 0, cu[n] = T)
    pos_offsets  [n] position of each sequence's first token (default 0)

    Each sequence is the layer applied to it alone: its rows attend only to
    earlier rows of the same sequence, at positions pos_offsets[b] + i.
    Returns dict y [T, d_model], Z [T, nS*d_v], cache [T, kv_rank + d_rope]
    (the row each token would store) and lam [T, nS].
    """
    x = _f64(x)
    T = x.shape[0]
    segs = packed_segments(cu_seqlens)
    if pos_offsets is None:
        pos_offsets = [0] * len(segs)
    RL = cfg.kv_rank + cfg.d_rope
    y = np.zeros((T, cfg.d_model))
    Z = np.zeros((T, cfg.n_signal * cfg.d_v))
    cache = np.zeros((T, RL))
    lam = np.zeros((T, cfg.n_signal))
    for (s0, s1), p0 in zip(segs, pos_offsets):
        if s1 <= s0:
            continue
        r = gdla_layer(x[None, s0:s1], W, cfg, pos_offset=int(p0))
        y[s0:s1] = r["y"][0]
        Z[s0:s1] = r["Z"][0]
        cache[s0:s1] = r["cache"][0]
        lam[s0:s1] = r["lam"][0]
    return dict(y=y, Z=Z, cache=cache, lam=lam)


def paged_slot(block_table, page_rows, b, p):
    """(page, row) that holds position p of sequence b."""
    return int(block_table[b][p // page_rows]), p % page_rows


def paged_rows(pages, block_table, page_rows, b, n_rows):
    """Rows 0 .. n_rows-1 of sequence b read out of a paged cache
    pages [num_pages, page_rows, kv_rank + d_rope]."""
    pages = _f64(pages)
    out = np.zeros((n_rows, pages.shape[-1]))
    for p in range(n_rows):
        pg, r = paged_slot(block_table, page_rows, b, p)
        out[p] = pages[pg, r]
    return out


def paged_write(pages, block_table, page_rows, b, positions, rows):
    """Copy of the pool with rows stored at the given positions of sequence b."""
    out = np.array(_f64(pages))
    for p, row in zip(positions, _f64(rows)):
        pg, r = paged_slot(block_table, page_rows, b, int(p))
        out[pg, r] = row
    return out


def gdla_decode_paged(x_new, W, cfg: Cfg, pages, block_table, page_rows, cache_lens):
    """One decode step against a paged cache: each sequence's cached rows are
    read through its block table, then the step is gdla_decode's.  Returns
    gdla_decode's dict plus `slots`, the (page, row) each new row goes to."""
    B = len(cache_lens)
    RL = cfg.kv_rank + cfg.d_rope
    cap = int(max(cache_lens)) + 1
    dense = np.zeros((B, cap, RL))
    for b in range(B):
        n = int(cache_lens[b])
        dense[b, :n] = paged_rows(pages, block_table, page_rows, b, n)
    out = gdla_decode(x_new, W, cfg, dense, cache_lens)
    out["slots"] = [paged_slot(block_table, page_rows, b, int(cache_lens[b])) for b in range(B)]
    return out


# --------------------------------------------------------------------------
# Backward of one layer ([M3-train]: training recomputes the forward's
# activations; the gradient is the chain rule of the steps above, taken in
# reverse order)
# --------------------------------------------------------------------------

def rms_norm_backward(c, gamma, eps, g):
    """Gradients of y = c r gamma, r = (mean(c^2) + eps)^(-1/2), for upstream
    g = dL/dy: dc = r (g gamma) - c r^3 mean((g gamma) c), dgamma = sum over
    rows of g c r."""
    c, g = _f64(c), _f64(g)
    n = c.shape[-1]
    r = 1.0 / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    u = g * _f64(gamma)
    dc = r * u - c * r ** 3 * np.sum(u * c, axis=-1, keepdims=True) / n
    dgamma = np.sum((g * c * r).reshape(-1, n), axis=0)
    return dc, dgamma


def rope_backward(g, pos, base, yarn=None):
    """Gradient through rope(): the transpose of the pairwise rotation (scaled
    by m with YaRN), i.e. rotation by the opposite angle."""
    g = _f64(g)
    d = g.shape[-1]
    half = d // 2
    inv, m = _yarn_table(d, base, yarn)
    ang = _f64(pos)[:, None] * inv[None, :]
    cos, sin = m * np.cos(ang), m * np.sin(ang)
    g1, g2 = g[..., :half], g[..., half:]
    return np.concatenate([g1 * cos + g2 * sin, g2 * cos - g1 * sin], axis=-1)


def attention_heads_backward(q, kc, kr, v, dH, cfg: Cfg, rows=None):
    """Gradients of attention_heads for upstream dH [R, H, d_v] on the query
    rows `rows` (default: every row 0..L-1; q holds those rows' queries):
    per head, P = softmax(S) with S = q k^T / sqrt(d_qk) masked, O = P v;
    dv += P^T dO, dP = dO v^T, dS = P (dP - rowsum(dP P)), dq = dS k / sqrt(d_qk),
    dk += dS^T q / sqrt(d_qk).  k = [k^C_n | k_R]: the content part of dk goes
    to KV head n, the rotary part (one k_R per token) collects every head.
    Rows outside `rows` have zero upstream gradient.  Returns dq [R, H, d_qk],
    dkc [L, nN, d_nope], dkr [L, d_rope], dv [L, nN, d_v]."""
    L = kc.shape[0]
    R = np.arange(L) if rows is None else np.asarray(rows)
    scale = logit_scale(cfg)
    dq = np.zeros_like(_f64(q))
    dkc = np.zeros((L, cfg.n_noise, cfg.d_nope))
    dkr = np.zeros((L, cfg.d_rope))
    dv = np.zeros((L, cfg.n_noise, cfg.d_v))
    t = np.arange(L)
    lo = np.array([attended_keys(int(i), cfg.window)[0] for i in R])
    allowed = (t[None, :] <= R[:, None]) & (t[None, :] >= lo[:, None])
    for h in range(cfg.n_heads):
        n = kv_head_of(h, cfg)
        k = np.concatenate([kc[:, n, :], kr], axis=-1)
        s = np.where(allowed, (q[:, h, :] @ k.T) * scale, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        P = np.exp(s)
        P /= P.sum(axis=-1, keepdims=True)
        dO = dH[:, h, :]
        dv[:, n, :] += P.T @ dO
        dP = dO @ v[:, n, :].T
        dS = P * (dP - np.sum(dP * P, axis=-1, keepdims=True))
        dq[:, h, :] = (dS @ k) * scale
        dk = (dS.T @ q[:, h, :]) * scale
        dkc[:, n, :] += dk[:, :cfg.d_nope]
        dkr += dk[:, cfg.d_nope:]
    return dq, dkc, dkr, dv


def gdla_layer_backward(x, W, cfg: Cfg, dy, pos_offset=0, rows=None):
    """Gradients of one GDLA layer's output y (gdla_layer) with respect to its
    input and every weight, for upstream dy [B, L, d_model] -- or, with
    `rows` (a sorted list of positions, the same for every sequence), dy
    [B, R, d_model] on those rows and zero elsewhere.  The forward's
    activations are recomputed from x, then the steps are differentiated in
    reverse: output projection, gate and differential, attention, query
    up-projection with RoPE, latent expansion, the two RMSNorms, RoPE of the
    rotary key, and the fused down-projection.  The query path is evaluated
    only on the rows with a gradient (every other row's query-side gradient is
    zero); the key/value path on every row.  Returns dict dx [B, L, d_model]
    and one entry per weight name (same shapes as the weights)."""
    x, dy = _f64(x), _f64(dy)
    B, L, _ = x.shape
    R = list(range(L)) if rows is None else sorted(int(r) for r in rows)
    nR = len(R)
    nS, nN, g = cfg.n_signal, cfg.n_noise, cfg.group
    grads = {k: np.zeros_like(_f64(v)) for k, v in W.items()}
    dx = np.zeros_like(x)
    base, yarn = rope_params(cfg)
    for b in range(B):
        xb, dyb = x[b], dy[b]
        xr = xb[R]
        pos = pos_offset + np.arange(L, dtype=np.float64)
        # recompute the forward: keys and values on every row, queries on rows R
        ckv_kr = linear(xb, W["w_dkv"])
        c_kv, kr_raw = ckv_kr[:, :cfg.kv_rank], ckv_kr[:, cfg.kv_rank:]
        ckvn = rms_norm(c_kv, W["g_kv"], cfg.rms_eps)
        kr = rope(kr_raw, pos, base, yarn)
        kc, v, _ = latent_expand_from_norm(ckvn, W["w_ukv"], cfg)
        cq = linear(xr, W["w_dq"])
        cqn = rms_norm(cq, W["g_q"], cfg.rms_eps)
        qf = linear(cqn, W["w_uq"]).reshape(nR, cfg.n_heads, cfg.d_qk)
        q_rot = rope(np.transpose(qf[:, :, cfg.d_nope:], (1, 0, 2)), pos[R], base, yarn)
        q = np.concatenate([qf[:, :, :cfg.d_nope], np.transpose(q_rot, (1, 0, 2))], axis=-1)
        lam = sigmoid(linear(xr, W["w_lambda"]))
        gate = sigmoid(linear(cqn, W["w_gate"]))
        Hh = attention_heads(q, kc, kr, v, R, cfg)
        Hs, Hn = Hh[:, :nS], Hh[:, nS:]
        D = Hs - lam[:, :, None] * np.repeat(Hn, g, axis=1)
        Z = gate * D.reshape(nR, -1)
        # output projection
        grads["w_o"] += dyb.T @ Z
        dZ = dyb @ _f64(W["w_o"])
        # gate and differential
        dgate = dZ * D.reshape(nR, -1)
        dD = (dZ * gate).reshape(nR, nS, cfg.d_v)
        dlam = -np.sum(dD * np.repeat(Hn, g, axis=1), axis=-1)
        dHn = -np.sum((lam[:, :, None] * dD).reshape(nR, nN, g, cfg.d_v), axis=2)
        dH = np.concatenate([dD, dHn], axis=1)
        # attention
        dq, dkc, dkr, dv = attention_heads_backward(q, kc, kr, v, dH, cfg, rows=R)
        # query side: RoPE on the rotary parts, W_UQ, the gate, RMSNorm, W_DQ
        dq_rot = rope_backward(np.transpose(dq[:, :, cfg.d_nope:], (1, 0, 2)), pos[R], base, yarn)
        dqf = np.concatenate([dq[:, :, :cfg.d_nope], np.transpose(dq_rot, (1, 0, 2))], axis=-1).reshape(nR, -1)
        grads["w_uq"] += dqf.T @ cqn
        dcqn = dqf @ _f64(W["w_uq"])
        dglogit = dgate * gate * (1.0 - gate)
        grads["w_gate"] += dglogit.T @ cqn
        dcqn += dglogit @ _f64(W["w_gate"])
        dcq, dgq = rms_norm_backward(cq, W["g_q"], cfg.rms_eps, dcqn)
        grads["g_q"] += dgq
        grads["w_dq"] += dcq.T @ xr
        dxr = dcq @ _f64(W["w_dq"])
        # lambda
        dllogit = dlam * lam * (1.0 - lam)
        grads["w_lambda"] += dllogit.T @ xr
        dxr += dllogit @ _f64(W["w_lambda"])
        # KV side: expansion, RMSNorm, RoPE of the rotary key, W_DKV
        dkv = np.concatenate([dkc.reshape(L, -1), dv.reshape(L, -1)], axis=-1)
        grads["w_ukv"] += dkv.T @ ckvn
        dckvn = dkv @ _f64(W["w_ukv"])
        dckv, dgkv = rms_norm_backward(c_kv, W["g_kv"], cfg.rms_eps, dckvn)
        grads["g_kv"] += dgkv
        dkr_raw = rope_backward(dkr, pos, base, yarn)
        dckv_kr = np.concatenate([dckv, dkr_raw], axis=-1)
        grads["w_dkv"] += dckv_kr.T @ xb
        dxb = dckv_kr @ _f64(W["w_dkv"])
        dxb[R] += dxr
        dx[b] = dxb
    return dict(dx=dx, **grads)


def gdla_layer_packed_backward(x, W, cfg: Cfg, dy, cu_seqlens, pos_offsets=None):
    """Backward of gdla_layer_packed ([M3-pack] streams in the training pass of
    [M3-train]): every sequence of the stream is the layer applied to it
    alone, so its rows of dx are that sequence's dx and each weight gradient
    is the sum of the sequences' gradients.  x, dy [T, d_model]; returns dict
    dx [T, d_model] and one entry per weight name."""
    x, dy = _f64(x), _f64(dy)
    segs = packed_segments(cu_seqlens)
    if pos_offsets is None:
        pos_offsets = [0] * len(segs)
    grads = {k: np.zeros_like(_f64(v)) for k, v in W.items()}
    dx = np.zeros_like(x)
    for (s0, s1), p0 in zip(segs, pos_offsets):
        if s1 <= s0:
            continue
        g = gdla_layer_backward(x[None, s0:s1], W, cfg, dy[None, s0:s1], pos_offset=int(p0))
        dx[s0:s1] = g["dx"][0]
        for k in grads:
            grads[k] += g[k]
    return dict(dx=dx, **grads)


# --------------------------------------------------------------------------
# Hybrid block ([M3-arch]): 1 full-causal layer then 3 sliding-window layers
# --------------------------------------------------------------------------

def hybrid_windows(n_layers, window):
    """Window of each layer in a hybrid block: layer 0 of every group of four
    is full causal (0), the other three use `window`."""
    return [0 if (l % 4) == 0 else int(window) for l in range(n_layers)]


def gdla_block(x, Ws, cfg: Cfg, window):
    """A plain residual stand-in joins the layers: x_{l+1} = x_l + y_l (the
    pages' hyper-connections are another component).  Returns the list of
    per-layer outputs and the final stream."""
    x = _f64(x)
    outs = []
    for l, (W, win) in enumerate(zip(Ws, hybrid_windows(len(Ws), window))):
        y = gdla_layer(x, W, _with_window(cfg, win))["y"]
        outs.append(y)
        x = x + y
    return outs, x
