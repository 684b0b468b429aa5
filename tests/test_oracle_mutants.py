"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin catches each of them; this shows the pins constrain every part
of the oracle rather than restating it."""

import math

import numpy as np
import pytest

import oracle.gdla_ref as R
from tests import oracle_pins as P

# unpatched oracle functions, for mutants built on top of them
_ORIG = {name: getattr(R, name) for name in ("rope", "attention_heads_backward")}


def _rope_wrong_sign(u, pos, base, yarn=None):
    u = np.asarray(u, np.float64)
    half = u.shape[-1] // 2
    ang = np.asarray(pos, np.float64)[:, None] * R.rope_inv_freq(u.shape[-1], base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    u1, u2 = u[..., :half], u[..., half:]
    return np.concatenate([u1 * c + u2 * s, u2 * c - u1 * s * 0.5], axis=-1)


def _rope_adjacent_pairs(u, pos, base, yarn=None):
    u = np.asarray(u, np.float64)
    d = u.shape[-1]
    ang = np.asarray(pos, np.float64)[:, None] * R.rope_inv_freq(d, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _inv_freq_wrong(d, base):
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -1.0 * i / d)


def _kv_head_modulo(h, cfg):
    return h % cfg.n_noise if h < cfg.n_signal else h - cfg.n_signal


def _window_off_by_one(t, window):
    lo = 0 if window <= 0 else max(0, t - window)
    return lo, t + 1


def _not_causal(t, window):
    return 0, t + 2


def _diff_one_minus_lambda(Hs, Hn, lam, gate, w_o, cfg):
    rep = np.repeat(Hn, cfg.group, axis=1)
    D = Hs - (1.0 - lam)[:, :, None] * rep
    Z = gate * D.reshape(D.shape[0], -1)
    return R.linear(Z, w_o), Z, D


def _diff_tile_not_repeat(Hs, Hn, lam, gate, w_o, cfg):
    rep = np.tile(Hn, (1, cfg.group, 1))
    D = Hs - lam[:, :, None] * rep
    Z = gate * D.reshape(D.shape[0], -1)
    return R.linear(Z, w_o), Z, D


def _diff_no_gate(Hs, Hn, lam, gate, w_o, cfg):
    rep = np.repeat(Hn, cfg.group, axis=1)
    D = Hs - lam[:, :, None] * rep
    Z = D.reshape(D.shape[0], -1)
    return R.linear(Z, w_o), Z, D


def _rms_no_eps_sqrt(c, gamma, eps):
    c = np.asarray(c, np.float64)
    return c / (np.mean(c * c, axis=-1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def _sigmoid_tanh_wrong(z):
    return 0.5 * (1.0 + np.tanh(np.asarray(z, np.float64)))


_orig_query = R.query_tokens
_orig_kv = R.kv_tokens


def _gate_from_raw_latent(x, W, cfg, pos):
    out = _orig_query(x, W, cfg, pos)
    cq = R.linear(x, W["w_dq"])
    out["gate"] = R.sigmoid(R.linear(cq, W["w_gate"]))
    return out


def _key_not_roped(x, W, cfg, pos):
    ckvn, _ = _orig_kv(x, W, cfg, pos)
    return ckvn, R.linear(x, W["w_dkv"])[:, cfg.kv_rank:]


def _kv_not_normalized(x, W, cfg, pos):
    _, kr = _orig_kv(x, W, cfg, pos)
    return R.linear(x, W["w_dkv"])[:, :cfg.kv_rank] * np.asarray(W["g_kv"], np.float64), kr


def _query_rope_on_content(x, W, cfg, pos):
    out = _orig_query(x, W, cfg, pos)
    q = out["q"]
    # rotate the first d_rope dims (content) instead of the last ones
    rot = R.rope(np.transpose(q[:, :, :cfg.d_rope], (1, 0, 2)), pos, cfg.rope_base)
    raw = R.linear(R.rms_norm(R.linear(x, W["w_dq"]), W["g_q"], cfg.rms_eps), W["w_uq"]).reshape(q.shape)
    out["q"] = np.concatenate([np.transpose(R.rope(np.transpose(raw[:, :, :cfg.d_rope], (1, 0, 2)), pos, cfg.rope_base), (1, 0, 2)),
                               raw[:, :, cfg.d_rope:]], axis=-1)
    del rot
    return out


_orig_attn = R.attention_heads


def _attn_scale_dnope(q, kc, kr, v, rows, cfg, scale=None):
    # a scale of 1/sqrt(d_nope) instead of 1/sqrt(d_nope + d_rope)
    f = math.sqrt(cfg.d_nope / cfg.d_qk)
    return _orig_attn(np.asarray(q) / f, kc, kr, v, rows, cfg, scale)


def _attn_drop_rope_term(q, kc, kr, v, rows, cfg, scale=None):
    return _orig_attn(q, kc, np.zeros_like(np.asarray(kr, np.float64)), v, rows, cfg, scale)


_orig_decode = R.gdla_decode


def _decode_without_append(x_new, W, cfg, cache, cache_lens):
    # attend only to the rows already cached (forgets the new token's own row)
    lens = np.asarray(cache_lens)
    out = []
    for b in range(len(lens)):
        o = _orig_decode(x_new[b:b + 1], W, cfg, cache[b:b + 1], lens[b:b + 1] - 1)
        out.append(o)
    return dict(y=np.concatenate([o["y"] for o in out]), Z=np.concatenate([o["Z"] for o in out]),
                new_rows=np.concatenate([o["new_rows"] for o in out]))


def _linear_transposed(x, w):
    w = np.asarray(w, np.float64)
    if w.shape[0] == w.shape[1]:
        return np.asarray(x, np.float64) @ w
    return np.asarray(x, np.float64) @ w.T * (1.0 + 1e-3)


_orig_le = R.latent_expand


def _latent_expand_swapped(c_kv, g_kv, w_ukv, cfg):
    # value heads read from the key rows and vice versa
    kn, v, cn = _orig_le(c_kv, g_kv, w_ukv, cfg)
    return v[..., :cfg.d_nope], kn[..., :cfg.d_v], cn


def _hybrid_last_full(n, w):
    return [0 if (l % 4) == 3 else int(w) for l in range(n)]


def _block_no_residual(x, Ws, cfg, window):
    # each layer replaces the stream instead of adding to it
    x = np.asarray(x, np.float64)
    outs = []
    for W, win in zip(Ws, R.hybrid_windows(len(Ws), window)):
        y = R.gdla_layer(x, W, R._with_window(cfg, win))["y"]
        outs.append(y)
        x = y
    return outs, x


def _block_residual_from_input(x, Ws, cfg, window):
    # every layer reads the block input, not the running stream
    x0 = np.asarray(x, np.float64)
    outs = [R.gdla_layer(x0, W, R._with_window(cfg, win))["y"]
            for W, win in zip(Ws, R.hybrid_windows(len(Ws), window))]
    return outs, x0 + sum(outs)


def _block_all_full(x, Ws, cfg, window):
    # the schedule's windows dropped
    x = np.asarray(x, np.float64)
    outs = []
    for W in Ws:
        y = R.gdla_layer(x, W, R._with_window(cfg, 0))["y"]
        outs.append(y)
        x = x + y
    return outs, x


_orig_yif = R.yarn_inv_freq


def _yarn_ramp_reversed(d, base, s, orig, bf, bs):
    # interpolate the short wavelengths instead of the long ones
    th = R.rope_inv_freq(d, base)
    y = _orig_yif(d, base, s, orig, bf, bs)
    ramp = (th - y) / (th - th / s)
    return ramp * th + (1.0 - ramp) * th / s


def _yarn_times_s(d, base, s, orig, bf, bs):
    th = R.rope_inv_freq(d, base)
    ramp = (th - _orig_yif(d, base, s, orig, bf, bs)) / (th - th / s)
    return (1.0 - ramp) * th + ramp * th * s


def _yarn_mscale_sqrt(s):
    return math.sqrt(1.0 + 0.1 * math.log(s))


def _rope_params_every_layer(cfg):
    if cfg.yarn_factor > 1.0:
        return cfg.rope_base, (float(cfg.yarn_factor), float(cfg.yarn_orig_len),
                               float(cfg.yarn_beta_fast), float(cfg.yarn_beta_slow))
    return cfg.rope_base, None


def _logit_scale_without_temperature(cfg):
    # the "logit" temperature forgotten: plain 1/sqrt(d_qk) everywhere
    return 1.0 / math.sqrt(cfg.d_qk)


_orig_rope_params = R.rope_params


def _rope_params_m_in_both_modes(cfg):
    # cos and sin scaled by m under the "logit" temperature too
    base, yarn = _orig_rope_params(cfg)
    return base, (None if yarn is None else yarn[:4])


_orig_packed_bwd = R.gdla_layer_packed_backward


def _packed_backward_last_sequence_grads(x, W, cfg, dy, cu_seqlens, pos_offsets=None):
    # weight gradients of the last non-empty sequence only (overwritten, not summed)
    out = _orig_packed_bwd(x, W, cfg, dy, cu_seqlens, pos_offsets)
    segs = R.packed_segments(cu_seqlens)
    b = max(i for i, (s0, s1) in enumerate(segs) if s1 > s0)
    s0, s1 = segs[b]
    p0 = 0 if pos_offsets is None else int(pos_offsets[b])
    last = R.gdla_layer_backward(np.asarray(x, np.float64)[None, s0:s1], W, cfg,
                                 np.asarray(dy, np.float64)[None, s0:s1], pos_offset=p0)
    return dict(out, **{k: last[k] for k in W})


def _packed_global_positions(x, W, cfg, cu_seqlens, pos_offsets=None):
    # positions run on through the stream instead of restarting per sequence
    segs = R.packed_segments(cu_seqlens)
    pos = pos_offsets if pos_offsets is not None else [0] * len(segs)
    x = np.asarray(x, np.float64)
    y = np.zeros((x.shape[0], cfg.d_model))
    cache = np.zeros((x.shape[0], cfg.kv_rank + cfg.d_rope))
    lam = np.zeros((x.shape[0], cfg.n_signal))
    for (s0, s1), p0 in zip(segs, pos):
        if s1 > s0:
            r = R.gdla_layer(x[None, s0:s1], W, cfg, pos_offset=int(p0) + s0)
            y[s0:s1], cache[s0:s1], lam[s0:s1] = r["y"][0], r["cache"][0], r["lam"][0]
    return dict(y=y, Z=None, cache=cache, lam=lam)


def _packed_leaky(x, W, cfg, cu_seqlens, pos_offsets=None):
    # each sequence also sees the rows of the sequences before it
    segs = R.packed_segments(cu_seqlens)
    pos = pos_offsets if pos_offsets is not None else [0] * len(segs)
    x = np.asarray(x, np.float64)
    y = np.zeros((x.shape[0], cfg.d_model))
    cache = np.zeros((x.shape[0], cfg.kv_rank + cfg.d_rope))
    lam = np.zeros((x.shape[0], cfg.n_signal))
    for (s0, s1), p0 in zip(segs, pos):
        if s1 > s0:
            r = R.gdla_layer(x[None, 0:s1], W, cfg, pos_offset=int(p0) - s0)
            y[s0:s1], cache[s0:s1], lam[s0:s1] = r["y"][0, s0:], r["cache"][0, s0:], r["lam"][0, s0:]
    return dict(y=y, Z=None, cache=cache, lam=lam)


def _packed_segments_skip_first(cu):
    cu = [int(c) for c in cu]
    return [(min(cu[b] + 1, cu[b + 1]), cu[b + 1]) for b in range(len(cu) - 1)]


def _paged_slot_swapped(block_table, page_rows, b, p):
    return int(block_table[b][p % page_rows]), p // page_rows


def _paged_slot_no_table(block_table, page_rows, b, p):
    return b * len(block_table[b]) + p // page_rows, p % page_rows


def _rope_backward_forward_rotation(g, pos, base, yarn=None):
    # applies the forward rotation instead of its transpose
    return _ORIG["rope"](g, pos, base, yarn)


def _rms_backward_no_projection(c, gamma, eps, g):
    c, g = np.asarray(c, np.float64), np.asarray(g, np.float64)
    r = 1.0 / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)
    return r * g * np.asarray(gamma, np.float64), np.sum((g * c * r).reshape(-1, c.shape[-1]), axis=0)


def _attn_backward_no_rowsum(q, kc, kr, v, dH, cfg, rows=None):
    # dS = P * dP, the softmax's rowsum term dropped
    import math as _m
    L = kc.shape[0]
    Rw = np.arange(L) if rows is None else np.asarray(rows)
    scale = 1.0 / _m.sqrt(cfg.d_qk)
    dq = np.zeros_like(q)
    dkc = np.zeros((L, cfg.n_noise, cfg.d_nope))
    dkr = np.zeros((L, cfg.d_rope))
    dv = np.zeros((L, cfg.n_noise, cfg.d_v))
    t = np.arange(L)
    lo = np.array([R.attended_keys(int(i), cfg.window)[0] for i in Rw])
    allowed = (t[None, :] <= Rw[:, None]) & (t[None, :] >= lo[:, None])
    for h in range(cfg.n_heads):
        n = R.kv_head_of(h, cfg)
        k = np.concatenate([kc[:, n, :], kr], axis=-1)
        s = np.where(allowed, (q[:, h, :] @ k.T) * scale, -np.inf)
        P = np.exp(s - s.max(axis=-1, keepdims=True))
        P /= P.sum(axis=-1, keepdims=True)
        dv[:, n, :] += P.T @ dH[:, h, :]
        dS = P * (dH[:, h, :] @ v[:, n, :].T)
        dq[:, h, :] = (dS @ k) * scale
        dk = (dS.T @ q[:, h, :]) * scale
        dkc[:, n, :] += dk[:, :cfg.d_nope]
        dkr += dk[:, cfg.d_nope:]
    return dq, dkc, dkr, dv


def _attn_backward_rotary_key_per_group(q, kc, kr, v, dH, cfg, rows=None):
    # the rotary key's gradient kept from the noise heads only (not every head)
    dq, dkc, dkr, dv = _ORIG["attention_heads_backward"](q, kc, kr, v, dH, cfg, rows)
    dH2 = np.array(dH)
    dH2[:, :cfg.n_signal] = 0.0
    _, _, dkr_noise, _ = _ORIG["attention_heads_backward"](q, kc, kr, v, dH2, cfg, rows)
    return dq, dkc, dkr_noise, dv


MUTANTS = {
    "rope_wrong_sign": ("rope", _rope_wrong_sign),
    "rope_adjacent_pairs": ("rope", _rope_adjacent_pairs),
    "rope_theta_exponent": ("rope_inv_freq", _inv_freq_wrong),
    "kv_head_modulo": ("kv_head_of", _kv_head_modulo),
    "window_off_by_one": ("attended_keys", _window_off_by_one),
    "not_causal": ("attended_keys", _not_causal),
    "diff_one_minus_lambda": ("differential_gate_out", _diff_one_minus_lambda),
    "diff_tile_not_repeat": ("differential_gate_out", _diff_tile_not_repeat),
    "diff_no_gate": ("differential_gate_out", _diff_no_gate),
    "rms_missing_sqrt": ("rms_norm", _rms_no_eps_sqrt),
    "sigmoid_wrong": ("sigmoid", _sigmoid_tanh_wrong),
    "gate_from_raw_latent": ("query_tokens", _gate_from_raw_latent),
    "rotary_key_not_roped": ("kv_tokens", _key_not_roped),
    "kv_latent_not_normalized": ("kv_tokens", _kv_not_normalized),
    "query_rope_on_content": ("query_tokens", _query_rope_on_content),
    "scale_sqrt_dnope": ("attention_heads", _attn_scale_dnope),
    "dropped_rope_term": ("attention_heads", _attn_drop_rope_term),
    "decode_without_append": ("gdla_decode", _decode_without_append),
    "linear_transposed": ("linear", _linear_transposed),
    "latent_expand_swapped": ("latent_expand", _latent_expand_swapped),
    "hybrid_last_full": ("hybrid_windows", _hybrid_last_full),
    "block_no_residual": ("gdla_block", _block_no_residual),
    "block_residual_from_input": ("gdla_block", _block_residual_from_input),
    "block_all_full": ("gdla_block", _block_all_full),
    "yarn_ramp_reversed": ("yarn_inv_freq", _yarn_ramp_reversed),
    "yarn_times_s": ("yarn_inv_freq", _yarn_times_s),
    "yarn_mscale_sqrt": ("yarn_mscale", _yarn_mscale_sqrt),
    "yarn_on_window_layers": ("rope_params", _rope_params_every_layer),
    "yarn_logit_temperature_dropped": ("logit_scale", _logit_scale_without_temperature),
    "yarn_m_on_rope_in_logit_mode": ("rope_params", _rope_params_m_in_both_modes),
    "packed_global_positions": ("gdla_layer_packed", _packed_global_positions),
    "packed_leaky": ("gdla_layer_packed", _packed_leaky),
    "packed_segments_skip_first": ("packed_segments", _packed_segments_skip_first),
    "packed_backward_last_sequence_grads": ("gdla_layer_packed_backward", _packed_backward_last_sequence_grads),
    "paged_slot_swapped": ("paged_slot", _paged_slot_swapped),
    "paged_slot_no_table": ("paged_slot", _paged_slot_no_table),
    "rope_backward_forward_rotation": ("rope_backward", _rope_backward_forward_rotation),
    "rms_backward_no_projection": ("rms_norm_backward", _rms_backward_no_projection),
    "attn_backward_no_rowsum": ("attention_heads_backward", _attn_backward_no_rowsum),
    "attn_backward_rotary_key_per_group": ("attention_heads_backward", _attn_backward_rotary_key_per_group),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # AssertionError, or a shape error from the mutant
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
