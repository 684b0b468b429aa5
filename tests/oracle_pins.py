"""Pins that tie the GDLA oracle to facts outside itself: closed forms,
invariants, special cases that reduce to textbook routines, and brute force on
tiny inputs.  Each pin is a plain function that raises AssertionError; the
pytest module test_oracle_pins.py runs them, and test_oracle_mutants.py runs
them again against deliberately broken copies of the oracle to show that each
plausible mistake is caught by at least one pin.

Every call goes through the module object R so that a patched oracle function
is seen by the pins.
"""

from __future__ import annotations

import math
from dataclasses import replace

import numpy as np

import oracle.gdla_ref as R

# A tiny layer: 2 noise heads, g = 2 (4 signal heads), 4-dim content / rotary
# parts, so every loop below is cheap.
TINY = R.Cfg(d_model=24, q_rank=12, kv_rank=8, n_noise=2, group=2, d_nope=4, d_rope=4, d_v=4)
L_TINY = 11


def tiny_weights(cfg=TINY, seed=0, sharp=2.0, gamma_random=True):
    """Random weights with std sharp/sqrt(fan_in) so attention is not uniform."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nS, H = cfg.n_signal, cfg.n_heads

    def w(o, i, s=1.0):
        return rng.standard_normal((o, i)) * (s / math.sqrt(i))

    W = dict(
        w_dq=w(cfg.q_rank, cfg.d_model),
        w_dkv=w(cfg.kv_rank + cfg.d_rope, cfg.d_model, sharp),
        w_lambda=w(nS, cfg.d_model),
        w_uq=w(H * cfg.d_qk, cfg.q_rank, sharp),
        w_ukv=w(cfg.n_noise * (cfg.d_nope + cfg.d_v), cfg.kv_rank),
        w_gate=w(nS * cfg.d_v, cfg.q_rank),
        w_o=w(cfg.d_model, nS * cfg.d_v),
    )
    if gamma_random:
        W["g_q"] = 1.0 + 0.2 * rng.standard_normal(cfg.q_rank)
        W["g_kv"] = 1.0 + 0.2 * rng.standard_normal(cfg.kv_rank)
    else:
        W["g_q"] = np.ones(cfg.q_rank)
        W["g_kv"] = np.ones(cfg.kv_rank)
    return W


def tiny_x(B=2, L=L_TINY, cfg=TINY, seed=1):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((B, L, cfg.d_model))


def close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- projections

def pin_linear_explicit_sums():
    """x W^T with W stored [out, in], against explicit triple loops."""
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    ref = [[sum(x[i, k] * w[o, k] for k in range(5)) for o in range(4)] for i in range(3)]
    close(R.linear(x, w), ref)


def pin_rms_norm_closed_form():
    """[3, 4] has mean square 12.5; unit gain makes the output RMS one; scaling
    the input does not change the output (up to eps)."""
    eps = 1e-6
    close(R.rms_norm(np.array([3.0, 4.0]), np.ones(2), eps),
          np.array([3.0, 4.0]) / math.sqrt(12.5 + eps))
    rng = np.random.Generator(np.random.PCG64(6))
    c = rng.standard_normal((7, 16)) * 3.0
    out = R.rms_norm(c, np.ones(16), 0.0)
    close(np.sqrt(np.mean(out ** 2, axis=-1)), np.ones(7))
    close(R.rms_norm(5.0 * c, np.ones(16), 0.0), out)
    g = rng.standard_normal(16)
    close(R.rms_norm(c, g, 0.0), out * g)


def pin_sigmoid_values():
    close(R.sigmoid(0.0), 0.5)
    close(R.sigmoid(math.log(3.0)), 0.75)
    z = np.linspace(-30, 30, 61)
    close(R.sigmoid(z) + R.sigmoid(-z), np.ones_like(z))


# ---------------------------------------------------------------------- RoPE

def pin_rope_frequencies():
    """theta_i = base^(-2i/d): d = 4, base 10000 gives (1, 1/100); d = 64 ends
    at base^(-62/64)."""
    close(R.rope_inv_freq(4, 10000.0), [1.0, 0.01])
    th = R.rope_inv_freq(64, 10000.0)
    assert th.shape == (32,)
    close(th[-1], 10000.0 ** (-62.0 / 64.0))


def pin_rope_complex_rotation():
    """Rotate-half RoPE multiplies z_i = u_i + 1j*u_{i+d/2} by exp(1j*p*theta_i)
    (complex form of the block-diagonal rotation); p = 0 is the identity and
    the rotation keeps the norm."""
    rng = np.random.Generator(np.random.PCG64(7))
    d, base = 8, 10000.0
    u = rng.standard_normal((5, d))
    pos = np.array([0.0, 1.0, 2.0, 37.0, 40000.0])
    out = R.rope(u, pos, base)
    z = u[:, :d // 2] + 1j * u[:, d // 2:]
    th = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None] * th[None, :])
    close(out[:, :d // 2], zr.real)
    close(out[:, d // 2:], zr.imag)
    close(out[0], u[0])
    close(np.linalg.norm(out, axis=1), np.linalg.norm(u, axis=1))
    # the first pair turns by exactly p radians: (1, 0) -> (cos 1, sin 1)
    e = np.zeros((1, d)); e[0, 0] = 1.0
    r1 = R.rope(e, np.array([1.0]), base)[0]
    close([r1[0], r1[d // 2]], [math.cos(1.0), math.sin(1.0)])


def pin_rope_relative():
    """<rope(q, m), rope(k, n)> depends only on m - n; rotations compose."""
    rng = np.random.Generator(np.random.PCG64(8))
    q, k = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    a = float((R.rope(q, np.array([100.0]), 1e4) @ R.rope(k, np.array([93.0]), 1e4).T)[0, 0])
    b = float((R.rope(q, np.array([7.0]), 1e4) @ R.rope(k, np.array([0.0]), 1e4).T)[0, 0])
    close(a, b, 1e-10)
    close(R.rope(R.rope(q, np.array([3.0]), 1e4), np.array([4.0]), 1e4),
          R.rope(q, np.array([7.0]), 1e4), 1e-12)


# ----------------------------------------------------------------- attention

def brute_force_heads(q, kc, kr, v, rows, cfg):
    """Per-head, per-row softmax attention with scalar loops and math.exp."""
    out = np.zeros((len(rows), cfg.n_heads, cfg.d_v))
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)
    for ri, t in enumerate(rows):
        lo = 0 if cfg.window <= 0 else max(0, t - cfg.window + 1)
        for h in range(cfg.n_heads):
            n = h // cfg.group if h < cfg.group * cfg.n_noise else h - cfg.group * cfg.n_noise
            sc = []
            for s in range(lo, t + 1):
                dot = 0.0
                for i in range(cfg.d_nope):
                    dot += q[ri, h, i] * kc[s, n, i]
                for i in range(cfg.d_rope):
                    dot += q[ri, h, cfg.d_nope + i] * kr[s, i]
                sc.append(dot * scale)
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            tot = sum(e)
            for j in range(cfg.d_v):
                out[ri, h, j] = sum(e[s - lo] * v[s, n, j] for s in range(lo, t + 1)) / tot
    return out


def _rand_qkv(cfg, L, seed, sharp=2.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((L, cfg.n_heads, cfg.d_qk)) * sharp
    kc = rng.standard_normal((L, cfg.n_noise, cfg.d_nope))
    kr = rng.standard_normal((L, cfg.d_rope))
    v = rng.standard_normal((L, cfg.n_noise, cfg.d_v))
    return q, kc, kr, v


def pin_attention_brute_force():
    for window in (0, 3, 1, 50):
        cfg = replace(TINY, window=window)
        q, kc, kr, v = _rand_qkv(cfg, 9, seed=11 + window)
        rows = list(range(9))
        close(R.attention_heads(q, kc, kr, v, rows, cfg), brute_force_heads(q, kc, kr, v, rows, cfg), 1e-12)
        sub = [0, 4, 8]
        close(R.attention_heads(q[sub], kc, kr, v, sub, cfg), brute_force_heads(q[sub], kc, kr, v, sub, cfg), 1e-12)


def pin_attention_two_key_closed_form():
    """Row 1 sees keys 0 and 1: H = v0 + sigmoid((s1 - s0)/sqrt(d_qk)) (v1 - v0)."""
    cfg = TINY
    q, kc, kr, v = _rand_qkv(cfg, 2, seed=21)
    H = R.attention_heads(q[1:2], kc, kr, v, [1], cfg)[0]
    for h in range(cfg.n_heads):
        n = h // cfg.group if h < cfg.n_signal else h - cfg.n_signal
        k0 = np.concatenate([kc[0, n], kr[0]])
        k1 = np.concatenate([kc[1, n], kr[1]])
        a = 1.0 / (1.0 + math.exp(-(q[1, h] @ k1 - q[1, h] @ k0) / math.sqrt(cfg.d_qk)))
        close(H[h], v[0, n] + a * (v[1, n] - v[0, n]), 1e-12)


def pin_attention_head_mapping():
    """With KV head n's values all equal to n + 1, every query head returns the
    number of the KV head it reads: signal j -> j // g, noise nS + n -> n."""
    cfg = replace(TINY, n_noise=3, group=3)
    L = 5
    q, kc, kr, _ = _rand_qkv(cfg, L, seed=22)
    v = np.zeros((L, cfg.n_noise, cfg.d_v))
    for n in range(cfg.n_noise):
        v[:, n, :] = n + 1
    H = R.attention_heads(q, kc, kr, v, list(range(L)), cfg)
    expect = [1, 1, 1, 2, 2, 2, 3, 3, 3, 1, 2, 3]
    for h, e in enumerate(expect):
        close(H[:, h, :], np.full((L, cfg.d_v), float(e)))


def pin_attention_masks():
    """W >= L equals full causal; W = 1 returns the token's own value; row 0
    returns v_0; with q = 0 each row is the mean of v over its window."""
    L = 10
    q, kc, kr, v = _rand_qkv(TINY, L, seed=23)
    rows = list(range(L))
    full = R.attention_heads(q, kc, kr, v, rows, replace(TINY, window=0))
    close(R.attention_heads(q, kc, kr, v, rows, replace(TINY, window=L)), full, 1e-13)
    close(R.attention_heads(q, kc, kr, v, rows, replace(TINY, window=L + 5)), full, 1e-13)
    own = R.attention_heads(q, kc, kr, v, rows, replace(TINY, window=1))
    for h in range(TINY.n_heads):
        n = h // TINY.group if h < TINY.n_signal else h - TINY.n_signal
        close(own[:, h], v[:, n])
        close(full[0, h], v[0, n])
    zero_q = np.zeros_like(q)
    for window in (0, 4):
        Hm = R.attention_heads(zero_q, kc, kr, v, rows, replace(TINY, window=window))
        for t in range(L):
            lo = 0 if window == 0 else max(0, t - window + 1)
            for h in range(TINY.n_heads):
                n = h // TINY.group if h < TINY.n_signal else h - TINY.n_signal
                close(Hm[t, h], v[lo:t + 1, n].mean(axis=0), 1e-13)


# -------------------------------------------------------------- whole layer

def pin_layer_causality():
    """Changing x at s > t leaves row t unchanged; with a window W, so does
    changing x at s <= t - W, while s = t - W + 1 is inside the window."""
    W = tiny_weights()
    x = tiny_x(B=1)
    t = 7
    for window in (0, 3):
        cfg = replace(TINY, window=window)
        base = R.gdla_layer(x, W, cfg)["y"][0]
        x2 = x.copy(); x2[0, t + 1:] += 5.0
        close(R.gdla_layer(x2, W, cfg)["y"][0, :t + 1], base[:t + 1], 1e-12)
        if window:
            x3 = x.copy(); x3[0, :t - window + 1] += 5.0
            close(R.gdla_layer(x3, W, cfg)["y"][0, t], base[t], 1e-12)
            x4 = x.copy(); x4[0, t - window + 1] += 5.0
            d = np.max(np.abs(R.gdla_layer(x4, W, cfg)["y"][0, t] - base[t]))
            assert d > 1e-6, "the oldest key inside the window had no effect"


def pin_layer_position_shift():
    """Only relative positions enter the scores, so a common position offset
    leaves y unchanged; the cache's rotary key does change."""
    W = tiny_weights()
    x = tiny_x()
    a = R.gdla_layer(x, W, TINY, pos_offset=0)
    b = R.gdla_layer(x, W, TINY, pos_offset=1234)
    close(b["y"], a["y"], 1e-10)
    assert np.max(np.abs(b["cache"][..., TINY.kv_rank:] - a["cache"][..., TINY.kv_rank:])) > 1e-3


def pin_layer_norm_invariance():
    """Both latents are RMS-normalized: scaling W_DQ, or the latent rows of
    W_DKV, by c > 0 leaves y unchanged (eps = 0); scaling the rotary-key rows
    does change y (that key is not normalized)."""
    W = tiny_weights()
    x = tiny_x()
    cfg = replace(TINY, rms_eps=0.0)
    base = R.gdla_layer(x, W, cfg)["y"]
    W1 = dict(W, w_dq=W["w_dq"] * 3.7)
    close(R.gdla_layer(x, W1, cfg)["y"], base, 1e-12)
    w_dkv = W["w_dkv"].copy(); w_dkv[:cfg.kv_rank] *= 0.3
    close(R.gdla_layer(x, dict(W, w_dkv=w_dkv), cfg)["y"], base, 1e-12)
    w_dkv = W["w_dkv"].copy(); w_dkv[cfg.kv_rank:] *= 3.0
    assert np.max(np.abs(R.gdla_layer(x, dict(W, w_dkv=w_dkv), cfg)["y"] - base)) > 1e-6


def mla_gqa_reference(x, W, cfg):
    """Multi-head latent attention with grouped KV heads written the standard
    way (per-head q, k, v, then softmax attention), for the signal heads only,
    followed by the gate and the output projection; this is what GDLA reduces
    to when lambda = 0."""
    B, L, _ = x.shape
    out = np.zeros((B, L, cfg.d_model))
    th = np.array([cfg.rope_base ** (-2.0 * i / cfg.d_rope) for i in range(cfg.d_rope // 2)])
    for b in range(B):
        cq = x[b] @ W["w_dq"].T
        cqn = cq / np.sqrt((cq ** 2).mean(-1, keepdims=True) + cfg.rms_eps) * W["g_q"]
        ckr = x[b] @ W["w_dkv"].T
        c = ckr[:, :cfg.kv_rank]
        cn = c / np.sqrt((c ** 2).mean(-1, keepdims=True) + cfg.rms_eps) * W["g_kv"]
        kr = ckr[:, cfg.kv_rank:]
        qall = (cqn @ W["w_uq"].T).reshape(L, cfg.n_heads, cfg.d_qk)
        kv = cn @ W["w_ukv"].T
        gate = 1.0 / (1.0 + np.exp(-(cqn @ W["w_gate"].T)))
        Z = np.zeros((L, cfg.n_signal * cfg.d_v))
        for j in range(cfg.n_signal):
            n = j // cfg.group
            qh = qall[:, j, :].copy()
            kh = np.concatenate([kv[:, n * cfg.d_nope:(n + 1) * cfg.d_nope], kr], axis=1)
            vh = kv[:, cfg.n_noise * cfg.d_nope + n * cfg.d_v:cfg.n_noise * cfg.d_nope + (n + 1) * cfg.d_v]
            # rotary parts as complex numbers turned by p * theta
            half = cfg.d_rope // 2
            ang = np.arange(L)[:, None] * th[None, :]
            for arr in (qh, kh):
                z = (arr[:, cfg.d_nope:cfg.d_nope + half] + 1j * arr[:, cfg.d_nope + half:]) * np.exp(1j * ang)
                arr[:, cfg.d_nope:cfg.d_nope + half] = z.real
                arr[:, cfg.d_nope + half:] = z.imag
            s = qh @ kh.T / math.sqrt(cfg.d_qk)
            s[np.triu_indices(L, 1)] = -np.inf
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            Z[:, j * cfg.d_v:(j + 1) * cfg.d_v] = p @ vh
        out[b] = (gate * Z) @ W["w_o"].T
    return out


def pin_layer_lambda_zero_is_latent_attention():
    W = tiny_weights()
    x = tiny_x()
    got = R.gdla_layer(x, W, TINY, lam_override=0.0)["y"]
    close(got, mla_gqa_reference(x, W, TINY), 1e-11)


def pin_layer_closed_forms():
    """W_lambda = 0 gives lambda = 1/2; W_G = 0 gives gate = 1/2 so Z = D/2;
    with g = 1 and each noise head's query rows equal to its signal head's,
    H_N = H_S and D = (1 - lambda) H_S."""
    W = tiny_weights()
    x = tiny_x()
    out = R.gdla_layer(x, dict(W, w_lambda=np.zeros_like(W["w_lambda"])), TINY)
    close(out["lam"], np.full_like(out["lam"], 0.5), 0)
    Wg = dict(W, w_gate=np.zeros_like(W["w_gate"]))
    o = R.gdla_layer(x, Wg, TINY)
    H = o["H"]
    nS, g = TINY.n_signal, TINY.group
    D = H[:, :, :nS] - o["lam"][..., None] * np.repeat(H[:, :, nS:], g, axis=2)
    close(o["Z"], 0.5 * D.reshape(*D.shape[:2], -1), 1e-13)
    # g = 1: copy each signal head's W_UQ rows into its noise partner
    c1 = replace(TINY, group=1, n_noise=2)
    W1 = tiny_weights(c1, seed=3)
    wuq = W1["w_uq"].reshape(c1.n_heads, c1.d_qk, c1.q_rank).copy()
    wuq[c1.n_signal:] = wuq[:c1.n_signal]
    W1["w_uq"] = wuq.reshape(-1, c1.q_rank)
    o1 = R.gdla_layer(x, W1, c1)
    Hs = o1["H"][:, :, :c1.n_signal]
    close(o1["H"][:, :, c1.n_signal:], Hs, 1e-13)
    Dexp = (1.0 - o1["lam"])[..., None] * Hs
    o1g = R.gdla_layer(x, dict(W1, w_gate=np.zeros_like(W1["w_gate"])), c1)
    close(o1g["Z"], 0.5 * Dexp.reshape(*Dexp.shape[:2], -1), 1e-12)


def pin_differential_pairing():
    """Signal head j subtracts noise head j // g (g = 2, two noise heads:
    heads 0, 1 pair with noise 0 and heads 2, 3 with noise 1)."""
    cfg = TINY
    Hs = np.arange(4 * cfg.d_v, dtype=np.float64).reshape(1, 4, cfg.d_v)
    Hn = np.array([[[100.0] * cfg.d_v, [1000.0] * cfg.d_v]])
    lam = np.array([[0.5, 0.25, 0.5, 0.25]])
    _, Z, D = R.differential_gate_out(Hs, Hn, lam, np.ones((1, 4 * cfg.d_v)),
                                      np.zeros((3, 4 * cfg.d_v)), cfg)
    close(D[0, 0], Hs[0, 0] - 50.0)
    close(D[0, 1], Hs[0, 1] - 25.0)
    close(D[0, 2], Hs[0, 2] - 500.0)
    close(D[0, 3], Hs[0, 3] - 250.0)


def pin_decode_matches_prefill():
    """Decoding token L-1 against the cache prefill wrote for tokens 0..L-2
    gives prefill's row L-1, for full and windowed layers."""
    W = tiny_weights()
    x = tiny_x(B=2)
    L = x.shape[1]
    for window in (0, 4):
        cfg = replace(TINY, window=window)
        full = R.gdla_layer(x, W, cfg)
        pre = R.gdla_layer(x[:, :L - 1], W, cfg)
        cap = L + 3
        cache = np.zeros((2, cap, cfg.kv_rank + cfg.d_rope))
        cache[:, :L - 1] = pre["cache"]
        dec = R.gdla_decode(x[:, L - 1], W, cfg, cache, np.array([L - 1, L - 1]))
        close(dec["y"], full["y"][:, L - 1], 1e-11)
        close(dec["new_rows"], full["cache"][:, L - 1], 1e-12)


def pin_latent_expand():
    """latent_expand = RMSNorm then W_UKV split into key heads then value
    heads, checked element by element with explicit sums."""
    cfg = TINY
    rng = np.random.Generator(np.random.PCG64(31))
    c = rng.standard_normal((3, cfg.kv_rank))
    g = rng.standard_normal(cfg.kv_rank)
    w = rng.standard_normal((cfg.n_noise * (cfg.d_nope + cfg.d_v), cfg.kv_rank))
    kn, v, cn = R.latent_expand(c, g, w, cfg)
    for t in range(3):
        r = math.sqrt(sum(c[t, i] ** 2 for i in range(cfg.kv_rank)) / cfg.kv_rank + cfg.rms_eps)
        for n in range(cfg.n_noise):
            for i in range(cfg.d_nope):
                row = n * cfg.d_nope + i
                close(kn[t, n, i], sum(c[t, k] / r * g[k] * w[row, k] for k in range(cfg.kv_rank)), 1e-12)
            for i in range(cfg.d_v):
                row = cfg.n_noise * cfg.d_nope + n * cfg.d_v + i
                close(v[t, n, i], sum(c[t, k] / r * g[k] * w[row, k] for k in range(cfg.kv_rank)), 1e-12)


def pin_hybrid_schedule():
    """One full-causal layer, then three sliding-window layers, repeating."""
    assert R.hybrid_windows(4, 4096) == [0, 4096, 4096, 4096]
    assert R.hybrid_windows(8, 128) == [0, 128, 128, 128, 0, 128, 128, 128]


def _zero_out_proj(W):
    return dict(W, w_o=np.zeros_like(W["w_o"]))


def pin_block_residual_and_schedule():
    """The hybrid block ([M3-arch]) joins its layers by x_{l+1} = x_l + y_l
    and runs layer 0 full causal, layers 1-3 windowed.  With every output
    projection zero each y_l = 0, so the block is the identity; with only
    layer k's projection non-zero the block is x + layer_k(x) at that layer's
    window (full for k = 0, W otherwise), and every other layer output is 0;
    with layers 0 and 1 non-zero, layer 1 sees x + y_0."""
    window = 3
    Ws = [tiny_weights(seed=60 + l) for l in range(4)]
    x = tiny_x(B=2, seed=64)
    full_cfg, win_cfg = replace(TINY, window=0), replace(TINY, window=window)
    # the window must matter at this size, or the schedule would go unchecked
    assert np.max(np.abs(R.gdla_layer(x, Ws[1], full_cfg)["y"] - R.gdla_layer(x, Ws[1], win_cfg)["y"])) > 1e-6
    outs, xf = R.gdla_block(x, [_zero_out_proj(W) for W in Ws], TINY, window)
    assert len(outs) == 4
    close(xf, x, 0.0)
    for y in outs:
        assert np.all(y == 0.0)
    for k in range(4):
        Wk = [W if l == k else _zero_out_proj(W) for l, W in enumerate(Ws)]
        outs, xf = R.gdla_block(x, Wk, TINY, window)
        yk = R.gdla_layer(x, Ws[k], full_cfg if k == 0 else win_cfg)["y"]
        close(outs[k], yk, 1e-12)
        close(xf, x + yk, 1e-12)
        for l in range(4):
            if l != k:
                assert np.all(outs[l] == 0.0), f"layer {l} output with a zero projection"
    W01 = [Ws[0], Ws[1], _zero_out_proj(Ws[2]), _zero_out_proj(Ws[3])]
    outs, xf = R.gdla_block(x, W01, TINY, window)
    y0 = R.gdla_layer(x, Ws[0], full_cfg)["y"]
    y1 = R.gdla_layer(x + y0, Ws[1], win_cfg)["y"]
    close(outs[1], y1, 1e-12)
    close(xf, x + y0 + y1, 1e-12)


def pin_block_causality():
    """Every layer of the block is causal, so changing x at s > t leaves
    rows 0..t of the block's output unchanged, while row t itself depends on x_t."""
    Ws = [tiny_weights(seed=70 + l) for l in range(4)]
    x = tiny_x(B=1, seed=74)
    t = 6
    _, base = R.gdla_block(x, Ws, TINY, 2)
    x2 = x.copy(); x2[0, t + 1:] += 3.0
    close(R.gdla_block(x2, Ws, TINY, 2)[1][0, :t + 1], base[0, :t + 1], 1e-12)
    x3 = x.copy(); x3[0, t] += 3.0
    assert np.max(np.abs(R.gdla_block(x3, Ws, TINY, 2)[1][0, t] - base[0, t])) > 1e-3


# YaRN ([OSM-yarn]) with the long-context settings of [M3-ctx]: factor 64 over
# a native 4096, beta_fast 32, beta_slow 1, on a 64-wide rotary part, base 1e4.
YARN = (64.0, 4096.0, 32.0, 1.0)


def pin_yarn_identity_at_factor_one():
    """s = 1 is plain RoPE: no frequency moves and m = 1 + 0.1 ln 1 = 1."""
    th = R.rope_inv_freq(64, 1e4)
    assert np.max(np.abs(R.yarn_inv_freq(64, 1e4, 1.0, 4096.0, 32.0, 1.0) / th - 1.0)) < 1e-15
    assert R.yarn_mscale(1.0) == 1.0
    u = np.random.Generator(np.random.PCG64(3)).standard_normal((5, 64))
    pos = np.array([0.0, 1.0, 17.0, 4095.0, 70000.0])
    close(R.rope(u, pos, 1e4, (1.0, 4096.0, 32.0, 1.0)), R.rope(u, pos, 1e4), 1e-12)


def pin_yarn_bands_and_values():
    """Pair i has wavelength 2 pi 10^(i/8).  It is below 4096/32 = 128 exactly
    for i <= 10 (10^(10/8) = 17.8 < 20.37 < 10^(11/8) = 23.7), so those
    frequencies are unchanged; it is above 4096 exactly for i >= 23
    (10^(22/8) = 562 < 651.9 < 10^(23/8) = 750), so those are divided by 64.
    Pair 16 (wavelength 200 pi = 628.32) sits at (628.32 - 128) / 3968 =
    0.126088 of the ramp: 0.01 (0.873912 + 0.126088 / 64) = 0.0087588179.
    m = 1 + 0.1 ln 64 = 1.4158883083."""
    th = R.rope_inv_freq(64, 1e4)
    y = R.yarn_inv_freq(64, 1e4, *YARN)
    assert [i for i in range(32) if y[i] == th[i]] == list(range(11))
    assert [i for i in range(32) if abs(y[i] * 64.0 / th[i] - 1.0) < 1e-12] == list(range(23, 32))
    assert abs(y[16] - 0.0087588179) < 1e-10, y[16]
    assert abs(R.yarn_mscale(64.0) - 1.4158883083) < 1e-10
    assert np.all(np.diff(y) < 0)


def pin_yarn_is_rope_at_scaled_positions():
    """Each rotary pair turns on its own, so a vector living in the high band
    (pairs <= 10) rotates like plain RoPE at position p and one in the low
    band (pairs >= 23) like plain RoPE at p / 64, both times m."""
    rng = np.random.Generator(np.random.PCG64(4))
    pos = np.array([0.0, 5.0, 4096.0, 100000.0, 262143.0])
    m = 1.0 + 0.1 * math.log(64.0)
    for pairs, scale in ((range(0, 11), 1.0), (range(23, 32), 1.0 / 64.0)):
        u = np.zeros((5, 64))
        for i in pairs:
            u[:, i] = rng.standard_normal(5)
            u[:, 32 + i] = rng.standard_normal(5)
        close(R.rope(u, pos, 1e4, YARN), m * R.rope(u, pos * scale, 1e4), 1e-9)


def pin_yarn_relative_and_norm():
    """Fixed frequencies keep <rope(q, a), rope(k, b)> a function of a - b;
    the rotated vectors are m times as long."""
    rng = np.random.Generator(np.random.PCG64(5))
    q, k = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    a = float((R.rope(q, np.array([9000.0]), 1e4, YARN) @ R.rope(k, np.array([1000.0]), 1e4, YARN).T)[0, 0])
    b = float((R.rope(q, np.array([8000.0]), 1e4, YARN) @ R.rope(k, np.array([0.0]), 1e4, YARN).T)[0, 0])
    assert abs(a - b) < 1e-9 * max(1.0, abs(a))
    m = 1.0 + 0.1 * math.log(64.0)
    r = R.rope(q, np.array([123456.0]), 1e4, YARN)
    assert abs(np.linalg.norm(r) - m * np.linalg.norm(q)) < 1e-12 * np.linalg.norm(q) * 10


def pin_yarn_full_layers_only():
    """[M3-ctx]: YaRN on the full-causal layers; a windowed layer with the
    same settings equals the plain-RoPE layer, a full one does not."""
    W = tiny_weights()
    x = tiny_x(B=1, L=7)
    yarn_cfg = replace(TINY, yarn_factor=64.0, yarn_orig_len=4, yarn_beta_fast=2.0, yarn_beta_slow=0.5)
    win = R.gdla_layer(x, W, replace(yarn_cfg, window=3))["y"]
    close(win, R.gdla_layer(x, W, replace(TINY, window=3))["y"], 1e-12)
    full = R.gdla_layer(x, W, yarn_cfg)["y"]
    assert np.max(np.abs(full - R.gdla_layer(x, W, TINY)["y"])) > 1e-6


YARN_TINY = dict(yarn_factor=64.0, yarn_orig_len=4, yarn_beta_fast=2.0, yarn_beta_slow=0.5)


def pin_yarn_logit_temperature_two_keys():
    """With the "logit" temperature every logit of a YaRN layer is multiplied
    by m^2 = (1 + 0.1 ln 64)^2: row 1 seeing keys 0 and 1 gives
    H = v0 + sigmoid(m^2 (s1 - s0) / sqrt(d_qk)) (v1 - v0).  The "rotary"
    temperature (the listing) puts m on cos and sin instead, so on given
    rotated queries and keys its attention carries no extra factor; nor does a
    windowed layer (YaRN only on full-causal layers)."""
    m2 = (1.0 + 0.1 * math.log(64.0)) ** 2
    q, kc, kr, v = _rand_qkv(TINY, 2, seed=23)
    for temp, win, f in (("logit", 0, m2), ("rotary", 0, 1.0), ("logit", 3, 1.0)):
        cfg = replace(TINY, window=win, yarn_temperature=temp, **YARN_TINY)
        H = R.attention_heads(q[1:2], kc, kr, v, [1], cfg)[0]
        for h in range(cfg.n_heads):
            n = h // cfg.group if h < cfg.n_signal else h - cfg.n_signal
            k0 = np.concatenate([kc[0, n], kr[0]])
            k1 = np.concatenate([kc[1, n], kr[1]])
            a = 1.0 / (1.0 + math.exp(-f * (q[1, h] @ k1 - q[1, h] @ k0) / math.sqrt(cfg.d_qk)))
            close(H[h], v[0, n] + a * (v[1, n] - v[0, n]), 1e-12)


def pin_yarn_temperature_modes():
    """The two temperatures differ only in where m goes.  The "logit" one
    leaves cos and sin unscaled (rotated vectors keep their length), the
    "rotary" one scales them by m.  With the content keys zeroed (the content
    rows of W_UKV), every logit is its rotary term, which both scale by m^2,
    so the two layers agree; with content keys they differ."""
    m = 1.0 + 0.1 * math.log(64.0)
    u = np.random.Generator(np.random.PCG64(6)).standard_normal((3, 4))
    pos = np.array([0.0, 3.0, 50.0])
    cfg_l = replace(TINY, yarn_temperature="logit", **YARN_TINY)
    cfg_r = replace(TINY, yarn_temperature="rotary", **YARN_TINY)
    for cfg, f in ((cfg_l, 1.0), (cfg_r, m)):
        r = R.rope(u, pos, *R.rope_params(cfg))
        close(np.linalg.norm(r, axis=-1), f * np.linalg.norm(u, axis=-1), 1e-12)
    W = tiny_weights(seed=40)
    x = tiny_x(B=1, L=7, seed=41)
    assert np.max(np.abs(R.gdla_layer(x, W, cfg_l)["y"] - R.gdla_layer(x, W, cfg_r)["y"])) > 1e-6
    W0 = dict(W, w_ukv=W["w_ukv"].copy())
    W0["w_ukv"][:TINY.n_noise * TINY.d_nope] = 0.0
    close(R.gdla_layer(x, W0, cfg_l)["y"], R.gdla_layer(x, W0, cfg_r)["y"], 1e-12)


# ------------------------------------------- packed sequences and the paged cache
PACK_LENS = (3, 1, 5, 0, 2)
PACK_POS = (0, 7, 2, 9, 4)


def _pack(lens, seed=3):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal((int(cu[-1]), TINY.d_model))
    return cu, x


def pin_packed_one_sequence_is_the_layer():
    """A stream holding one sequence is the layer over that sequence, at the
    sequence's position offset, full and windowed."""
    W = tiny_weights()
    x = tiny_x(B=1)
    L = x.shape[1]
    for window in (0, 3):
        cfg = replace(TINY, window=window)
        r = R.gdla_layer_packed(x[0], W, cfg, [0, L], [5])
        ref = R.gdla_layer(x, W, cfg, pos_offset=5)
        close(r["y"], ref["y"][0], 1e-13)
        close(r["cache"], ref["cache"][0], 1e-13)


def pin_packed_equal_lengths_is_the_batch():
    """Sequences of one length packed end to end give the batched layer's rows."""
    W = tiny_weights()
    x = tiny_x(B=3, L=6)
    r = R.gdla_layer_packed(x.reshape(18, -1), W, TINY, [0, 6, 12, 18])
    ref = R.gdla_layer(x, W, TINY)
    close(r["y"], ref["y"].reshape(18, -1), 1e-13)
    close(r["cache"], ref["cache"].reshape(18, -1), 1e-13)


def pin_packed_sequences_are_separate_layers():
    """Every packed sequence (an empty one included) matches the layer run on
    it alone at its own offset; row ranges come from the lengths here."""
    W = tiny_weights()
    cu, x = _pack(PACK_LENS)
    starts = np.cumsum((0,) + PACK_LENS[:-1])
    for window in (0, 2):
        cfg = replace(TINY, window=window)
        r = R.gdla_layer_packed(x, W, cfg, cu, PACK_POS)
        assert r["y"].shape == (sum(PACK_LENS), TINY.d_model)
        for b, n in enumerate(PACK_LENS):
            if n == 0:
                continue
            s0 = int(starts[b])
            ref = R.gdla_layer(x[None, s0:s0 + n], W, cfg, pos_offset=PACK_POS[b])
            close(r["y"][s0:s0 + n], ref["y"][0], 1e-13)
            close(r["lam"][s0:s0 + n], ref["lam"][0], 1e-13)


def pin_packed_isolation():
    """Changing one sequence leaves every other row bit for bit; dropping it
    from the stream shifts the others' rows without changing their values
    (positions restart per sequence, keys never cross a boundary)."""
    W = tiny_weights()
    cu, x = _pack(PACK_LENS)
    for window in (0, 4):
        cfg = replace(TINY, window=window)
        base = R.gdla_layer_packed(x, W, cfg, cu, PACK_POS)
        x2 = x.copy()
        x2[0:3] += 1.0
        r2 = R.gdla_layer_packed(x2, W, cfg, cu, PACK_POS)
        assert np.array_equal(r2["y"][3:], base["y"][3:]), "a change in sequence 0 reached another sequence"
        assert not np.allclose(r2["y"][:3], base["y"][:3])
        r3 = R.gdla_layer_packed(x[3:], W, cfg, [0, 1, 6, 6, 8], PACK_POS[1:])
        close(r3["y"], base["y"][3:], 1e-13)


def pin_packed_order_invariance():
    """Reordering the sequences in the stream reorders the output rows."""
    W = tiny_weights()
    cu, x = _pack(PACK_LENS)
    base = R.gdla_layer_packed(x, W, TINY, cu, PACK_POS)
    order = [2, 4, 0, 1, 3]
    parts = [np.arange(cu[b], cu[b + 1]) for b in order]
    idx = np.concatenate(parts)
    cu2 = np.concatenate([[0], np.cumsum([len(q) for q in parts])])
    r = R.gdla_layer_packed(x[idx], W, TINY, cu2, [PACK_POS[b] for b in order])
    close(r["y"], base["y"][idx], 1e-13)


def _dense_and_pages(seed=4, B=3, cap=12, page_rows=4):
    rng = np.random.Generator(np.random.PCG64(seed))
    RL = TINY.kv_rank + TINY.d_rope
    dense = rng.standard_normal((B, cap, RL))
    k = cap // page_rows
    return rng, dense, dense.reshape(B * k, page_rows, RL), [[b * k + j for j in range(k)] for b in range(B)]


def pin_paged_identity_table_is_reshape():
    """With the table that numbers the pages in order, the pool is the dense
    cache reshaped: every sequence reads back its own rows."""
    _, dense, pages, bt = _dense_and_pages()
    for b in range(3):
        close(R.paged_rows(pages, bt, 4, b, 11), dense[b, :11], 0.0)
        assert R.paged_slot(bt, 4, b, 9) == (b * 3 + 2, 1)


def pin_paged_pool_permutation():
    """Moving the pages around the pool with the table updated to match leaves
    every sequence's rows unchanged; a write then a read returns what was
    written and changes no other sequence."""
    rng, dense, pages, bt = _dense_and_pages()
    perm = rng.permutation(9)
    pages2 = np.zeros_like(pages)
    pages2[perm] = pages
    bt2 = [[int(perm[p]) for p in row] for row in bt]
    for b in range(3):
        close(R.paged_rows(pages2, bt2, 4, b, 12), dense[b], 0.0)
    rows = rng.standard_normal((5, pages.shape[-1]))
    positions = [0, 3, 4, 7, 11]
    w = R.paged_write(pages2, bt2, 4, 1, positions, rows)
    expect = dense[1].copy()
    expect[positions] = rows
    close(R.paged_rows(w, bt2, 4, 1, 12), expect, 0.0)
    for b in (0, 2):
        close(R.paged_rows(w, bt2, 4, b, 12), dense[b], 0.0)


def pin_decode_paged_is_dense_decode():
    """Decoding against a shuffled paged copy of a cache equals decoding
    against the dense cache, and the new row goes to the slot the table names
    for its position."""
    W = tiny_weights()
    rng = np.random.Generator(np.random.PCG64(6))
    RL = TINY.kv_rank + TINY.d_rope
    lens = np.array([9, 5])
    dense = np.zeros((2, 12, RL))
    dense[0, :9] = rng.standard_normal((9, RL))
    dense[1, :5] = rng.standard_normal((5, RL))
    bt = [[5, 2, 7], [0, 6, 3]]
    pages = np.full((8, 4, RL), np.nan)      # pages and rows nobody owns stay NaN
    for b in range(2):
        for p in range(int(lens[b])):
            pages[bt[b][p // 4], p % 4] = dense[b, p]
    x_new = tiny_x(B=2, L=1)[:, 0]
    for window in (0, 4):
        cfg = replace(TINY, window=window)
        dec = R.gdla_decode_paged(x_new, W, cfg, pages, bt, 4, lens)
        ref = R.gdla_decode(x_new, W, cfg, dense, lens)
        close(dec["y"], ref["y"], 1e-13)
        close(dec["new_rows"], ref["new_rows"], 1e-13)
        assert dec["slots"] == [(7, 1), (6, 1)], dec["slots"]


# ------------------------------------------------------------------ backward
def _fd_check(cfg, pos_offset=0, B=1, L=7, seed=11, per_tensor=6, tol=2e-6):
    """Central differences of the loss sum(dy * y) against the analytic
    gradients of gdla_layer_backward, on sampled elements of x and of every
    weight (fp64, h = 1e-5: truncation error ~1e-10 relative)."""
    W = tiny_weights(cfg, seed=seed)
    x = tiny_x(B=B, L=L, cfg=cfg, seed=seed + 1)
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    dy = rng.standard_normal((B, L, cfg.d_model))
    grads = R.gdla_layer_backward(x, W, cfg, dy, pos_offset=pos_offset)

    def loss(x_, W_):
        return float(np.sum(dy * R.gdla_layer(x_, W_, cfg, pos_offset=pos_offset)["y"]))

    h = 1e-5
    checks = [("dx", x, None)] + [(k, W[k], k) for k in sorted(W)]
    for name, arr, key in checks:
        flat = np.arange(arr.size)
        for idx in rng.choice(flat, size=min(per_tensor, arr.size), replace=False):
            i = np.unravel_index(idx, arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[i] += h
            minus[i] -= h
            if key is None:
                fd = (loss(plus, W) - loss(minus, W)) / (2 * h)
            else:
                fd = (loss(x, dict(W, **{key: plus})) - loss(x, dict(W, **{key: minus}))) / (2 * h)
            got = grads["dx" if key is None else key][i]
            scale = max(1.0, float(np.max(np.abs(grads["dx" if key is None else key]))))
            assert abs(got - fd) <= tol * scale, f"{name}{i}: analytic {got:.9e} vs finite difference {fd:.9e}"


def pin_backward_finite_differences_full():
    """Every gradient of a full-causal layer (x and all nine weights) matches
    central finite differences of sum(dy * y)."""
    _fd_check(TINY, pos_offset=0)


def pin_backward_finite_differences_window_batch():
    """The same for a windowed layer over two sequences at a position offset."""
    _fd_check(replace(TINY, window=3), pos_offset=5, B=2, L=6, seed=21)


def pin_backward_finite_differences_yarn():
    """The same with YaRN frequencies and the cos/sin factor on a full layer,
    and with the temperature on the whole logit instead."""
    cfg = replace(TINY, yarn_factor=8.0, yarn_orig_len=8, yarn_beta_fast=32.0, yarn_beta_slow=1.0)
    _fd_check(cfg, pos_offset=3, seed=31)
    _fd_check(replace(cfg, yarn_temperature="logit"), pos_offset=3, seed=32)


def pin_packed_backward_finite_differences():
    """The packed backward ([M3-pack] in the training pass) against central
    finite differences of sum(dy * y) through the packed forward: x and every
    weight, a stream of PACK_LENS (one sequence empty) at PACK_POS, full
    causal and windowed."""
    cu, x = _pack(PACK_LENS, seed=51)
    rng = np.random.Generator(np.random.PCG64(52))
    dy = rng.standard_normal(x.shape)
    h = 1e-5
    for cfg in (TINY, replace(TINY, window=2)):
        W = tiny_weights(cfg, seed=53)
        grads = R.gdla_layer_packed_backward(x, W, cfg, dy, cu, PACK_POS)

        def loss(x_, W_):
            return float(np.sum(dy * R.gdla_layer_packed(x_, W_, cfg, cu, PACK_POS)["y"]))

        for name, arr, key in [("dx", x, None)] + [(k, W[k], k) for k in sorted(W)]:
            for idx in rng.choice(np.arange(arr.size), size=min(5, arr.size), replace=False):
                i = np.unravel_index(idx, arr.shape)
                plus, minus = arr.copy(), arr.copy()
                plus[i] += h
                minus[i] -= h
                if key is None:
                    fd = (loss(plus, W) - loss(minus, W)) / (2 * h)
                else:
                    fd = (loss(x, dict(W, **{key: plus})) - loss(x, dict(W, **{key: minus}))) / (2 * h)
                got = grads["dx" if key is None else key][i]
                scale = max(1.0, float(np.max(np.abs(grads["dx" if key is None else key]))))
                assert abs(got - fd) <= 2e-6 * scale, f"packed {name}{i}: analytic {got:.9e} vs {fd:.9e}"


def pin_packed_backward_equal_lengths_is_the_batch():
    """Equal lengths packed end to end are the batched layer: dx is the
    batched dx row for row and each weight gradient the batched one (the
    batch sums over its sequences)."""
    B, L = 3, 5
    W = tiny_weights(seed=54)
    x = tiny_x(B=B, L=L, seed=55)
    dy = np.random.Generator(np.random.PCG64(56)).standard_normal(x.shape)
    cu = [i * L for i in range(B + 1)]
    for cfg in (TINY, replace(TINY, window=2)):
        batched = R.gdla_layer_backward(x, W, cfg, dy, pos_offset=4)
        packed = R.gdla_layer_packed_backward(x.reshape(B * L, -1), W, cfg, dy.reshape(B * L, -1), cu, [4] * B)
        close(packed["dx"], batched["dx"].reshape(B * L, -1), 1e-12)
        for k in W:
            close(packed[k], batched[k], 1e-12)


def pin_rope_backward_is_adjoint():
    """<rope(u), g> = <u, rope_backward(g)> for plain and YaRN frequencies."""
    rng = np.random.Generator(np.random.PCG64(41))
    u = rng.standard_normal((3, 9, 8))
    g = rng.standard_normal((3, 9, 8))
    pos = np.arange(9) * 3.0 + 1.0
    for yarn in (None, (16.0, 4.0, 32.0, 1.0)):
        a = float(np.sum(R.rope(u, pos, 100.0, yarn) * g))
        b = float(np.sum(u * R.rope_backward(g, pos, 100.0, yarn)))
        assert abs(a - b) <= 1e-12 * max(1.0, abs(a)), (a, b)


def pin_rms_norm_backward_finite_differences():
    """RMSNorm's input and gain gradients against central differences."""
    rng = np.random.Generator(np.random.PCG64(43))
    c = rng.standard_normal((4, 10))
    gamma = 1.0 + 0.3 * rng.standard_normal(10)
    g = rng.standard_normal((4, 10))
    dc, dgamma = R.rms_norm_backward(c, gamma, 1e-3, g)
    h = 1e-6
    for i in range(4):
        for j in range(10):
            p, m = c.copy(), c.copy()
            p[i, j] += h
            m[i, j] -= h
            fd = (np.sum(g * R.rms_norm(p, gamma, 1e-3)) - np.sum(g * R.rms_norm(m, gamma, 1e-3))) / (2 * h)
            assert abs(fd - dc[i, j]) < 1e-8, (i, j, fd, dc[i, j])
    for j in range(10):
        p, m = gamma.copy(), gamma.copy()
        p[j] += h
        m[j] -= h
        fd = (np.sum(g * R.rms_norm(c, p, 1e-3)) - np.sum(g * R.rms_norm(c, m, 1e-3))) / (2 * h)
        assert abs(fd - dgamma[j]) < 1e-8, (j, fd, dgamma[j])


def pin_backward_rows_equals_sparse_dy():
    """The row-restricted backward (upstream gradient on a few rows) equals
    the full backward with dy zero on every other row."""
    W = tiny_weights(seed=51)
    x = tiny_x(B=2, L=9, seed=52)
    rng = np.random.Generator(np.random.PCG64(53))
    rows = [0, 4, 5, 8]
    dy_rows = rng.standard_normal((2, len(rows), TINY.d_model))
    dy = np.zeros((2, 9, TINY.d_model))
    dy[:, rows] = dy_rows
    for window in (0, 3):
        cfg = replace(TINY, window=window)
        full = R.gdla_layer_backward(x, W, cfg, dy, pos_offset=2)
        part = R.gdla_layer_backward(x, W, cfg, dy_rows, pos_offset=2, rows=rows)
        for k in full:
            close(part[k], full[k], 1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
