"""Pins for the layer part of the float64 oracle (CPU only).

The layer oracle composes pinned pieces (the token recurrence, the chunkwise
core, the gate activation, the conv) in the order "KDAChunkwise" gives in
"From the hidden states to causal Q, K, and V", "FP32 core and log-space
decay" and "Returning to the model dimension". Its composition is pinned here
by cases whose result follows by hand, independently of the oracle's own
composition:
  * a single token, where the core collapses to o = scale * beta * (k . q) v
    and q = k makes k . q = 1 (unit norm);
  * reduced weights (conv taps (0, 0, 0, 1): identity; Wgd = 0: output gate
    exactly 1/2; norm weight 1), where x_new is half the per-head RMS-normed
    output of the token recurrence (oracle R) times Wo^T;
  * with M = H * D and Wo = I, the RMS of every head of x_new is fixed by the
    RMS of the same head of o;
  * RMSNorm of a constant vector: a / sqrt(a^2 + eps) * w.
At the end, plausible mistakes are planted in each layer step and at least
one pin must fail for each.
"""
import numpy as np
import pytest

import oracle.kda_oracle as orc


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _weights(rng, M, H, D, r, rg):
    HD = H * D

    def lin(o, i):
        return rng.standard_normal((o, i)) * i ** -0.5

    return {
        "Wqkv": lin(3 * HD, M), "conv_q": rng.standard_normal((HD, 4)) * 0.7,
        "conv_k": rng.standard_normal((HD, 4)) * 0.7, "conv_v": rng.standard_normal((HD, 4)) * 0.7,
        "Wb": lin(H, M), "Wad": lin(r, M), "Wau": lin(HD, r),
        "A_log": np.log(rng.uniform(1.0, 4.0, size=H)),
        "dt_bias": rng.uniform(-1.0, 1.0, size=HD),
        "Wgd": lin(rg, M), "Wgu": lin(HD, rg), "norm_w": rng.uniform(0.5, 1.5, size=D), "Wo": lin(M, HD),
    }


def _per_head_rmsnorm(o, eps, w=1.0):
    """o: [..., D]; written out here: o / sqrt(mean_D(o^2) + eps) * w."""
    return o / np.sqrt((o ** 2).sum(-1, keepdims=True) / o.shape[-1] + eps) * w


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
def pin_single_token(eps_norm=0.02):
    """T = 1 by hand. q and k share their projection rows and conv taps, so
    q = k, a unit vector per head, and with a zero initial state the core
    gives o = scale * beta * v (the decay acts on a zero state). The conv
    sees three zero pads, so only tap 3 touches the token."""
    rng = np.random.default_rng(7)
    M, H, D, r, rg = 12, 3, 4, 4, 5
    HD = H * D
    w = _weights(rng, M, H, D, r, rg)
    w["Wqkv"][HD:2 * HD] = w["Wqkv"][:HD]
    w["conv_k"] = w["conv_q"].copy()
    x = rng.standard_normal((1, 1, M))
    P = x[0, 0] @ w["Wqkv"].T
    qf = _silu(w["conv_q"][:, 3] * P[:HD]).reshape(H, D)
    qf = qf / np.linalg.norm(qf, axis=-1, keepdims=True)
    v = _silu(w["conv_v"][:, 3] * P[2 * HD:]).reshape(H, D)
    beta = _sig(x[0, 0] @ w["Wb"].T)
    o = D ** -0.5 * beta[:, None] * (qf * qf).sum(-1, keepdims=True) * v
    gate = _sig((x[0, 0] @ w["Wgd"].T) @ w["Wgu"].T).reshape(H, D)
    y = _per_head_rmsnorm(o, eps_norm, w["norm_w"]) * gate
    expect = y.reshape(HD) @ w["Wo"].T
    got, inter = orc.kda_layer_ref(x, w, H, D, chunk_size=64, norm_eps=eps_norm)
    assert np.max(np.abs(inter["o"][0, 0] - o)) <= 1e-13 * np.max(np.abs(o))
    assert np.max(np.abs(got[0, 0] - expect)) <= 1e-12 * np.max(np.abs(expect))


def _reduced(seed, M, H, D, T, r=4, rg=6, wo_identity=False):
    rng = np.random.default_rng(seed)
    w = _weights(rng, M, H, D, r, rg)
    tap = np.zeros((H * D, 4))
    tap[:, 3] = 1.0
    w["conv_q"], w["conv_k"], w["conv_v"] = tap, tap.copy(), tap.copy()
    w["Wgd"] = np.zeros_like(w["Wgd"])
    w["norm_w"] = np.ones(D)
    if wo_identity:
        assert M == H * D
        w["Wo"] = np.eye(M)
    x = rng.standard_normal((1, T, M))
    return x, w


def pin_reduced_weights(eps_norm=0.05):
    """Identity conv, output gate 1/2, unit norm weight: x_new is half the
    per-head RMS-normed output of the token recurrence (oracle R) times Wo^T,
    with R fed l2norm(SiLU(x Wq^T)), l2norm(SiLU(x Wk^T)), SiLU(x Wv^T), the
    lower-bound gate and sigmoid(x Wb^T). Checks time and head axes, the
    SiLU / L2 order and the core's inputs."""
    M, H, D, T = 10, 2, 4, 40
    HD = H * D
    x, w = _reduced(11, M, H, D, T)
    P = x @ w["Wqkv"].T
    q = _silu(P[..., :HD]).reshape(1, T, H, D)
    k = _silu(P[..., HD:2 * HD]).reshape(1, T, H, D)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    v = _silu(P[..., 2 * HD:]).reshape(1, T, H, D)
    beta = _sig(x @ w["Wb"].T)
    raw = ((x @ w["Wad"].T) @ w["Wau"].T).reshape(1, T, H, D)
    g = orc.gate_activation(raw, w["A_log"], w["dt_bias"].reshape(H, D), "lower_bound_sigmoid", -5.0)
    o, _ = orc.kda_recurrent(q, k, v, g, beta, D ** -0.5)
    expect = (0.5 * _per_head_rmsnorm(o, eps_norm)).reshape(1, T, HD) @ w["Wo"].T
    got, inter = orc.kda_layer_ref(x, w, H, D, chunk_size=16, norm_eps=eps_norm)
    assert np.max(np.abs(inter["o"] - o)) <= 1e-10 * np.max(np.abs(o))
    assert np.max(np.abs(got - expect)) <= 1e-10 * np.max(np.abs(expect))


def pin_head_rms(eps_norm=0.01):
    """M = H D, Wo = I, gate 1/2, norm weight 1: every head of x_new has RMS
    1/2 sqrt(ms / (ms + eps)), ms the mean square of the same head of o. The
    heads' scales differ, so a norm over H * D breaks it."""
    H, D, T = 3, 4, 24
    x, w = _reduced(12, H * D, H, D, T, wo_identity=True)
    w["Wqkv"][2 * H * D:2 * H * D + D] *= 6.0       # head 0 of v much larger than the others
    got, inter = orc.kda_layer_ref(x, w, H, D, chunk_size=8, norm_eps=eps_norm)
    ms = (inter["o"] ** 2).mean(-1)
    rms = np.sqrt((got.reshape(1, T, H, D) ** 2).mean(-1))
    assert np.allclose(rms, 0.5 * np.sqrt(ms / (ms + eps_norm)), rtol=1e-12, atol=0)


def pin_rms_norm_constant():
    """RMSNorm of a constant vector a * 1: a / sqrt(a^2 + eps) * w, for an eps
    comparable to a^2 (where the eps placement matters)."""
    D = 8
    wt = np.linspace(0.5, 2.0, D)
    for a, eps in ((1e-3, 1e-6), (0.3, 0.09), (2.0, 1e-6)):
        got = orc.rms_norm(np.full((2, D), a), wt, eps)
        assert np.allclose(got, a / np.sqrt(a * a + eps) * wt, rtol=1e-14, atol=0)


def pin_delay_tap():
    """Conv taps (0, 0, 1, 0) delay by one token: v_t = SiLU(p_{t-1}),
    v_0 = SiLU(0) = 0; with taps (0, 0, 0, c), v_t = SiLU(c p_t)."""
    rng = np.random.default_rng(13)
    p = rng.standard_normal((2, 9, 5))
    tap = np.zeros((5, 4))
    tap[:, 2] = 1.0
    out = orc.short_conv_silu(p, tap)
    assert np.all(out[:, 0] == 0.0)
    assert np.allclose(out[:, 1:], _silu(p[:, :-1]), rtol=1e-14, atol=1e-15)
    c = rng.uniform(-3.0, 3.0, size=5)
    tap = np.zeros((5, 4))
    tap[:, 3] = c
    assert np.allclose(orc.short_conv_silu(p, tap), _silu(c * p), rtol=1e-14, atol=1e-15)


LAYER_PINS = [pin_single_token, pin_reduced_weights, pin_head_rms, pin_rms_norm_constant, pin_delay_tap]


@pytest.mark.parametrize("pin", LAYER_PINS, ids=lambda f: f.__name__)
def test_layer_pin(pin):
    pin()


def test_layer_heads_subset_matches_full():
    """heads= restricts the core; its intermediates equal the full run's."""
    rng = np.random.default_rng(14)
    w = _weights(rng, 10, 3, 4, 4, 6)
    x = rng.standard_normal((2, 20, 10))
    _, full = orc.kda_layer_ref(x, w, 3, 4, chunk_size=8)
    none, sub = orc.kda_layer_ref(x, w, 3, 4, chunk_size=8, heads=[2, 0])
    assert none is None
    for n in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(sub[n], full[n][:, :, [2, 0]])
    ref = full["o"][:, :, [2, 0]]
    assert np.max(np.abs(sub["o"] - ref)) <= 1e-13 * np.max(np.abs(ref))


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------
def _layer_pins_pass():
    try:
        for pin in LAYER_PINS:
            pin()
        return True
    except (AssertionError, ValueError):
        return False


def _mut_silu_before_conv(p, conv_w):
    return orc.depthwise_causal_conv(orc.silu(p), conv_w)


def _mut_l2_before_silu(p, conv_w, num_heads, head_dim, eps):
    B, T, _ = p.shape
    c = orc.depthwise_causal_conv(p, conv_w).reshape(B, T, num_heads, head_dim)
    return orc.silu(orc.l2norm(c, eps))


def _mut_norm_over_all_heads(o, weight, eps):
    B, T, H, D = o.shape
    flat = o.reshape(B, T, H * D)
    y = flat / np.sqrt(np.mean(flat * flat, axis=-1, keepdims=True) + eps)
    return y.reshape(B, T, H, D) * np.asarray(weight, np.float64)


def _mut_gate_no_sigmoid(x, Wgd, Wgu, num_heads, head_dim):
    B, T, _ = x.shape
    return ((np.asarray(x, np.float64) @ np.asarray(Wgd).T) @ np.asarray(Wgu).T).reshape(B, T, num_heads, head_dim)


def _mut_gate_swapped(x, Wgd, Wgu, num_heads, head_dim):
    return orig_output_gate(x, Wgu, Wgd, num_heads, head_dim)


orig_output_gate = orc.output_gate


def _mut_eps_outside_root(x, weight, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * np.asarray(weight, np.float64)


def _mut_no_l2(p, conv_w, num_heads, head_dim, eps):
    B, T, _ = p.shape
    return orc.short_conv_silu(p, conv_w).reshape(B, T, num_heads, head_dim)


def _mut_no_dt_bias(x, w, num_heads, head_dim, lower_bound):
    B, T, _ = x.shape
    raw = (np.asarray(x, np.float64) @ np.asarray(w["Wad"]).T) @ np.asarray(w["Wau"]).T
    return orc.gate_activation(raw.reshape(B, T, num_heads, head_dim), w["A_log"], None, "lower_bound_sigmoid",
                               lower_bound)


@pytest.mark.parametrize("name,fn", [
    ("short_conv_silu", _mut_silu_before_conv),
    ("qk_features", _mut_l2_before_silu),
    ("qk_features", _mut_no_l2),
    ("head_rms_norm", _mut_norm_over_all_heads),
    ("output_gate", _mut_gate_no_sigmoid),
    ("output_gate", _mut_gate_swapped),
    ("rms_norm", _mut_eps_outside_root),
    ("decay_gate", _mut_no_dt_bias),
], ids=["silu_before_conv", "l2_before_silu", "no_l2", "norm_over_HD", "gate_no_sigmoid", "Wgd_Wgu_swapped",
        "eps_outside_root", "no_dt_bias"])
def test_layer_planted_mistake_is_caught(monkeypatch, name, fn):
    assert _layer_pins_pass()
    monkeypatch.setattr(orc, name, fn)
    assert not _layer_pins_pass(), f"a mistake planted in {name} went unnoticed"
