"""Pins of the oracle's layer wrapper (picx.dev summary of "On the Design of
Qwen3.8-Next Architecture", "1. GDN Hybrid Token Mixing": short causal
convolution, L2-normalised q/k, eqs (9)-(11)).  CPU only.

Each stage is checked against a library routine, a closed form or a special
case; the full layer is checked for causality and for its reduction to the
core recurrence when the wrapper is made trivial.
"""
import numpy as np
import pytest
import scipy.special as sps


def test_l4_decay_closed_form(oracle_mod):
    """A = b_alpha = 0: exp(-softplus(a)) = sigmoid(-a) exactly (scipy expit)."""
    a = np.linspace(-12, 12, 97)
    got = oracle_mod.decay(a[:, None], np.zeros(1), np.zeros(1))[:, 0]
    np.testing.assert_allclose(got, sps.expit(-a), rtol=1e-13, atol=1e-300)
    # general A, b: compare with numpy's logaddexp for softplus
    A = np.array([0.3]); ba = np.array([-0.7])
    got = oracle_mod.decay(a[:, None], A, ba)[:, 0]
    np.testing.assert_allclose(got, np.exp(-np.exp(0.3) * np.logaddexp(0.0, a - 0.7)), rtol=1e-13)


def test_write_strength_is_sigmoid(oracle_mod):
    b = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle_mod.write_strength(b), sps.expit(b), rtol=1e-14, atol=1e-300)


def test_l2_normalise_examples(oracle_mod):
    x = np.array([[3.0, 4.0], [0.0, 0.0]])
    got = oracle_mod.l2_normalize(x, eps=0.0 + 1e-300)
    np.testing.assert_allclose(got[0], [0.6, 0.8], rtol=1e-15)
    assert np.all(got[1] == 0)
    rng = np.random.default_rng(0)
    y = oracle_mod.l2_normalize(rng.standard_normal((5, 3, 128)) * 7.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-7)


def test_l3_rmsnorm_unit_rms_and_gain(oracle_mod):
    rng = np.random.default_rng(1)
    y = rng.standard_normal((4, 6, 32)) * 3.0
    out = oracle_mod.rmsnorm_zero_centred(y, np.zeros(32))
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-6)
    # constant vector c -> sign(c) (1+gamma) up to eps; gamma is zero-centred
    g = rng.standard_normal(32) * 0.1
    const = np.full((1, 32), -2.5)
    np.testing.assert_allclose(oracle_mod.rmsnorm_zero_centred(const, g)[0], -(1 + g), rtol=1e-6)


def test_l5_zero_gate_weight_halves(oracle_mod):
    np.testing.assert_array_equal(oracle_mod.sigmoid(np.zeros(5)), 0.5)


def test_l6_conv_taps_are_shifts(oracle_mod):
    """A one-hot filter on tap j delays the channel by K-1-j tokens."""
    rng = np.random.default_rng(2)
    u = rng.standard_normal((2, 9, 5))
    K = 4
    for j in range(K):
        w = np.zeros((5, K)); w[:, j] = 1.0
        out = oracle_mod.causal_depthwise_conv(u, w)
        lag = K - 1 - j
        ref = np.zeros_like(u)
        ref[:, lag:] = u[:, :9 - lag]
        np.testing.assert_array_equal(out, ref)


def test_conv_matches_numpy_convolve(oracle_mod):
    """Per channel the causal conv is numpy's full convolution with the
    reversed filter, truncated to the first T outputs."""
    rng = np.random.default_rng(3)
    u = rng.standard_normal((1, 12, 3))
    w = rng.standard_normal((3, 4))
    out = oracle_mod.causal_depthwise_conv(u, w)
    for c in range(3):
        ref = np.convolve(u[0, :, c], w[c, ::-1])[:12]
        np.testing.assert_allclose(out[0, :, c], ref, rtol=1e-13, atol=1e-14)


def _small_layer(rng, B=2, T=21, hidden=24, H=2, Dk=4, Dv=6, K=4):
    n = H * (2 * Dk + Dv)
    return dict(
        x=rng.standard_normal((B, T, hidden)),
        W_qkv=rng.standard_normal((n, hidden)) * 0.3,
        conv_w=rng.uniform(-0.5, 0.5, (n, K)),
        W_ab=rng.standard_normal((2 * H, hidden)) * 0.3,
        A=rng.standard_normal(H) * 0.2,
        b_alpha=rng.standard_normal(H) * 0.2,
        W_gate=rng.standard_normal((H * Dv, hidden)) * 0.3,
        norm_gamma=rng.standard_normal(Dv) * 0.1,
        W_o=rng.standard_normal((hidden, H * Dv)) * 0.3,
    ), (H, Dk, Dv)


def test_l1_layer_is_causal(oracle_mod):
    rng = np.random.default_rng(4)
    p, (H, Dk, Dv) = _small_layer(rng)
    o, _ = oracle_mod.gdn_layer_fwd(H=H, Dk=Dk, Dv=Dv, **p)
    t = 9
    p2 = dict(p)
    x2 = p["x"].copy()
    x2[:, t + 1:] += rng.standard_normal(x2[:, t + 1:].shape)
    p2["x"] = x2
    o2, _ = oracle_mod.gdn_layer_fwd(H=H, Dk=Dk, Dv=Dv, **p2)
    np.testing.assert_array_equal(o2[:, :t + 1], o[:, :t + 1])
    assert np.abs(o2[:, t + 1:] - o[:, t + 1:]).max() > 1e-3


def test_layer_reduces_to_core(oracle_mod):
    """With identity-like in-projection, current-tap-only conv and the parts it
    returns, the layer's core call sees exactly the normalised conv outputs,
    the gates follow eqs (9)-(10), and o equals W_o(sigmoid(z) * RMSNorm(y))."""
    rng = np.random.default_rng(5)
    p, (H, Dk, Dv) = _small_layer(rng, B=1, T=8)
    p["conv_w"][:] = 0.0
    p["conv_w"][:, -1] = 1.0
    parts = oracle_mod.gdn_layer_fwd(H=H, Dk=Dk, Dv=Dv, return_parts=True, **p)
    qkv = p["x"] @ p["W_qkv"].T
    np.testing.assert_allclose(parts["conv"], qkv, rtol=1e-13)
    qn = qkv[..., :H * Dk].reshape(1, 8, H, Dk)
    qn = qn / np.linalg.norm(qn, axis=-1, keepdims=True)
    np.testing.assert_allclose(parts["q"], qn, rtol=1e-6)
    y, _ = oracle_mod.gdn_recurrence(parts["q"], parts["k"], parts["v"], parts["alpha"], parts["beta"])
    np.testing.assert_array_equal(parts["y"], y)
    z = p["x"] @ p["W_gate"].T
    g = sps.expit(z).reshape(1, 8, H, Dv) * parts["yn"]
    np.testing.assert_allclose(parts["o"], g.reshape(1, 8, H * Dv) @ p["W_o"].T, rtol=1e-12)


def _layer_params(oracle_mod, inp):
    from linear_attention_token_gated_amd import workloads as wl
    names = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")
    return [wl.widen(inp[n]) for n in names]


@pytest.mark.parametrize("conv_k", [1, 2, 4])
def test_layer_decode_steps_equal_layer(oracle_mod, conv_k):
    """T single-token steps of the layer from an empty history and a given state
    reproduce the whole-sequence layer on those T tokens (same section, computed
    by an independent route: conv over a carried window, recurrence one token at
    a time)."""
    from linear_attention_token_gated_amd import workloads as wl
    B, T, hidden, H, Dk, Dv = 2, 9, 64, 2, 8, 4
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=conv_k, w_std=0.2, seed=5 + conv_k,
                          gamma_std=0.2, A_val=0.4, b_alpha_val=-0.3)
    P = _layer_params(oracle_mod, inp)
    x = wl.widen(inp["x"])
    S0 = np.random.default_rng(2).standard_normal((B, H, Dk, Dv)) * 0.3
    o_ref, S_ref = oracle_mod.gdn_layer_fwd(x, *P, H=H, Dk=Dk, Dv=Dv, S0=S0)
    Ch = H * (2 * Dk + Dv)
    conv_state = np.zeros((B, conv_k - 1, Ch))
    S = S0.copy()
    for t in range(T):
        o, conv_state, S = oracle_mod.gdn_layer_decode_step(x[:, t], *P, H=H, Dk=Dk, Dv=Dv,
                                                            conv_state=conv_state, S=S)
        np.testing.assert_allclose(o, o_ref[:, t], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-10, atol=1e-12)
    # the carried window holds the last conv_k-1 in-projection rows
    qkv = oracle_mod.linear(x, P[0])
    if conv_k > 1:
        np.testing.assert_allclose(conv_state, qkv[:, T - (conv_k - 1):], rtol=1e-13, atol=1e-13)


def test_layer_decode_step_leaves_inputs(oracle_mod):
    from linear_attention_token_gated_amd import workloads as wl
    B, hidden, H, Dk, Dv = 3, 64, 1, 8, 8
    inp = wl.layer_inputs(B, 1, hidden, H, Dk, Dv, conv_k=4, w_std=0.2, seed=1)
    P = _layer_params(oracle_mod, inp)
    cs = np.random.default_rng(0).standard_normal((B, 3, H * (2 * Dk + Dv)))
    S = np.random.default_rng(1).standard_normal((B, H, Dk, Dv))
    cs0, S0 = cs.copy(), S.copy()
    oracle_mod.gdn_layer_decode_step(wl.widen(inp["x"])[:, 0], *P, H=H, Dk=Dk, Dv=Dv, conv_state=cs, S=S)
    assert np.array_equal(cs, cs0) and np.array_equal(S, S0)
