"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is checked against closed forms,
special cases that reduce to a library routine, invariants of the recurrence
and a hand-worked example; none of them re-types the oracle's loop.

Source of the recurrence: "On the Design of Qwen3.8-Next Architecture", picx.dev
summary, section "Theoretical foundations", eqs (1)-(4) (alpha, beta in (0,1);
eq (3) adds beta k e^T, where e is the prediction error of eq (2)).  Non-square d_k != d_v shapes
are used throughout so that a transposed state cannot pass.
"""
import numpy as np
import pytest

from chunked_reference import chunked_gdn


def _rand_inputs(rng, B, T, H, Dk, Dv, unit_keys=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    alpha = 1.0 / (1.0 + np.exp(-rng.uniform(0.5, 6.9, (B, T, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.3 * rng.standard_normal((B, H, Dk, Dv))
    return q, k, v, alpha, beta, S0


def test_worked_example_by_hand(oracle_mod):
    """Two tokens, d_k=2, d_v=1, S0=0, worked by hand from eqs (1)-(4).

    t=1: k=(1,0), v=2, alpha=0.5, beta=0.5, q=(1,1)
         S~=0, e=2, S1=0.5*(1,0)^T*2=(1,0)^T, y1=S1^T q=1
    t=2: k=(0.6,0.8), v=1, alpha=0.5, beta=1, q=(0,1)
         S~=(0.5,0)^T, e=1-0.3=0.7, S2=(0.5+0.42, 0.56)^T=(0.92,0.56)^T, y2=0.56
    """
    q = np.array([[1.0, 1.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    k = np.array([[1.0, 0.0], [0.6, 0.8]]).reshape(1, 2, 1, 2)
    v = np.array([2.0, 1.0]).reshape(1, 2, 1, 1)
    alpha = np.array([0.5, 0.5]).reshape(1, 2, 1)
    beta = np.array([0.5, 1.0]).reshape(1, 2, 1)
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, None)
    np.testing.assert_allclose(y.ravel(), [1.0, 0.56], rtol=0, atol=1e-15)
    np.testing.assert_allclose(ST.ravel(), [0.92, 0.56], rtol=0, atol=1e-15)


def test_p1_identity_steps(oracle_mod):
    """alpha=1, beta=0: S_t = S0 for every t and y_t = S0^T q_t (library matvec)."""
    rng = np.random.default_rng(1)
    q, k, v, _, _, S0 = _rand_inputs(rng, 2, 9, 3, 5, 7)
    a = np.ones((2, 9, 3))
    b = np.zeros((2, 9, 3))
    y, ST = oracle_mod.gdn_recurrence(q, k, v, a, b, S0)
    np.testing.assert_array_equal(ST, S0)
    ref = np.einsum("bhkv,bthk->bthv", S0, q)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)


def test_p2_delta_writes_residual_exactly(oracle_mod):
    """beta=1 and unit keys make the written state reproduce v_t at k_t, for any
    decay and any prior state: S_t^T k_t = v_t.  With q_t = k_t this shows up in
    y_t directly, token by token."""
    rng = np.random.default_rng(2)
    _, k, v, alpha, _, S0 = _rand_inputs(rng, 2, 17, 2, 6, 4)
    beta = np.ones_like(alpha)
    y, _ = oracle_mod.gdn_recurrence(k, k, v, alpha, beta, S0)
    np.testing.assert_allclose(y, v, rtol=1e-12, atol=1e-12)


def test_p3_orthonormal_retrieval(oracle_mod):
    """alpha=1, beta=1, orthonormal keys k_1..k_T (T <= d_k): S_T^T k_j = v_j for
    every j, whatever S0; with a general decay the retrieved value is
    (prod_{i>j} alpha_i) v_j."""
    rng = np.random.default_rng(3)
    Dk, Dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm[:, :T].T                                  # T orthonormal rows
    k = keys.reshape(1, T, 1, Dk)
    v = rng.standard_normal((1, T, 1, Dv))
    q = rng.standard_normal((1, T, 1, Dk))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    _, ST = oracle_mod.gdn_recurrence(q, k, v, np.ones((1, T, 1)), np.ones((1, T, 1)), S0)
    np.testing.assert_allclose(keys @ ST[0, 0], v[0, :, 0], rtol=1e-12, atol=1e-12)

    alpha = rng.uniform(0.5, 0.99, (1, T, 1))
    _, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, np.ones((1, T, 1)), S0)
    a = alpha[0, :, 0]
    for j in range(T):
        decay_after = np.prod(a[j + 1:])
        np.testing.assert_allclose(keys[j] @ ST[0, 0], decay_after * v[0, j, 0], rtol=1e-12, atol=1e-12)


def test_p4_orthogonal_keys_decayed_linear_attention(oracle_mod):
    """S0 = 0 and mutually orthogonal (not unit) keys: the prediction error is
    v_t itself, and y_t = sum_{j<=t} (prod_{i=j+1..t} alpha_i) beta_j (k_j.q_t) v_j
    (an O(T^2) brute force)."""
    rng = np.random.default_rng(4)
    Dk, Dv, T = 7, 3, 7
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    keys = Qm.T * rng.uniform(0.3, 1.7, (Dk, 1))           # orthogonal rows, mixed norms
    k = keys[:T].reshape(1, T, 1, Dk)
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    alpha = rng.uniform(0.3, 0.99, (1, T, 1))
    beta = rng.uniform(0.05, 0.95, (1, T, 1))
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, None)
    a, bt = alpha[0, :, 0], beta[0, :, 0]
    for t in range(T):
        ref = np.zeros(Dv)
        for j in range(t + 1):
            ref += np.prod(a[j + 1:t + 1]) * bt[j] * (keys[j] @ q[0, t, 0]) * v[0, j, 0]
        np.testing.assert_allclose(y[0, t, 0], ref, rtol=1e-12, atol=1e-13)
    Sref = sum(np.prod(a[j + 1:]) * bt[j] * np.outer(keys[j], v[0, j, 0]) for j in range(T))
    np.testing.assert_allclose(ST[0, 0], Sref, rtol=1e-12, atol=1e-13)


def test_p5_pure_decay(oracle_mod):
    """beta = 0: S_t = (prod_{i<=t} alpha_i) S0 and y_t = (prod alpha) S0^T q_t."""
    rng = np.random.default_rng(5)
    q, k, v, alpha, _, S0 = _rand_inputs(rng, 1, 11, 2, 4, 6)
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, np.zeros_like(alpha), S0)
    cum = np.cumprod(alpha, axis=1)                               # [B, T, H]
    np.testing.assert_allclose(ST, cum[:, -1, :, None, None] * S0, rtol=1e-13)
    ref = cum[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_p6_linear_in_state_and_values(oracle_mod):
    rng = np.random.default_rng(6)
    q, k, v1, alpha, beta, S1 = _rand_inputs(rng, 1, 13, 2, 5, 3)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    c1, c2 = 0.7, -1.3
    ya, Sa = oracle_mod.gdn_recurrence(q, k, v1, alpha, beta, S1)
    yb, Sb = oracle_mod.gdn_recurrence(q, k, v2, alpha, beta, S2)
    yc, Sc = oracle_mod.gdn_recurrence(q, k, c1 * v1 + c2 * v2, alpha, beta, c1 * S1 + c2 * S2)
    np.testing.assert_allclose(yc, c1 * ya + c2 * yb, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sc, c1 * Sa + c2 * Sb, rtol=1e-11, atol=1e-12)


def test_p7_columns_independent(oracle_mod):
    """Column j of (S_T, Y) depends only on column j of (S0, V)."""
    rng = np.random.default_rng(7)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 10, 2, 6, 8)
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0)
    cols = [1, 4, 7]
    ys, Ss = oracle_mod.gdn_recurrence(q, k, v[..., cols], alpha, beta, S0[..., cols])
    np.testing.assert_allclose(ys, y[..., cols], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Ss, ST[..., cols], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("form", ["W", "R"])
@pytest.mark.parametrize("C", [1, 2, 3, 4, 8, 16])
def test_p8_p9_chunked_algebra_matches_sequential(oracle_mod, C, form):
    """The chunkwise algebra (independent numpy fp64) equals the token-by-token
    oracle for every chunk size, including a ragged tail chunk."""
    rng = np.random.default_rng(100 + C)
    for T, Dk, Dv in [(37, 5, 7), (40, 8, 8), (13, 6, 3), (1, 4, 2)]:
        q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, T, 2, Dk, Dv)
        y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0)
        yc, Sc = chunked_gdn(q, k, v, alpha, beta, S0, C, form=form)
        np.testing.assert_allclose(yc, y, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(Sc, ST, rtol=1e-10, atol=1e-12)


def test_p10_split_and_resume(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 29, 3, 4, 6)
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0)
    T1 = 11
    y1, S1 = oracle_mod.gdn_recurrence(q[:, :T1], k[:, :T1], v[:, :T1], alpha[:, :T1], beta[:, :T1], S0)
    y2, S2 = oracle_mod.gdn_recurrence(q[:, T1:], k[:, T1:], v[:, T1:], alpha[:, T1:], beta[:, T1:], S1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(S2, ST)


def test_p11_decode_equals_one_token_prefill(oracle_mod):
    rng = np.random.default_rng(11)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 5, 1, 3, 6, 4)
    y, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0)
    yd, Sd = oracle_mod.gdn_decode_step(q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], S0)
    np.testing.assert_array_equal(yd, y[:, 0])
    np.testing.assert_array_equal(Sd, ST)


def test_p12_identity_padding(oracle_mod):
    """Appending tokens with alpha=1, beta=0 leaves the final state unchanged
    (what a ragged tail chunk relies on)."""
    rng = np.random.default_rng(12)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 9, 2, 5, 3)
    _, ST = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0)
    pad = 7
    qp = np.concatenate([q, rng.standard_normal((1, pad, 2, 5))], axis=1)
    kp = np.concatenate([k, rng.standard_normal((1, pad, 2, 5))], axis=1)
    vp = np.concatenate([v, rng.standard_normal((1, pad, 2, 3))], axis=1)
    ap = np.concatenate([alpha, np.ones((1, pad, 2))], axis=1)
    bp = np.concatenate([beta, np.zeros((1, pad, 2))], axis=1)
    _, STp = oracle_mod.gdn_recurrence(qp, kp, vp, ap, bp, S0)
    np.testing.assert_array_equal(STp, ST)


def test_contractive_state_norm(oracle_mod):
    """With unit keys, beta in [0,1] and alpha in (0,1], one step cannot grow the
    Frobenius norm of the state beyond |S| + beta |v| (I - beta k k^T is a
    contraction): a bound that a dropped decay or a sign slip would break."""
    rng = np.random.default_rng(13)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 1, 1, 4, 6, 5)
    _, S1 = oracle_mod.gdn_decode_step(q[:, 0], k[:, 0], v[:, 0], alpha[:, 0], beta[:, 0], S0)
    for h in range(4):
        bound = alpha[0, 0, h] * np.linalg.norm(S0[0, h]) + beta[0, 0, h] * np.linalg.norm(v[0, 0, h])
        assert np.linalg.norm(S1[0, h]) <= bound * (1 + 1e-12)


def test_threads_do_not_change_result(oracle_mod):
    rng = np.random.default_rng(14)
    q, k, v, alpha, beta, S0 = _rand_inputs(rng, 2, 20, 4, 8, 8)
    y1, S1 = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0, nthreads=1)
    y4, S4 = oracle_mod.gdn_recurrence(q, k, v, alpha, beta, S0, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(S1, S4)
