"""Pins of the oracle's reverse mode (gradients of eqs (1)-(4) of the picx.dev
summary of "On the Design of Qwen3.8-Next Architecture", "Theoretical
foundations") against what the mathematics fixes.  CPU only.

The loss is L = sum_t <dy_t, y_t> + <dST, S_T>, so the oracle's outputs are the
partial derivatives of L.  Pins:

* central finite differences of the FORWARD oracle, every element of every
  input, with and without an initial state and a final-state gradient;
* the one-token closed form, derived by hand from y = alpha S0^T q +
  beta (q.k)(v - alpha S0^T k);
* homogeneity: y and S_T are jointly linear in (v, S0), and y is linear in q
  with S_T independent of q, so <dv, v> + <dS0, S0> = L and <dq, q> = sum <dy, y>
  (Euler's theorem), at sizes finite differences cannot reach;
* alpha = 1, beta = 0 freezes the state: dS0 = sum_t q_t dy_t^T + dST and
  dk = dv = 0;
* the chunkwise reverse mode of tests/chunked_reference.py agrees.
"""
import numpy as np
import pytest

from chunked_reference import chunked_gdn_bwd

NAMES = ("q", "k", "v", "alpha", "beta", "S0")
GRADS = dict(q="dq", k="dk", v="dv", alpha="dalpha", beta="dbeta", S0="dS0")


def _inputs(rng, B, T, H, Dk, Dv):
    q = rng.standard_normal((B, T, H, Dk)) * 0.6
    k = rng.standard_normal((B, T, H, Dk)) * 0.6
    v = rng.standard_normal((B, T, H, Dv))
    alpha = rng.uniform(0.4, 0.99, (B, T, H))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    dy = rng.standard_normal((B, T, H, Dv))
    dST = rng.standard_normal((B, H, Dk, Dv))
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0), dy, dST


def _loss(om, x, dy, dST):
    y, ST = om.gdn_recurrence(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    return float((y * dy).sum() + (0.0 if dST is None else (ST * dST).sum()))


def _fd_check(om, x, dy, dST, h=1e-6, tol=1e-7):
    g = om.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], dy, dST)
    for n in NAMES:
        if x[n] is None:
            continue
        fd = np.zeros_like(x[n])
        for i in np.ndindex(x[n].shape):
            xp = dict(x); xp[n] = x[n].copy(); xp[n][i] += h
            xm = dict(x); xm[n] = x[n].copy(); xm[n][i] -= h
            fd[i] = (_loss(om, xp, dy, dST) - _loss(om, xm, dy, dST)) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        err = np.abs(fd - g[GRADS[n]]).max() / scale
        assert err < tol, f"d{n}: finite differences differ by {err:.2e}"


def test_bwd_finite_differences(oracle_mod):
    rng = np.random.default_rng(31)
    x, dy, dST = _inputs(rng, 1, 6, 2, 3, 2)
    _fd_check(oracle_mod, x, dy, dST)


def test_bwd_finite_differences_no_state(oracle_mod):
    """S0 = None and dST = None: zero initial state, no final-state term; dS0 is
    still the gradient at S0 = 0 (checked against an explicit zero state)."""
    rng = np.random.default_rng(32)
    x, dy, _ = _inputs(rng, 2, 4, 1, 2, 3)
    x["S0"] = None
    _fd_check(oracle_mod, x, dy, None)
    g0 = oracle_mod.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], None, dy, None)
    z = np.zeros((2, 1, 2, 3))
    gz = oracle_mod.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], z, dy, z)
    for n in GRADS.values():
        np.testing.assert_array_equal(g0[n], gz[n])


def test_bwd_finite_differences_long(oracle_mod):
    """More tokens than one checkpoint segment of the oracle's reverse pass."""
    rng = np.random.default_rng(33)
    x, dy, dST = _inputs(rng, 1, 70, 1, 2, 2)
    x["alpha"] = rng.uniform(0.9, 0.999, x["alpha"].shape)
    _fd_check(oracle_mod, x, dy, dST, tol=3e-7)


def test_bwd_one_token_closed_form(oracle_mod):
    rng = np.random.default_rng(34)
    Dk, Dv = 5, 3
    q, k = rng.standard_normal((2, Dk))
    v, dy = rng.standard_normal((2, Dv))
    S0 = rng.standard_normal((Dk, Dv))
    a, b = 0.7, 0.35
    e = v - a * (S0.T @ k)
    qk = q @ k
    ref = dict(
        dq=a * (S0 @ dy) + b * k * (dy @ e),
        dk=b * q * (dy @ e) - a * b * qk * (S0 @ dy),
        dv=b * qk * dy,
        dbeta=qk * (dy @ e),
        dalpha=dy @ (S0.T @ q) - b * qk * (dy @ (S0.T @ k)),
        dS0=a * np.outer(q, dy) - a * b * qk * np.outer(k, dy),
    )
    g = oracle_mod.gdn_recurrence_bwd(q.reshape(1, 1, 1, Dk), k.reshape(1, 1, 1, Dk), v.reshape(1, 1, 1, Dv),
                                      np.full((1, 1, 1), a), np.full((1, 1, 1), b), S0.reshape(1, 1, Dk, Dv),
                                      dy.reshape(1, 1, 1, Dv), None)
    for n, r in ref.items():
        np.testing.assert_allclose(g[n].reshape(np.shape(r)), r, rtol=1e-13, atol=1e-13, err_msg=n)


def test_bwd_homogeneity(oracle_mod):
    rng = np.random.default_rng(35)
    x, dy, dST = _inputs(rng, 2, 150, 3, 8, 6)
    y, ST = oracle_mod.gdn_recurrence(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
    g = oracle_mod.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], dy, dST)
    Ly, LS = (y * dy).sum(), (ST * dST).sum()
    lin = (g["dv"] * x["v"]).sum() + (g["dS0"] * x["S0"]).sum()
    assert abs(lin - (Ly + LS)) < 1e-10 * (abs(Ly) + abs(LS))
    assert abs((g["dq"] * x["q"]).sum() - Ly) < 1e-10 * abs(Ly)


def test_bwd_frozen_state(oracle_mod):
    rng = np.random.default_rng(36)
    x, dy, dST = _inputs(rng, 1, 9, 2, 4, 3)
    x["alpha"] = np.ones_like(x["alpha"])
    x["beta"] = np.zeros_like(x["beta"])
    g = oracle_mod.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], dy, dST)
    ref = np.einsum("bthk,bthv->bhkv", x["q"], dy) + dST
    np.testing.assert_allclose(g["dS0"], ref, rtol=1e-13, atol=1e-13)
    assert not g["dk"].any() and not g["dv"].any()
    # dq_t = S0 dy_t while the state stays S0
    np.testing.assert_allclose(g["dq"], np.einsum("bhkv,bthv->bthk", x["S0"], dy), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("shape", [(1, 37, 2, 5, 7, 8), (2, 40, 1, 8, 8, 16), (1, 13, 1, 6, 3, 4),
                                   (1, 64, 1, 16, 16, 16)])
def test_bwd_chunked_form_agrees(oracle_mod, shape):
    B, T, H, Dk, Dv, C = shape
    rng = np.random.default_rng(T + C)
    x, dy, dST = _inputs(rng, B, T, H, Dk, Dv)
    g = oracle_mod.gdn_recurrence_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], dy, dST)
    c = chunked_gdn_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], dy, dST, C)
    for n in GRADS.values():
        err = np.abs(g[n] - c[n]).max() / np.abs(g[n]).max()
        assert err < 1e-12, (n, err)
