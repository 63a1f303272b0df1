"""Independent fp64 numpy implementation of the chunkwise form of the gated
delta rule, used only to pin the algebra that the GPU prefill kernel follows
against the token-by-token oracle (test-only; imports nothing from the oracle
or from the GPU package).

Derivation, per (batch, head), for one chunk of tokens r = 1..C entering with
state S (from "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
"Theoretical foundations", eqs (1)-(4)):

* g_r = ln alpha_r, G_r = g_1 + ... + g_r, Gamma_rj = exp(G_r - G_j) for r >= j.
* With u_r := beta_r e_r, eq (3) reads S_r = alpha_r S_{r-1} + k_r u_r^T, so
  S_r = e^{G_r} S + sum_{j<=r} Gamma_rj k_j u_j^T.
* Substituting into eq (2): (I + A) U = diag(beta) (V - diag(e^G) K S) with
  A = strict_lower[beta_r Gamma_rj (k_r . k_j)].
* Eq (4): Y = diag(e^G) Q S + P U with P = lower_incl[Gamma_rj (q_r . k_j)].
* Chunk exit: S' = e^{G_C} S + K^T diag(e^{G_C - G}) U.

Two equivalent ways to get U are provided: through W = T diag(beta e^G) K and
U~ = T diag(beta) V (U = U~ - W S), and through R = diag(beta)(V - diag(e^G) K S),
U = T R, with T = (I + A)^-1.
"""
import numpy as np


def chunked_gdn(q, k, v, alpha, beta, S0, C, form="R"):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    y = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], np.float64)
            for c0 in range(0, T, C):
                sl = slice(c0, min(c0 + C, T))
                Q, K, V = q[b, sl, h], k[b, sl, h], v[b, sl, h]
                a, bt = alpha[b, sl, h], beta[b, sl, h]
                n = K.shape[0]
                G = np.cumsum(np.log(a))
                diff = G[:, None] - G[None, :]
                lower_incl = np.tril(np.ones((n, n), dtype=bool))
                Gam = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
                A = np.tril(bt[:, None] * Gam * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                eG = np.exp(G)
                if form == "W":
                    W = Tm @ ((bt * eG)[:, None] * K)
                    Ut = Tm @ (bt[:, None] * V)
                    U = Ut - W @ S
                else:
                    R = bt[:, None] * (V - eG[:, None] * (K @ S))
                    U = Tm @ R
                P = Gam * (Q @ K.T)
                y[b, sl, h] = eG[:, None] * (Q @ S) + P @ U
                S = np.exp(G[-1]) * S + K.T @ (np.exp(G[-1] - G)[:, None] * U)
            ST[b, h] = S
    return y, ST
