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


def chunked_gdn_bwd(q, k, v, alpha, beta, S0, dy, dST, C):
    """Chunkwise reverse mode of the form above (the algebra the GPU backward
    follows).  Per (batch, head), three passes:

    1. forward over chunks, keeping the state S_c entering every chunk;
    2. reverse over chunks for dS'_c, the gradient of the state leaving chunk c:
       dU = P^T dY + diag(d) K dS',  dR = diag(beta) T^T dU,
       dS = e^{G_C} dS' + Q^T diag(e^G) dY - K^T diag(e^G) dR;
    3. per chunk, given S_c and dS'_c, the gradients of its tokens: with
       X = diag(beta) (V - diag(e^G) K S), U = T X, dX = T^T dU,
       dV = diag(beta) dX,  dP = dY U^T (lower incl),  dA = -(dX U^T) (strict lower),
       dQ = diag(e^G) dY S^T + (Gamma o dP) K,
       dK = -diag(e^G beta) dX S^T + diag(d) U dS'^T + (dKK + dKK^T) K + (Gamma o dP)^T Q
            with dKK = Gamma o diag(beta) dA,
       dbeta_r = dX_r . (V - e^G K S)_r + sum_j dA_rj Gamma_rj k_r.k_j,
       and the gradient of each cumulative log-decay G_r (natural log) gathered
       from every factor e^G, e^{G_C - G}, e^{G_C} and Gamma it appears in, then
       d ln alpha_i = sum_{r >= i} dG_r.
    Here d_r = e^{G_C - G_r}.  Returns a dict like the oracle's.
    """
    q, k, v, alpha, beta, dy = (np.asarray(a, np.float64) for a in (q, k, v, alpha, beta, dy))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
               dalpha=np.zeros((B, T, H)), dbeta=np.zeros((B, T, H)), dS0=np.zeros((B, H, Dk, Dv)))
    for b in range(B):
        for h in range(H):
            chunks = []
            for c0 in range(0, T, C):
                sl = slice(c0, min(c0 + C, T))
                Q, K, V, dY = q[b, sl, h], k[b, sl, h], v[b, sl, h], dy[b, sl, h]
                a, bt = alpha[b, sl, h], beta[b, sl, h]
                n = K.shape[0]
                G = np.cumsum(np.log(a))
                low = np.tril(np.ones((n, n), dtype=bool))
                Gam = np.where(low, np.exp(np.where(low, G[:, None] - G[None, :], 0.0)), 0.0)
                Ak = np.tril(Gam * (K @ K.T), -1)
                Tm = np.linalg.inv(np.eye(n) + bt[:, None] * Ak)
                P = Gam * (Q @ K.T)
                eG, d = np.exp(G), np.exp(G[-1] - G)
                chunks.append(dict(sl=sl, Q=Q, K=K, V=V, dY=dY, a=a, bt=bt, G=G, Gam=Gam, Ak=Ak, Tm=Tm, P=P,
                                   eG=eG, d=d, gC=np.exp(G[-1])))
            # pass 1
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], np.float64)
            for ch in chunks:
                ch["S"] = S
                U = ch["Tm"] @ (ch["bt"][:, None] * (ch["V"] - ch["eG"][:, None] * (ch["K"] @ S)))
                S = ch["gC"] * S + ch["K"].T @ (ch["d"][:, None] * U)
            # pass 2
            dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST[b, h], np.float64)
            for ch in reversed(chunks):
                ch["dSp"] = dS
                dU = ch["P"].T @ ch["dY"] + ch["d"][:, None] * (ch["K"] @ dS)
                dR = ch["bt"][:, None] * (ch["Tm"].T @ dU)
                dS = ch["gC"] * dS + ch["Q"].T @ (ch["eG"][:, None] * ch["dY"]) - ch["K"].T @ (ch["eG"][:, None] * dR)
            out["dS0"][b, h] = dS
            # pass 3
            for ch in chunks:
                Q, K, V, dY, bt, eG, d, Gam = ch["Q"], ch["K"], ch["V"], ch["dY"], ch["bt"], ch["eG"], ch["d"], ch["Gam"]
                S, dSp = ch["S"], ch["dSp"]
                KS, QS, KdS = K @ S, Q @ S, K @ dSp
                Wt = V - eG[:, None] * KS
                U = ch["Tm"] @ (bt[:, None] * Wt)
                dU = ch["P"].T @ dY + d[:, None] * KdS
                dX = ch["Tm"].T @ dU
                dWt = bt[:, None] * dX
                n = K.shape[0]
                dP = np.tril(dY @ U.T)
                dA = -np.tril(dX @ U.T, -1)
                dAk = bt[:, None] * dA
                dKK = Gam * dAk
                dQK = Gam * dP
                dQ = eG[:, None] * (dY @ S.T) + dQK @ K
                dK = (-(eG * bt)[:, None] * (dX @ S.T) + d[:, None] * (U @ dSp.T)
                      + (dKK + dKK.T) @ K + dQK.T @ Q)
                dbeta = (dX * Wt).sum(1) + (dA * ch["Ak"]).sum(1)
                E = dAk * ch["Ak"] + dP * ch["P"]
                s3 = (U * KdS).sum(1)
                dG = (eG * (dY * QS).sum(1) - eG * (dWt * KS).sum(1) - d * s3 + E.sum(1) - E.sum(0))
                dG[-1] += ch["gC"] * (S * dSp).sum() + (d * s3).sum()
                dlna = np.cumsum(dG[::-1])[::-1]
                sl = ch["sl"]
                out["dq"][b, sl, h] = dQ
                out["dk"][b, sl, h] = dK
                out["dv"][b, sl, h] = dWt
                out["dbeta"][b, sl, h] = dbeta
                out["dalpha"][b, sl, h] = dlna / ch["a"]
    return out
