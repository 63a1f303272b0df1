"""Oracle: plain, slow, fp64 CPU implementation of the Gated DeltaNet token mixer.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``linear_attention_token_gated_amd``) and imports nothing
from it; the two meet only through the seeded input generators.

Sources (all on the picx.dev summary page of "On the Design of Qwen3.8-Next
Architecture"):

* core recurrence -- section "Theoretical foundations", eqs (1)-(4); computed by
  ``oracle.c`` token by token in double precision;
* its reverse mode (gradients of a loss through eqs (1)-(4)) -- the chain rule
  applied to the same four steps in reverse token order, also in ``oracle.c``;
* layer wrapper -- section "Methodology / 1. GDN Hybrid Token Mixing": short
  causal convolution, L2-normalised queries and keys, eq (9) write strength,
  eq (10) decay, eq (11) sigmoid-gated, zero-centred RMSNorm output.

Every function takes and returns float64 numpy arrays and never rounds an
intermediate.  Readings of points the pages leave open (all "parity unpinned"
against the pages themselves, pinned only by the invariants in the tests):

* the short convolution is depthwise and causal over the q, k and v channels
  that the fused in-projection produces; no bias, no activation after it;
  ``out[t, c] = sum_j w[c, j] * in[t - (K-1) + j, c]`` with zero history;
* L2 normalisation is ``x / sqrt(sum(x^2) + 1e-6)`` per (token, head);
* no query scaling (eq (4) has none);
* eq (10): ``A`` and ``b_alpha`` are per-head scalars;
* eq (9) has no bias;
* RMSNorm is per (token, head) over d_v, ``y / sqrt(mean(y^2) + 1e-6)``, with
  a zero-centred gain ``(1 + gamma)``, ``gamma`` of length d_v shared by heads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc into ``liboracle.so`` (generic x86-64, no
    fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off",
               os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _configure(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_gdn_recurrence.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                          i64, i64, i64, i64, i64,
                                          ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_gdn_recurrence.restype = ctypes.c_int
    lib.oracle_gdn_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                           i64, i64, i64, i64,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_gdn_decode_step.restype = ctypes.c_int
    lib.oracle_gdn_recurrence_bwd.argtypes = [dp] * 14 + [i64] * 5 + [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_gdn_recurrence_bwd.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


last_threads_used = 0


def gdn_recurrence(q, k, v, alpha, beta, S0=None, nthreads: int = 0, _core=None):
    """Eqs (1)-(4) over whole sequences.

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; alpha, beta: [B, T, H];
    S0: [B, H, Dk, Dv] or None (zero state).  Returns (y [B,T,H,Dv], S_T).
    """
    global last_threads_used
    q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (B, H, Dk, Dv)
    y = np.empty((B, T, H, Dv), dtype=np.float64)
    ST = np.empty((B, H, Dk, Dv), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = (_core or _load()).oracle_gdn_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(S0), _ptr(y), _ptr(ST), B, T, H, Dk, Dv,
                                       int(nthreads), ctypes.byref(used))
    if rc != 0:
        raise MemoryError("oracle_gdn_recurrence: allocation failed")
    last_threads_used = used.value
    return y, ST


def gdn_recurrence_bwd(q, k, v, alpha, beta, S0, dy, dST=None, nthreads: int = 0, _core=None):
    """Gradients of eqs (1)-(4) over whole sequences (reverse mode, token by
    token, in ``oracle.c``).

    Inputs as for :func:`gdn_recurrence`, plus dy [B, T, H, Dv] = dL/dy and
    dST [B, H, Dk, Dv] = dL/dS_T (None: zero).  Returns a dict with dq, dk
    [B,T,H,Dk], dv [B,T,H,Dv], dalpha, dbeta [B,T,H] and dS0 [B,H,Dk,Dv]
    (the gradient with respect to the initial state, also when S0 is None,
    i.e. zero).
    """
    global last_threads_used
    q, k, v, alpha, beta, dy = (_f64(a) for a in (q, k, v, alpha, beta, dy))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv) and dy.shape == (B, T, H, Dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    S0 = None if S0 is None else _f64(S0)
    dST = None if dST is None else _f64(dST)
    for s in (S0, dST):
        assert s is None or s.shape == (B, H, Dk, Dv)
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)), dv=np.zeros((B, T, H, Dv)),
               dalpha=np.zeros((B, T, H)), dbeta=np.zeros((B, T, H)), dS0=np.zeros((B, H, Dk, Dv)))
    used = ctypes.c_int(0)
    rc = (_core or _load()).oracle_gdn_recurrence_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(dy), _ptr(dST),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
        _ptr(out["dS0"]), B, T, H, Dk, Dv, int(nthreads), ctypes.byref(used))
    if rc != 0:
        raise MemoryError("oracle_gdn_recurrence_bwd: allocation failed")
    last_threads_used = used.value
    return out


def gdn_decode_step(q, k, v, alpha, beta, S, nthreads: int = 0, _core=None):
    """One token of eqs (1)-(4) for each of N sequences.

    q, k: [N, H, Dk]; v: [N, H, Dv]; alpha, beta: [N, H]; S: [N, H, Dk, Dv].
    Returns (y [N,H,Dv], S_new); the input S is not modified.
    """
    global last_threads_used
    q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    S_new = np.array(S, dtype=np.float64, order="C", copy=True)
    assert S_new.shape == (N, H, Dk, Dv)
    y = np.empty((N, H, Dv), dtype=np.float64)
    used = ctypes.c_int(0)
    rc = (_core or _load()).oracle_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                        _ptr(S_new), _ptr(y), N, H, Dk, Dv,
                                        int(nthreads), ctypes.byref(used))
    if rc != 0:
        raise MemoryError("oracle_gdn_decode_step: allocation failed")
    last_threads_used = used.value
    return y, S_new


def gdn_decode_verify(q, k, v, alpha, beta, S):
    """T consecutive tokens of each of N sequences from stored states (eqs
    (1)-(4) token by token), keeping the state after every token.

    q, k: [N, T, H, Dk]; v: [N, T, H, Dv]; alpha, beta: [N, T, H]; S: [N, H, Dk, Dv].
    Returns (y [N, T, H, Dv], states [N, T, H, Dk, Dv]); S is not modified.
    """
    q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
    N, T, H, Dk = q.shape
    Dv = v.shape[-1]
    y = np.empty((N, T, H, Dv))
    states = np.empty((N, T, H, Dk, Dv))
    cur = _f64(S)
    for t in range(T):
        y[:, t], cur = gdn_decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], cur)
        states[:, t] = cur
    return y, states


# ---------------------------------------------------------------------------
# Layer wrapper (picx.dev summary, "1. GDN Hybrid Token Mixing", eqs (9)-(11)).
# Each stage is its own function so the tests can pin it on its own.
# ---------------------------------------------------------------------------

L2_EPS = 1e-6
RMS_EPS = 1e-6


def linear(x, W):
    """x @ W^T: a plain projection, W stored [out_features, in_features]."""
    return _f64(x) @ _f64(W).T


def causal_depthwise_conv(u, w):
    """Short causal convolution, one filter per channel.

    u: [B, T, Ch]; w: [Ch, K] with tap K-1 applied to the current token.
    out[b, t, c] = sum_j w[c, j] * u[b, t-(K-1)+j, c], u at negative t = 0.
    """
    u = _f64(u)
    w = _f64(w)
    B, T, Ch = u.shape
    K = w.shape[1]
    out = np.zeros_like(u)
    for j in range(K):
        lag = K - 1 - j            # tap j reads the token `lag` steps back
        if lag >= T:
            continue
        out[:, lag:, :] += w[None, None, :, j] * u[:, :T - lag, :]
    return out


def l2_normalize(x, eps: float = L2_EPS):
    """Per-vector L2 normalisation over the last axis: x / sqrt(|x|^2 + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    """log(1 + e^x), written so that large |x| does not overflow."""
    x = _f64(x)
    return np.where(x > 0, x + np.log1p(np.exp(-np.abs(x))), np.log1p(np.exp(np.minimum(x, 0))))


def write_strength(b):
    """Eq (9): beta_t = sigmoid(W_beta x_t); `b` is the projection W_beta x_t."""
    return sigmoid(b)


def decay(a, A, b_alpha):
    """Eq (10): alpha_t = exp(-exp(A) * softplus(W_alpha x_t + b_alpha)).

    a: [..., H] projections W_alpha x_t; A, b_alpha: [H] per-head scalars."""
    return np.exp(-np.exp(_f64(A)) * softplus(_f64(a) + _f64(b_alpha)))


def rmsnorm_zero_centred(y, gamma, eps: float = RMS_EPS):
    """RMSNorm over the last axis with gain (1 + gamma)."""
    y = _f64(y)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * (1.0 + _f64(gamma))


def gdn_layer_fwd(x, W_qkv, conv_w, W_ab, A, b_alpha, W_gate, norm_gamma, W_o,
                  H: int, Dk: int, Dv: int, S0=None, nthreads: int = 0, return_parts=False):
    """Full GDN token-mixing layer, x [B, T, hidden] -> o [B, T, hidden].

    W_qkv: [H*(2Dk+Dv), hidden] rows q | k | v (head-major); conv_w: [H*(2Dk+Dv), K];
    W_ab: [2H, hidden] rows a (decay input) | b (write-strength input);
    A, b_alpha: [H]; W_gate: [H*Dv, hidden] (W_z); norm_gamma: [Dv];
    W_o: [hidden, H*Dv].  Returns (o, S_T) or, with return_parts, a dict.
    """
    x = _f64(x)
    B, T, _ = x.shape
    qkv = linear(x, W_qkv)                              # fused in-projection
    ab = linear(x, W_ab)                                # W_alpha x_t | W_beta x_t
    z = linear(x, W_gate)                               # W_z x_t
    conv = causal_depthwise_conv(qkv, conv_w)           # short causal convolution
    q = conv[..., :H * Dk].reshape(B, T, H, Dk)
    k = conv[..., H * Dk:2 * H * Dk].reshape(B, T, H, Dk)
    v = conv[..., 2 * H * Dk:].reshape(B, T, H, Dv)
    q = l2_normalize(q)
    k = l2_normalize(k)
    alpha = decay(ab[..., :H], A, b_alpha)              # eq (10)
    beta = write_strength(ab[..., H:])                  # eq (9)
    y, ST = gdn_recurrence(q, k, v, alpha, beta, S0, nthreads=nthreads)   # eqs (1)-(4)
    yn = rmsnorm_zero_centred(y, norm_gamma)
    g = sigmoid(z).reshape(B, T, H, Dv) * yn            # eq (11) gate
    o = linear(g.reshape(B, T, H * Dv), W_o)            # eq (11) W_o
    if return_parts:
        return dict(qkv=qkv, ab=ab, z=z, conv=conv, q=q, k=k, v=v, alpha=alpha,
                    beta=beta, y=y, yn=yn, g=g, o=o, ST=ST)
    return o, ST


def gdn_layer_decode_step(x, W_qkv, conv_w, W_ab, A, b_alpha, W_gate, norm_gamma, W_o,
                          H: int, Dk: int, Dv: int, conv_state, S):
    """One new token of the layer for each of N sequences (same section and
    formulas as ``gdn_layer_fwd``, one token at a time with its history given).

    x: [N, hidden]; conv_state: [N, K-1, Ch], the in-projection rows of the
    previous K-1 tokens, oldest first (zeros before a sequence starts);
    S: [N, H, Dk, Dv] the state after the previous token.
    Returns (o [N, hidden], new conv_state, new S); the inputs are not modified.
    """
    x = _f64(x)
    conv_w = _f64(conv_w)
    N = x.shape[0]
    K = conv_w.shape[1]
    qkv = linear(x, W_qkv)                              # this token's in-projection
    ab = linear(x, W_ab)
    z = linear(x, W_gate)
    hist = _f64(conv_state).reshape(N, K - 1, -1) if K > 1 else np.zeros((N, 0, qkv.shape[1]))
    window = np.concatenate([hist, qkv[:, None, :]], axis=1)      # [N, K, Ch], tap j = row j
    conv = np.zeros_like(qkv)
    for j in range(K):
        conv += conv_w[None, :, j] * window[:, j, :]
    q = l2_normalize(conv[:, :H * Dk].reshape(N, H, Dk))
    k = l2_normalize(conv[:, H * Dk:2 * H * Dk].reshape(N, H, Dk))
    v = conv[:, 2 * H * Dk:].reshape(N, H, Dv)
    alpha = decay(ab[:, :H], A, b_alpha)
    beta = write_strength(ab[:, H:])
    y, S_new = gdn_decode_step(q, k, v, alpha, beta, _f64(S))
    g = sigmoid(z).reshape(N, H, Dv) * rmsnorm_zero_centred(y, norm_gamma)
    o = linear(g.reshape(N, H * Dv), W_o)
    return o, window[:, 1:, :].copy(), S_new
