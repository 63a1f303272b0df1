"""Seeded synthetic workloads shaped like the configurations the kernels are
measured on.

This module holds the input recipes only -- random draws, the recipe's own
normalisation of the drawn keys and queries, and the round-to-nearest-even cast
to bf16 -- and none of the gated delta rule's arithmetic.  Both the GPU path
and the CPU oracle take their inputs from here, so both see identical bits.

Values are drawn with ``numpy.random.Generator(PCG64(seed))`` in float32.  A
bf16 tensor is carried as its raw 16-bit pattern (``np.uint16``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (bit patterns)
# ---------------------------------------------------------------------------


def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def widen(a) -> np.ndarray:
    """Exact float64 copy of a float32 array or of bf16 bits."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# configurations
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str            # "f32" or "bf16" for q, k, v, y
    s0_std: Optional[float]  # None => no initial state (zero)
    seed: int


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    Dk: int
    Dv: int
    dtype: str
    s_std: float
    seed: int


@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int
    T: int
    hidden: int
    H: int
    Dk: int
    Dv: int
    conv_k: int
    chunk: int
    w_std: float
    seed: int


TINY = PrefillConfig("prefill-tiny-f32 (B=1 T=64 H=2 d=16 C=16)", 1, 64, 2, 16, 16, 16, "f32", None, 0)
PREFILL_4K = PrefillConfig("prefill-4k (B=2 T=4096 H=16 d=128 C=64 bf16)", 2, 4096, 16, 128, 128, 64, "bf16", 0.02, 1)
PREFILL_32K = PrefillConfig("prefill-32k (B=1 T=32768 H=32 d=128 C=64 bf16)", 1, 32768, 32, 128, 128, 64, "bf16", None, 2)
DECODE_256 = DecodeConfig("decode (N=256 H=32 d=128 fp32 state)", 256, 32, 128, 128, "bf16", 0.02, 3)
LAYER_16K = LayerConfig("layer (B=1 T=16384 hidden=2048 H=16 d=128 conv=4 C=64)", 1, 16384, 2048, 16, 128, 128, 4, 64, 0.02, 4)
# verification of 4 drafted tokens for each of 256 sequences from stored states
# (layout [N, T, H, *] of a prefill batch; the chunk field is unused)
VERIFY_256x4 = PrefillConfig("decode verify (N=256 T=4 H=32 d=128 fp32 states)", 256, 4, 32, 128, 128, 16, "bf16",
                             0.02, 6)
# one new token for each of 256 sequences (B = N, T = 1; chunk unused)
LAYER_DECODE_256 = LayerConfig("layer decode (N=256 hidden=2048 H=16 d=128 conv=4)", 256, 1, 2048, 16, 128, 128, 4, 64,
                               0.02, 5)


def _sigmoid32(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float32)))).astype(np.float32)


def _unit_rows(rng, shape):
    """N(0,1) vectors scaled to unit L2 norm along the last axis (float32)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _cast(x, dtype):
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def prefill_inputs(B, T, H, Dk, Dv, dtype="bf16", s0_std=None, seed=0):
    """q, k ~ N(0,1) then unit-normalised per (token, head); v ~ N(0,1);
    alpha = sigmoid(u), u ~ U(2.2, 6.9); beta = sigmoid(N(0,1));
    S0 ~ N(0, s0_std^2) or None.  Returns a dict of numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _unit_rows(rng, (B, T, H, Dk))
    k = _unit_rows(rng, (B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv), dtype=np.float32)
    u = rng.uniform(2.2, 6.9, size=(B, T, H)).astype(np.float32)
    alpha = _sigmoid32(u)
    beta = _sigmoid32(rng.standard_normal((B, T, H), dtype=np.float32))
    S0 = None
    if s0_std is not None:
        S0 = (rng.standard_normal((B, H, Dk, Dv), dtype=np.float32) * np.float32(s0_std)).astype(np.float32)
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                alpha=alpha, beta=beta, S0=S0, dtype=dtype)


def prefill_config_inputs(cfg: PrefillConfig):
    return prefill_inputs(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.dtype, cfg.s0_std, cfg.seed)


def bwd_inputs(B, T, H, Dk, Dv, dtype="bf16", s0_std=None, seed=0, dst_std=None):
    """Inputs of a prefill backward: the prefill recipe's inputs (same seed,
    same draws) plus the output gradients dy ~ N(0, 1) [B, T, H, Dv] and
    dST ~ N(0, dst_std^2) [B, H, Dk, Dv] (None if dst_std is None), float32,
    drawn from a generator seeded with seed + 500."""
    inp = prefill_inputs(B, T, H, Dk, Dv, dtype, s0_std, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 500))
    inp["dy"] = rng.standard_normal((B, T, H, Dv), dtype=np.float32)
    inp["dST"] = None
    if dst_std is not None:
        inp["dST"] = (rng.standard_normal((B, H, Dk, Dv), dtype=np.float32) * np.float32(dst_std)).astype(np.float32)
    return inp


def bwd_config_inputs(cfg: PrefillConfig, dst_std=1.0):
    return bwd_inputs(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, cfg.dtype, cfg.s0_std, cfg.seed, dst_std)


def decode_inputs(N, H, Dk, Dv, dtype="bf16", s_std=0.02, seed=3):
    """One token per sequence, same distributions as the prefill recipe;
    state S ~ N(0, s_std^2) in float32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _unit_rows(rng, (N, H, Dk))
    k = _unit_rows(rng, (N, H, Dk))
    v = rng.standard_normal((N, H, Dv), dtype=np.float32)
    alpha = _sigmoid32(rng.uniform(2.2, 6.9, size=(N, H)).astype(np.float32))
    beta = _sigmoid32(rng.standard_normal((N, H), dtype=np.float32))
    S = (rng.standard_normal((N, H, Dk, Dv), dtype=np.float32) * np.float32(s_std)).astype(np.float32)
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                alpha=alpha, beta=beta, S=S, dtype=dtype)


def decode_config_inputs(cfg: DecodeConfig):
    return decode_inputs(cfg.N, cfg.H, cfg.Dk, cfg.Dv, cfg.dtype, cfg.s_std, cfg.seed)


def layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=4, w_std=0.02, seed=4,
                 gamma_std=0.0, A_val=0.0, b_alpha_val=0.0):
    """x ~ N(0,1); projection weights ~ N(0, w_std^2); conv taps ~ U(-0.5, 0.5);
    A = A_val, b_alpha = b_alpha_val per head; gamma ~ N(0, gamma_std^2).
    bf16 for x and every weight matrix; float32 for A, b_alpha, gamma."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n_qkv = H * (2 * Dk + Dv)
    x = rng.standard_normal((B, T, hidden), dtype=np.float32)
    W_qkv = rng.standard_normal((n_qkv, hidden), dtype=np.float32) * np.float32(w_std)
    conv_w = rng.uniform(-0.5, 0.5, size=(n_qkv, conv_k)).astype(np.float32)
    W_ab = rng.standard_normal((2 * H, hidden), dtype=np.float32) * np.float32(w_std)
    W_gate = rng.standard_normal((H * Dv, hidden), dtype=np.float32) * np.float32(w_std)
    W_o = rng.standard_normal((hidden, H * Dv), dtype=np.float32) * np.float32(w_std)
    gamma = (rng.standard_normal((Dv,), dtype=np.float32) * np.float32(gamma_std)).astype(np.float32)
    A = np.full((H,), A_val, dtype=np.float32)
    b_alpha = np.full((H,), b_alpha_val, dtype=np.float32)
    return dict(x=to_bf16_bits(x), W_qkv=to_bf16_bits(W_qkv), conv_w=to_bf16_bits(conv_w),
                W_ab=to_bf16_bits(W_ab), A=A, b_alpha=b_alpha, W_gate=to_bf16_bits(W_gate),
                norm_gamma=gamma, W_o=to_bf16_bits(W_o))


def layer_decode_config_inputs(cfg: LayerConfig):
    """Inputs of one layer-decode step: the layer inputs of a one-token batch of
    cfg.B sequences, plus a history: conv rows ~ N(0, hidden * w_std^2) (the
    spread of x W_qkv^T with x ~ N(0, 1)) and states ~ N(0, 0.02^2)."""
    inp = layer_inputs(cfg.B, 1, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.conv_k, cfg.w_std, cfg.seed)
    rng = np.random.Generator(np.random.PCG64(cfg.seed + 1000))
    ch = cfg.H * (2 * cfg.Dk + cfg.Dv)
    cs = rng.standard_normal((cfg.B, cfg.conv_k - 1, ch), dtype=np.float32) * np.float32(
        np.sqrt(cfg.hidden) * cfg.w_std)
    S = rng.standard_normal((cfg.B, cfg.H, cfg.Dk, cfg.Dv), dtype=np.float32) * np.float32(0.02)
    return inp, cs, S


def layer_config_inputs(cfg: LayerConfig):
    return layer_inputs(cfg.B, cfg.T, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.conv_k,
                        cfg.w_std, cfg.seed)
