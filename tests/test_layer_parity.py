"""GPU parity of gdn_layer_fwd against the oracle's fp64 layer (in-projection,
causal conv, L2 norm, eqs (9)-(11), core, RMSNorm and gate, out-projection)."""
import numpy as np
import pytest

from helpers import TOL_BF16, dev, host, rel_err
from linear_attention_token_gated_amd import workloads as wl

pytestmark = pytest.mark.gpu

NAMES = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")


def _run(oracle, inp, B, T, hidden, H, Dk, Dv, chunk, S0=None, nthreads=0):
    import torch
    import linear_attention_token_gated_amd as gdn
    params = {n: dev(inp[n]) for n in NAMES}
    s0 = None if S0 is None else dev(S0)
    out, sT = gdn.layer_fwd(dev(inp["x"]), params, H, Dk, Dv, initial_state=s0, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_layer_fwd(wl.widen(inp["x"]), *(wl.widen(inp[n]) for n in NAMES),
                                        H=H, Dk=Dk, Dv=Dv, S0=None if S0 is None else wl.widen(S0),
                                        nthreads=nthreads)
    eo, eS = rel_err(host(out), o_ref), rel_err(host(sT), S_ref)
    print(f"  err out={eo:.3e} S={eS:.3e}", flush=True)
    return eo, eS, host(out)


@pytest.mark.parametrize("B,T,hidden,H,Dk,Dv,chunk", [
    (1, 64, 128, 2, 32, 64, 16),
    (2, 150, 256, 2, 64, 64, 64),
    (1, 77, 192, 4, 16, 32, 32),
    (1, 300, 512, 4, 128, 128, 64),
    # 3 slices: the core's launch shared with the gate projection starts the
    # projection's tiles at 8, so 5 workgroups between them end at once
    (1, 100, 256, 3, 32, 16, 32),
])
def test_layer_small(oracle_mod, B, T, hidden, H, Dk, Dv, chunk):
    print(f"case: layer B={B} T={T} hidden={hidden} H={H} Dk={Dk} Dv={Dv} C={chunk}", flush=True)
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=4, w_std=0.05, seed=T + H,
                          gamma_std=0.1, A_val=0.3, b_alpha_val=-0.5)
    rng = np.random.default_rng(T)
    S0 = (rng.standard_normal((B, H, Dk, Dv)) * 0.05).astype(np.float32)
    eo, eS, _ = _run(oracle_mod, inp, B, T, hidden, H, Dk, Dv, chunk, S0=S0)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


@pytest.mark.parametrize("conv_k", [1, 2, 3])
def test_layer_conv_widths(oracle_mod, conv_k):
    """Short convolutions narrower than 4 taps, over a tile boundary of the prologue."""
    B, T, hidden, H, Dk, Dv, chunk = 2, 70, 128, 2, 32, 32, 16
    print(f"case: layer B={B} T={T} conv_k={conv_k}", flush=True)
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=conv_k, w_std=0.05, seed=11 + conv_k,
                          gamma_std=0.1, A_val=0.3, b_alpha_val=-0.5)
    eo, eS, _ = _run(oracle_mod, inp, B, T, hidden, H, Dk, Dv, chunk)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def test_layer_causal_on_gpu(oracle_mod):
    """Changing tokens after t leaves out[:t+1] bit-identical on the GPU."""
    print("case: layer causality", flush=True)
    B, T, hidden, H, Dk, Dv = 1, 96, 128, 2, 32, 32
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, w_std=0.05, seed=3)
    _, _, o1 = _run(oracle_mod, inp, B, T, hidden, H, Dk, Dv, 32)
    inp2 = dict(inp)
    x = wl.bf16_bits_to_f32(inp["x"]).copy()
    x[:, 50:] += 1.0
    inp2["x"] = wl.to_bf16_bits(x)
    _, _, o2 = _run(oracle_mod, inp2, B, T, hidden, H, Dk, Dv, 32)
    np.testing.assert_array_equal(o1[:, :50], o2[:, :50])
    assert np.abs(o1[:, 50:] - o2[:, 50:]).max() > 0


@pytest.mark.slow
def test_layer_full_config(oracle_mod):
    cfg = wl.LAYER_16K
    print(f"case: {cfg.name}", flush=True)
    inp = wl.layer_config_inputs(cfg)
    eo, eS, _ = _run(oracle_mod, inp, cfg.B, cfg.T, cfg.hidden, cfg.H, cfg.Dk, cfg.Dv, cfg.chunk)
    assert eo <= TOL_BF16 and eS <= TOL_BF16


def test_layer_every_gemm_tile(oracle_mod):
    """A layer whose projections take each tile size of gemm_nt_kernel: the
    in-projection (4096 x 6144) 256 x 256, the out-projection (4096 x 2048)
    128 x 128, the gate pair a|b (4096 x 32) 64 x 64; the gate projection
    (4096 x 2048) runs in the core's launch on 256 x 256 tiles."""
    B, T, hidden, H, Dk, Dv, chunk = 1, 4096, 2048, 16, 128, 128, 64
    print("case: layer with every GEMM tile", flush=True)
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=4, w_std=0.02, seed=33)
    eo, eS, _ = _run(oracle_mod, inp, B, T, hidden, H, Dk, Dv, chunk, nthreads=16)
    assert eo <= TOL_BF16 and eS <= TOL_BF16
