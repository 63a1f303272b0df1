"""GPU parity of the prefill at the ends of the gate ranges (picx.dev summary
of "On the Design of Qwen3.8-Next Architecture", "Theoretical foundations":
alpha, beta in (0, 1) in eqs (1)-(3); eq (3) adds beta k e^T with e the
prediction error of eq (2), so with beta = 1 the read-out along the written key
equals the written value).  These are where (I + A) is furthest from the
identity and the decay prefix widest; every case has a ragged last chunk."""
import numpy as np
import pytest

from helpers import TOL_BF16, TOL_F32, dev, gate_endpoint_inputs, host, oracle_prefill, rel_err
from linear_attention_token_gated_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = ["beta1_qk", "ortho", "beta_near1", "alpha1", "alpha0"]
# the bf16 headline shape (C = 64, d = 128) in both bf16 forms (records +
# recurrence, one fused kernel) and two fp32 instances
PATHS = [("bf16", 64, 128, 128), ("bf16-fused", 64, 128, 128), ("f32", 64, 128, 128), ("f32", 16, 32, 16)]


@pytest.mark.parametrize("dtype,chunk,Dk,Dv", PATHS)
@pytest.mark.parametrize("case", CASES)
def test_prefill_gate_endpoints(oracle_mod, case, dtype, chunk, Dk, Dv):
    import torch
    import linear_attention_token_gated_amd as gdn
    T = min(Dk, 100) if case == "ortho" else 2 * chunk + 37
    B, H = 2, 2
    print(f"case: endpoints {case} B={B} T={T} H={H} Dk={Dk} Dv={Dv} C={chunk} {dtype}", flush=True)
    fused = dtype == "bf16-fused"
    dtype = "bf16" if fused else dtype
    inp = gate_endpoint_inputs(case, B, T, H, Dk, Dv, dtype, seed=100 + Dk + chunk)
    y, sT = gdn.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["alpha"]), dev(inp["beta"]),
                        dev(inp["S0"]), chunk=chunk, fused=fused)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle_prefill(oracle_mod, inp)
    ey, eS = rel_err(host(y), y_ref), rel_err(host(sT), S_ref)
    print(f"  err y={ey:.3e} S={eS:.3e}", flush=True)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert np.isfinite(host(y)).all() and np.isfinite(host(sT)).all()
    assert ey <= tol and eS <= tol, (ey, eS)
    if case == "beta1_qk" and dtype == "f32":
        # beta = 1 and a unit key: the state read along k_t after the write is v_t
        e = rel_err(host(y), wl.widen(inp["v"]))
        print(f"  read-out err={e:.3e}", flush=True)
        assert e <= 1e-4
    if case == "ortho" and dtype == "f32":
        # exact retrieval: S_T^T k_j = v_j for every written key j
        k, v = wl.widen(inp["k"]), wl.widen(inp["v"])
        got = np.einsum("bhkv,bthk->bthv", host(sT), k)
        e = rel_err(got, v)
        print(f"  retrieval err={e:.3e}", flush=True)
        assert e <= 1e-4


def test_layer_decay_underflow(oracle_mod):
    """eq (10) with exp(A) = e^3 and b_alpha = 5 drives alpha below the fp32
    normal range (about e^-100): the layer stays finite and matches the oracle."""
    import torch
    import linear_attention_token_gated_amd as gdn
    B, T, hidden, H, Dk, Dv, chunk = 1, 150, 256, 2, 64, 64, 64
    print("case: layer with alpha underflow (A=3, b_alpha=5)", flush=True)
    names = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")
    inp = wl.layer_inputs(B, T, hidden, H, Dk, Dv, conv_k=4, w_std=0.05, seed=9, gamma_std=0.1,
                          A_val=3.0, b_alpha_val=5.0)
    out, sT = gdn.layer_fwd(dev(inp["x"]), {n: dev(inp[n]) for n in names}, H, Dk, Dv, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_mod.gdn_layer_fwd(wl.widen(inp["x"]), *(wl.widen(inp[n]) for n in names),
                                            H=H, Dk=Dk, Dv=Dv)
    eo, eS = rel_err(host(out), o_ref), rel_err(host(sT), S_ref)
    print(f"  err out={eo:.3e} S={eS:.3e}", flush=True)
    assert np.isfinite(host(out)).all()
    assert eo <= TOL_BF16 and eS <= TOL_BF16
