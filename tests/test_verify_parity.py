"""GPU parity of gdn_decode_verify (T tokens per sequence from stored states,
every intermediate state written) against the oracle, and against T calls of
the GPU decode step."""
import numpy as np
import pytest

from helpers import TOL_BF16, TOL_F32, dev, host, rel_err
from linear_attention_token_gated_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run(inp):
    import torch
    import linear_attention_token_gated_amd as gdn
    S = dev(inp["S0"])
    keep = S.clone()
    y, so = gdn.decode_verify(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["alpha"]), dev(inp["beta"]), S)
    torch.cuda.synchronize()
    assert torch.equal(S, keep)          # the stored states are read only
    return y, so


def _check(oracle, inp, tol):
    y, so = _run(inp)
    y_ref, s_ref = oracle.gdn_decode_verify(*(wl.widen(inp[n]) for n in ("q", "k", "v", "alpha", "beta")),
                                            wl.widen(inp["S0"]))
    ey, es = rel_err(host(y), y_ref), rel_err(host(so), s_ref)
    print(f"  err y={ey:.3e} states={es:.3e}", flush=True)
    assert ey <= tol and es <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (128, 128), (128, 32)])
def test_verify_shapes(oracle_mod, dtype, T, Dk, Dv):
    print(f"case: verify N=3 T={T} H=2 Dk={Dk} Dv={Dv} {dtype}", flush=True)
    inp = wl.prefill_inputs(3, T, 2, Dk, Dv, dtype=dtype, s0_std=0.1, seed=T + Dk + Dv)
    _check(oracle_mod, inp, TOL_F32 if dtype == "f32" else TOL_BF16)


def test_verify_workload(oracle_mod):
    cfg = wl.VERIFY_256x4
    print(f"case: {cfg.name}", flush=True)
    _check(oracle_mod, wl.prefill_config_inputs(cfg), TOL_BF16)


def test_verify_equals_decode_steps():
    """Bit for bit the same arithmetic as T calls of the decode step."""
    import torch
    import linear_attention_token_gated_amd as gdn
    print("case: verify vs decode steps", flush=True)
    inp = wl.prefill_inputs(4, 4, 3, 64, 64, dtype="bf16", s0_std=0.1, seed=9)
    y, so = _run(inp)
    S = dev(inp["S0"])
    q, k, v, al, be = (dev(inp[n]) for n in ("q", "k", "v", "alpha", "beta"))
    for t in range(4):
        yt = gdn.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                             al[:, t].contiguous(), be[:, t].contiguous(), S)
        torch.cuda.synchronize()
        assert torch.equal(yt, y[:, t]) and torch.equal(S, so[:, t])


def test_verify_empty():
    import torch
    import linear_attention_token_gated_amd as gdn
    z = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    y, so = gdn.decode_verify(z(2, 0, 1, 16), z(2, 0, 1, 16), z(2, 0, 1, 16), z(2, 0, 1), z(2, 0, 1), z(2, 1, 16, 16))
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 1, 16) and so.shape == (2, 0, 1, 16, 16)
