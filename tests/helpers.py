"""Shared test helpers: moving seeded numpy inputs to the GPU and the parity
metric max|x - ref| / RMS(ref)."""
import numpy as np

from linear_attention_token_gated_amd import workloads as wl

TOL_F32 = 1e-4     # fp32-input runs
TOL_BF16 = 2e-2    # bf16-input runs


def dev(a, device="cuda"):
    """numpy float32 array or bf16 bit pattern (uint16) -> torch tensor on the GPU."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref):
    """max |x - ref| / RMS(ref); absolute max error when RMS(ref) < 1e-30."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    d = np.abs(x - ref).max()
    if not np.isfinite(d):
        return float("inf")
    return float(d / rms) if rms >= 1e-30 else float(d)


def oracle_prefill(oracle, inp, S0=None):
    return oracle.gdn_recurrence(wl.widen(inp["q"]), wl.widen(inp["k"]), wl.widen(inp["v"]),
                                 wl.widen(inp["alpha"]), wl.widen(inp["beta"]),
                                 wl.widen(inp["S0"]) if S0 is None else S0)
