"""The allocation-free layer decode step (gdn_layer_decode_step_noalloc, on the
library's own scratch) against gdn_layer_decode_step with a workspace: two
calls in a row, the second with fewer sequences, bit for bit."""
import numpy as np
import pytest

from helpers import dev, host
from linear_attention_token_gated_amd import workloads as wl

pytestmark = pytest.mark.gpu

NAMES = ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate", "norm_gamma", "W_o")


def test_noalloc_matches_workspace_call():
    import torch
    import linear_attention_token_gated_amd as gdn
    N, hidden, H, Dk, Dv, conv_k = 64, 512, 4, 128, 128, 4
    inp = wl.layer_inputs(N, 1, hidden, H, Dk, Dv, conv_k=conv_k, w_std=0.03, seed=71)
    params = {n: dev(inp[n]) for n in NAMES}
    rng = np.random.default_rng(72)
    nqkv = H * (2 * Dk + Dv)
    cs0 = rng.standard_normal((N, conv_k - 1, nqkv)).astype(np.float32)
    S0 = (0.02 * rng.standard_normal((N, H, Dk, Dv))).astype(np.float32)
    x = dev(inp["x"])[:, 0].contiguous()
    for n in (N, 17):                                      # the second call is smaller
        print(f"case: noalloc layer decode N={n}", flush=True)
        xs = x[:n].contiguous()
        cs_a, S_a = dev(cs0[:n]), dev(S0[:n])
        cs_b, S_b = dev(cs0[:n]), dev(S0[:n])
        out_a = gdn.layer_decode_step(xs, params, H, Dk, Dv, cs_a, S_a)
        out_b = torch.empty((n, hidden), dtype=torch.float32, device="cuda")
        gdn.layer_decode_step_noalloc(xs, params, H, Dk, Dv, cs_b, S_b, out_b)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out_b), host(out_a))
        np.testing.assert_array_equal(host(S_b), host(S_a))
        np.testing.assert_array_equal(host(cs_b), host(cs_a))
        print(f"  equal: out max |.| {np.abs(host(out_a)).max():.3e}", flush=True)


def test_noalloc_rejects_oversize():
    import torch
    import linear_attention_token_gated_amd as gdn
    N, hidden, H, Dk, Dv = 1024, 2048, 16, 128, 128     # 72 MB of intermediates > 32 MiB
    assert gdn.layer_decode_workspace_bytes(N, hidden, H, Dk, Dv) > 32 << 20
    inp = wl.layer_inputs(1, 1, hidden, H, Dk, Dv, conv_k=4, w_std=0.02, seed=73)
    params = {n: dev(inp[n]) for n in NAMES}
    x = torch.zeros((N, hidden), dtype=torch.bfloat16, device="cuda")
    cs = torch.zeros((N, 3, H * (2 * Dk + Dv)), dtype=torch.float32, device="cuda")
    S = torch.zeros((N, H, Dk, Dv), dtype=torch.float32, device="cuda")
    out = torch.empty((N, hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        gdn.layer_decode_step_noalloc(x, params, H, Dk, Dv, cs, S, out)
