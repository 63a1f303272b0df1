"""Pin of the oracle's multi-token verification against its sequence
recurrence (picx.dev summary of "On the Design of Qwen3.8-Next Architecture",
"Theoretical foundations", eqs (1)-(4)).  CPU only.

gdn_decode_verify runs the single-token step T times; gdn_recurrence runs the
whole sequence in one C loop.  The state after token t of the first must be
the final state of the second over the first t+1 tokens, and the outputs must
agree token by token.
"""
import numpy as np

from linear_attention_token_gated_amd import workloads as wl


def test_verify_states_are_prefix_final_states(oracle_mod):
    N, T, H, Dk, Dv = 3, 5, 2, 8, 6
    inp = wl.prefill_inputs(N, T, H, Dk, Dv, dtype="f32", s0_std=0.3, seed=13)
    q, k, v, al, be = (wl.widen(inp[n]) for n in ("q", "k", "v", "alpha", "beta"))
    S0 = wl.widen(inp["S0"])
    y, states = oracle_mod.gdn_decode_verify(q, k, v, al, be, S0)
    y_ref, _ = oracle_mod.gdn_recurrence(q, k, v, al, be, S0)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-14)
    for t in range(T):
        sl = slice(0, t + 1)
        _, S_t = oracle_mod.gdn_recurrence(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl], S0)
        np.testing.assert_allclose(states[:, t], S_t, rtol=1e-12, atol=1e-14)


def test_verify_leaves_state(oracle_mod):
    inp = wl.prefill_inputs(2, 3, 1, 4, 4, dtype="f32", s0_std=0.5, seed=2)
    S0 = wl.widen(inp["S0"]).copy()
    keep = S0.copy()
    oracle_mod.gdn_decode_verify(*(wl.widen(inp[n]) for n in ("q", "k", "v", "alpha", "beta")), S0)
    assert np.array_equal(S0, keep)
