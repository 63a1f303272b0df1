"""The oracle still reproduces the stored tiny-workload fixture bit for bit.

The fixture is written by tests/golden/make_golden.py, which calls only the
oracle; a change to the oracle's arithmetic shows up here first."""
import json
import os

import numpy as np

from linear_attention_token_gated_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_golden_fixture(oracle_mod):
    with open(os.path.join(HERE, "golden", "prefill_tiny_f32.json")) as f:
        g = json.load(f)
    inp = wl.prefill_config_inputs(wl.TINY)
    y, ST = oracle_mod.gdn_recurrence(wl.widen(inp["q"]), wl.widen(inp["k"]), wl.widen(inp["v"]),
                                      wl.widen(inp["alpha"]), wl.widen(inp["beta"]), None)
    y_ref = np.array([float.fromhex(a) for a in g["y"]]).reshape(g["shape_y"])
    S_ref = np.array([float.fromhex(a) for a in g["S_T"]]).reshape(g["shape_S"])
    np.testing.assert_allclose(y, y_ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ST, S_ref, rtol=1e-13, atol=1e-15)
