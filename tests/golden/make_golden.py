"""Write tests/golden/prefill_tiny_f32.json: the oracle's y and final state for
the tiny fp32 prefill workload (B=1, T=64, H=2, d_k=d_v=16, S0=0).

The pages print no worked numerical example for the gated delta rule, so this
fixture is not a pin of the oracle against the pages; it is a regression anchor
that makes any later change to the oracle's arithmetic visible.  It calls only
the oracle and the seeded input generator.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from linear_attention_token_gated_amd import workloads as wl  # noqa: E402


def main():
    cfg = wl.TINY
    inp = wl.prefill_config_inputs(cfg)
    y, ST = oracle.gdn_recurrence(wl.widen(inp["q"]), wl.widen(inp["k"]), wl.widen(inp["v"]),
                                  wl.widen(inp["alpha"]), wl.widen(inp["beta"]), None)
    out = {
        "source": "oracle.gdn_recurrence on workloads.TINY (seed 0); eqs (1)-(4) of the picx.dev "
                  "summary of 'On the Design of Qwen3.8-Next Architecture', 'Theoretical foundations'",
        "shape_y": list(y.shape), "shape_S": list(ST.shape),
        "y": [float.hex(float(a)) for a in y.ravel()],
        "S_T": [float.hex(float(a)) for a in ST.ravel()],
    }
    with open(os.path.join(HERE, "prefill_tiny_f32.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
