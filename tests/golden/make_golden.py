"""Writes the oracle regression fixtures in this folder (run from the repository root:
python tests/golden/make_golden.py). Calls only the oracle and the seeded input generator.

The pages print no numeric worked example of the method, so these fixtures are not pins of
the oracle against the pages (those are the reductions, closed forms and finite-difference
checks in tests/test_oracle_*pins.py). They freeze the oracle's results on small seeded
inputs: a later change to the oracle's arithmetic shows up as a failing regression test,
and has to name the passage of the pages that justifies it.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gdn2_inputs import make_decode_inputs, make_inputs  # noqa: E402
from oracle import gdn2_backward, gdn2_decode_steps, gdn2_forward  # noqa: E402

NAMES = ("q", "k", "v", "g", "b", "w")


def _fmt(name, a):
    a = np.asarray(a, np.float64).ravel()
    return f"{name} " + " ".join(f"{x:.17e}" for x in a)


def cases():
    """(name, list of (label, array)) for every fixture."""
    out = []
    x = make_inputs(1, 20, 2, 8, 4, "fp32", seed=7, s0_std=0.1)
    o, S = gdn2_forward(*(x[n] for n in NAMES), s0=x["s0"])
    out.append(("forward_B1_T20_H2_dk8_dv4_fp32", [("o", o), ("S_final", S)]))
    lens = [3, 0, 9, 5]
    xv = make_inputs(1, sum(lens), 1, 4, 6, "bf16", seed=8, lengths=lens, s0_std=0.1)
    o, S = gdn2_forward(*(xv[n] for n in NAMES), s0=xv["s0"], cu_seqlens=xv["cu_seqlens"])
    out.append(("forward_varlen_3_0_9_5_H1_dk4_dv6_bf16", [("o", o), ("S_final", S)]))
    xd = make_decode_inputs(3, 2, 4, 4, 5, "fp32", seed=9, s0_std=0.1)
    o, S = gdn2_decode_steps(xd["s0"], *(xd[n] for n in NAMES))
    out.append(("decode_N3_H2_dk4_dv4_5steps_fp32", [("o", o), ("S", S)]))
    xb = make_inputs(1, 12, 1, 4, 4, "fp32", seed=10, s0_std=0.1)
    rng = np.random.default_rng(11)
    do = rng.normal(size=(1, 12, 1, 4))
    ds = rng.normal(size=(1, 1, 4, 4))
    grads = gdn2_backward(*(xb[n] for n in NAMES), do, dS_final=ds, s0=xb["s0"])
    out.append(("backward_B1_T12_H1_dk4_dv4_fp32",
                list(zip(("dq", "dk", "dv", "dg", "db", "dw", "ds0"), grads))))
    return out


def main():
    for name, arrays in cases():
        with open(os.path.join(HERE, name + ".txt"), "w") as f:
            f.write(f"# oracle regression fixture {name}; written by tests/golden/make_golden.py\n")
            for label, a in arrays:
                f.write(_fmt(label, a) + "\n")
    print("written")


if __name__ == "__main__":
    main()
