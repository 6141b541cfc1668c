"""The whole-workload parity helper (tests/oracle_pool.py) on the CPU: the oracle's own
results give zero error over every shard layout, and a single wrong element anywhere (an
output of one chain, one state entry) is found with its size."""
import numpy as np

from gdn2_inputs import make_decode_inputs, make_inputs
from oracle import gdn2_decode_steps, gdn2_forward
from tests.oracle_pool import decode_errors, forward_errors

NAMES = ("q", "k", "v", "g", "b", "w")


def test_forward_errors_finds_one_wrong_element():
    x = make_inputs(1, 300, 3, 64, 64, "bf16", seed=11, lengths=[100, 0, 150, 50], s0_std=0.05)
    o, s = gdn2_forward(*(x[n] for n in NAMES), s0=x["s0"], cu_seqlens=x["cu_seqlens"])
    e = forward_errors(x, o, s)
    assert e["o"] == 0.0 and e["S"] == 0.0
    o2 = o.copy()
    o2[0, 260, 2, 5] += 0.25  # last sequence, last head
    e = forward_errors(x, o2, s)
    assert abs(e["o"] - 0.25 / np.max(np.abs(o))) < 1e-12 and e["S"] == 0.0
    s2 = s.copy()
    s2[1, 0, 3, 3] -= 0.5  # the empty sequence's state (its initial state)
    e = forward_errors(x, o, s2)
    assert e["o"] == 0.0 and abs(e["S"] - 0.5 / np.max(np.abs(s))) < 1e-12


def test_forward_errors_batched():
    x = make_inputs(3, 70, 2, 64, 64, "bf16", seed=12)
    o, s = gdn2_forward(*(x[n] for n in NAMES))
    assert forward_errors(x, o, s)["o"] == 0.0
    o2 = o.copy()
    o2[2, 69, 1, 63] += 1.0
    assert forward_errors(x, o2, s)["o"] > 0.0


def test_decode_errors_finds_one_wrong_element():
    x = make_decode_inputs(7, 2, 64, 64, 4, "bf16", seed=13, s0_std=0.02)
    o, s = gdn2_decode_steps(x["s0"], *(x[n] for n in NAMES))
    assert decode_errors(x["s0"], x, o, s, seqs_per_shard=3)["o"] == 0.0
    o2 = o.copy()
    o2[3, 6, 1, 0] += 0.1  # last step, last sequence (a shard of one)
    e = decode_errors(x["s0"], x, o2, s, seqs_per_shard=3)
    assert abs(e["o"] - 0.1 / np.max(np.abs(o))) < 1e-12 and e["S"] == 0.0
