"""Pins of the oracle's decode loop (gdn2_decode_steps) against the whole-sequence forward
(gdn2_forward, itself pinned by the reductions and closed forms in test_oracle_pins.py).

Consecutive decode steps on a pool are the per-token procedure of the GDN-2 reading note
(§3, forward pass) applied to one token of every sequence at a time, so `steps` decode
calls on inputs laid out [steps, N, H, d] must equal the forward over the same tokens laid
out [N, steps, H, d]: outputs step by step, and the state after the last step. The pin takes
the decode function as an argument; planted mistakes in copies of the loop must each fail.
"""
import numpy as np
import pytest

from oracle import gdn2_decode_steps, gdn2_forward, gdn2_step

NAMES = ("q", "k", "v", "g", "b", "w")


def _inputs(rng, steps, N, H, dk, dv):
    x = dict(q=rng.normal(size=(steps, N, H, dk)), k=rng.normal(size=(steps, N, H, dk)) / 3,
             v=rng.normal(size=(steps, N, H, dv)),
             g=-rng.uniform(0.01, 0.6, size=(steps, N, H, dk)),
             b=rng.uniform(0, 1, size=(steps, N, H, dk)), w=rng.uniform(0, 1, size=(steps, N, H, dv)))
    return x


def pin_decode_equals_forward(decode, steps=6, N=3, H=2, dk=5, dv=4, seed=21):
    rng = np.random.default_rng(seed)
    x = _inputs(rng, steps, N, H, dk, dv)
    S0 = rng.normal(size=(N, H, dk, dv))
    o, S = decode(S0.copy(), *(x[n] for n in NAMES))
    # the same tokens as N sequences of `steps` tokens each
    o_ref, S_ref = gdn2_forward(*(np.swapaxes(x[n], 0, 1) for n in NAMES), s0=S0)
    np.testing.assert_allclose(o, np.swapaxes(o_ref, 0, 1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


def test_decode_steps_equal_forward():
    pin_decode_equals_forward(gdn2_decode_steps)


def test_single_step_is_one_token():
    """One decode step on a pool equals one gdn2_step per (sequence, head)."""
    rng = np.random.default_rng(22)
    x = _inputs(rng, 1, 2, 3, 4, 6)
    S0 = rng.normal(size=(2, 3, 4, 6))
    o, S = gdn2_decode_steps(S0.copy(), *(x[n] for n in NAMES))
    for n in range(2):
        for h in range(3):
            on, Sn = gdn2_step(S0[n, h], *(x[m][0, n, h] for m in NAMES))
            np.testing.assert_allclose(o[0, n, h], on, rtol=0, atol=1e-13)
            np.testing.assert_allclose(S[n, h], Sn, rtol=0, atol=1e-13)


def _mutant(kind):
    def decode(S, q, k, v, g, b, w):
        S = np.asarray(S, dtype=np.float64).copy()
        S_init = S.copy()
        o = np.zeros(v.shape)
        for s in range(q.shape[0]):
            qs = q[0] if kind == "step0_query_reused" else q[s]
            start = S_init if kind == "state_not_carried" else S
            out, S = gdn2_step(start, qs, k[s], v[s], g[s], b[s], w[s])
            o[s if kind != "outputs_shifted" else (s + 1) % q.shape[0]] = out
        return o, (S_init if kind == "initial_state_returned" else S)
    return decode


MUTANTS = ["step0_query_reused", "state_not_carried", "outputs_shifted", "initial_state_returned"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_decode_mistakes_are_caught(kind):
    with pytest.raises(AssertionError):
        pin_decode_equals_forward(_mutant(kind))


def test_unmutated_copy_passes():
    pin_decode_equals_forward(_mutant("none"))
