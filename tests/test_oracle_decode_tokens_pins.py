"""Pins of the oracle's multi-token decode (gdn2_decode_tokens) against the whole-sequence
forward (gdn2_forward, itself pinned in test_oracle_pins.py): outputs, committed prefixes,
per-token states, skipped slots."""
import numpy as np

from oracle import gdn2_decode_tokens, gdn2_forward

NAMES = ("q", "k", "v", "g", "b", "w")


def _tokens(rng, N, L, H, dk, dv):
    return dict(q=rng.normal(size=(N, L, H, dk)), k=rng.normal(size=(N, L, H, dk)) / 3,
                v=rng.normal(size=(N, L, H, dv)), g=-rng.uniform(0.01, 0.5, size=(N, L, H, dk)),
                b=rng.uniform(0, 1, size=(N, L, H, dk)), w=rng.uniform(0, 1, size=(N, L, H, dv)))


def test_outputs_and_commits_match_the_forward():
    rng = np.random.default_rng(5)
    N, L, H, dk, dv, P = 4, 5, 2, 6, 4, 7
    x = _tokens(rng, N, L, H, dk, dv)
    pool = rng.normal(size=(P, H, dk, dv))
    idx = np.array([3, 0, 6, 1])
    commit = np.array([5, 0, 2, 9])  # 9 clamps to L
    o, states, new_pool = gdn2_decode_tokens(pool, *(x[n] for n in NAMES), indices=idx,
                                             commit=commit)
    o_ref, s_ref = gdn2_forward(*(x[n] for n in NAMES), s0=pool[idx])
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(states[:, -1], s_ref, rtol=0, atol=1e-12)
    for n in range(N):
        c = min(commit[n], L)
        if c == 0:
            assert np.array_equal(new_pool[idx[n]], pool[idx[n]])
        else:
            _, s_c = gdn2_forward(*(x[m][n:n + 1, :c] for m in NAMES), s0=pool[idx[n]][None])
            assert np.allclose(new_pool[idx[n]], s_c[0], rtol=0, atol=1e-12)
            assert np.allclose(states[n, c - 1], s_c[0], rtol=0, atol=1e-12)
    untouched = [s for s in range(P) if s not in idx]
    assert np.array_equal(new_pool[untouched], pool[untouched])


def test_skipped_slots():
    rng = np.random.default_rng(6)
    x = _tokens(rng, 3, 2, 1, 3, 3)
    pool = rng.normal(size=(2, 1, 3, 3))
    o, _, new_pool = gdn2_decode_tokens(pool, *(x[n] for n in NAMES), indices=[-1, 1, 2])
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.array_equal(new_pool[0], pool[0])
    assert not np.array_equal(new_pool[1], pool[1])
