"""Pins of the oracle's backward (gdn2_backward) against something other than itself:
central finite differences of the forward oracle, planted mistakes that must be caught, and
the chunk algebra that the GPU backward follows (chunked == sequential)."""
import numpy as np
import pytest

from oracle import gdn2_backward, gdn2_forward
from oracle import gdn2_oracle as O
from tests.chunk_form import chunked_backward

NAMES = ("q", "k", "v", "g", "b", "w")


def _problem(rng, B, T, H, dk, dv):
    x = dict(q=rng.normal(size=(B, T, H, dk)), k=rng.normal(size=(B, T, H, dk)) / 2,
             v=rng.normal(size=(B, T, H, dv)), g=-rng.uniform(0.01, 0.6, size=(B, T, H, dk)),
             b=rng.uniform(0, 1, size=(B, T, H, dk)), w=rng.uniform(0, 1, size=(B, T, H, dv)))
    return x


def _fd_grads(x, s0, R, R2, cu=None, eps=1e-6):
    """Central differences of L = <o, R> + <S_final, R2> w.r.t. every input and s0."""
    def loss(xx, s):
        o, S = gdn2_forward(*(xx[n] for n in NAMES), s0=s, cu_seqlens=cu)
        return float(np.sum(o * R) + np.sum(S * R2))
    out = []
    for n in NAMES:
        fd = np.zeros_like(x[n])
        for idx in np.ndindex(x[n].shape):
            xp = dict(x); xm = dict(x)
            xp[n] = x[n].copy(); xm[n] = x[n].copy()
            xp[n][idx] += eps
            xm[n][idx] -= eps
            fd[idx] = (loss(xp, s0) - loss(xm, s0)) / (2 * eps)
        out.append(fd)
    fd = np.zeros_like(s0)
    for idx in np.ndindex(s0.shape):
        sp, sm = s0.copy(), s0.copy()
        sp[idx] += eps
        sm[idx] -= eps
        fd[idx] = (loss(x, sp) - loss(x, sm)) / (2 * eps)
    out.append(fd)
    return out


def _max_rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 6, 1, 4, 3), (2, 5, 2, 3, 5)])
def test_backward_matches_finite_differences(B, T, H, dk, dv):
    rng = np.random.default_rng(100 + T + dk)
    x = _problem(rng, B, T, H, dk, dv)
    s0 = rng.normal(size=(B, H, dk, dv))
    R = rng.normal(size=(B, T, H, dv))
    R2 = rng.normal(size=(B, H, dk, dv))
    grads = gdn2_backward(*(x[n] for n in NAMES), R, dS_final=R2, s0=s0)
    fd = _fd_grads(x, s0, R, R2)
    for name, gr, f in zip(NAMES + ("s0",), grads, fd):
        assert _max_rel(gr, f) < 1e-7, name


def test_backward_varlen_matches_finite_differences():
    rng = np.random.default_rng(7)
    lens = [3, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _problem(rng, 1, sum(lens), 1, 3, 2)
    s0 = rng.normal(size=(3, 1, 3, 2))
    R = rng.normal(size=(1, sum(lens), 1, 2))
    R2 = rng.normal(size=(3, 1, 3, 2))
    grads = gdn2_backward(*(x[n] for n in NAMES), R, dS_final=R2, s0=s0, cu_seqlens=cu)
    fd = _fd_grads(x, s0, R, R2, cu=cu)
    for name, gr, f in zip(NAMES + ("s0",), grads, fd):
        assert _max_rel(gr, f) < 1e-7, name
    # the empty sequence passes its final-state gradient straight to its initial state
    assert np.array_equal(grads[6][1], R2[1])


def _mutants():
    """Broken copies of the reverse step: each must be caught by the finite differences."""
    def mk(kind):
        def step(S_prev, q, k, v, g, b, w, do, dS):
            alpha = np.exp(g)
            e, z = b * k, w * v
            S_bar = alpha[:, None] * S_prev
            r = S_bar.T @ e
            S_t = S_bar + np.outer(k, z - r)
            dS_t = dS + np.outer(q, do)
            dq = (S_prev if kind == "dq_old_state" else S_t) @ do
            dz = dS_t.T @ k
            dr = dz if kind == "dr_sign" else -dz
            de = S_bar @ dr
            dk = dS_t @ (z - r) + (0.0 if kind == "dk_no_erase_term" else b * de)
            dS_bar = dS_t + (np.outer(k, dr) if kind == "factor_transposed" else np.outer(e, dr))
            dg = np.sum(dS_bar * S_prev, axis=1) * (1.0 if kind == "dg_no_alpha" else alpha)
            dS_prev = dS_bar if kind == "no_decay_carry" else alpha[:, None] * dS_bar
            db = de * (b if kind == "db_wrong_factor" else k)
            return dq, dk, dz * w, dg, db, dz * v, dS_prev
        return step
    return ["dq_old_state", "dr_sign", "dk_no_erase_term", "factor_transposed", "dg_no_alpha",
            "no_decay_carry", "db_wrong_factor"], mk


def test_planted_backward_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(3)
    x = _problem(rng, 1, 5, 1, 4, 3)
    s0 = rng.normal(size=(1, 1, 4, 3))
    R = rng.normal(size=(1, 5, 1, 3))
    R2 = rng.normal(size=(1, 1, 4, 3))
    fd = _fd_grads(x, s0, R, R2)
    kinds, mk = _mutants()
    for kind in kinds:
        monkeypatch.setattr(O, "gdn2_step_backward", mk(kind))
        grads = O.gdn2_backward(*(x[n] for n in NAMES), R, dS_final=R2, s0=s0)
        worst = max(_max_rel(gr, f) for gr, f in zip(grads, fd))
        assert worst > 1e-3, kind
    monkeypatch.undo()


@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("L", [37, 130])
def test_chunked_backward_equals_sequential(C, L):
    rng = np.random.default_rng(C * 1000 + L)
    dk, dv = 8, 6
    x = _problem(rng, 1, L, 1, dk, dv)
    s0 = rng.normal(size=(1, 1, dk, dv)) * 0.3
    R = rng.normal(size=(1, L, 1, dv))
    R2 = rng.normal(size=(1, 1, dk, dv))
    ref = gdn2_backward(*(x[n] for n in NAMES), R, dS_final=R2, s0=s0)
    got = chunked_backward(*(x[n][0, :, 0] for n in NAMES), s0[0, 0], R[0, :, 0], R2[0, 0], C)
    for name, a, r in zip(NAMES, got[:6], ref[:6]):
        assert _max_rel(a, r[0, :, 0]) < 1e-9, name
    assert _max_rel(got[6], ref[6][0, 0]) < 1e-9


@pytest.mark.parametrize("n", [1, 5, 64])
def test_backward_regrouping_equals_chunk_backward(n):
    from tests.chunk_form import chunk_backward_parts, chunk_step_backward
    rng = np.random.default_rng(40 + n)
    dk, dv = 8, 6
    x = _problem(rng, 1, n, 1, dk, dv)
    args = [x[m][0, :, 0] for m in NAMES]
    S0 = rng.normal(size=(dk, dv))
    dO = rng.normal(size=(n, dv))
    dSn = rng.normal(size=(dk, dv))
    ref = chunk_step_backward(S0, *args, dO, dSn)
    got = chunk_backward_parts(S0, *args, dO, dSn)
    for a, r in zip(got, ref):
        assert _max_rel(a, r) < 1e-10
