"""Pins for the float64 oracle: what the pages and plain mathematics fix.

Each pin is written from its own formula (a reduction printed on a page, a closed form,
an invariant or a brute-force sum), never by calling the oracle's step twice. The pins
take the step function as an argument so that `test_pins_catch_planted_mistakes` can
run them against deliberately broken copies of the step (mistakes planted here, on the
CPU) and show that each mistake is caught.

Sources:
  GDN-2 reading note ("Gated DeltaNet-2: Decoupling Erase and Write in Linear
  Attention"): §2 objective and reductions, §3 forward pass and chunk form.
  GDN-2 abstract page: reduction to KDA (b = w = beta*1) and to Gated DeltaNet.
  "Gated Delta Net" review, §1.1: linear attention, Mamba2-style decay, DeltaNet and
  gated delta rule formulas (written there in the d_v x d_k layout).
  Gated DeltaNet visual reading: one-hot memory-slot simulation.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import gdn2_forward, gdn2_step
from tests.chunk_form import chunked_forward

RTOL = 1e-12


def _close(a, b, tol=RTOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol:.1e} * {scale:.3e}"


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(rng, L, dk, dv, *, gates="dense"):
    """Random single-head inputs in float64. k and q have unit norm."""
    c = dict(
        q=_unit(rng.standard_normal((L, dk))),
        k=_unit(rng.standard_normal((L, dk))),
        v=rng.standard_normal((L, dv)),
        g=-0.3 * np.log1p(np.exp(rng.standard_normal((L, dk)))),
        b=1.0 / (1.0 + np.exp(-rng.standard_normal((L, dk)))),
        w=1.0 / (1.0 + np.exp(-rng.standard_normal((L, dv)))),
    )
    return c


def _run(step, S0, c):
    """Token loop driven by `step` (the oracle's or a planted-mistake copy)."""
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((c["q"].shape[0], c["v"].shape[1]))
    for t in range(c["q"].shape[0]):
        o[t], S = step(S, c["q"][t], c["k"][t], c["v"][t], c["g"][t], c["b"][t], c["w"][t])
    return o, S


DIMS = [(8, 6), (6, 8), (16, 16)]


# ---------------------------------------------------------------- pins P1..P10
def pin_objective(step, dk, dv, seed=1):
    """P1. The state after a step minimises the GDN-2 fast-weight objective
    F(S) = ||S - S_bar||_F^2 - 2 <S^T k, z - S_bar^T e>  (note §2), with
    S_bar = Diag(alpha) S_prev, e = b*k, z = w*v. F is a convex quadratic, so the
    minimiser is unique: check a zero gradient and that random moves never lower F."""
    rng = np.random.default_rng(seed)
    c = _case(rng, 1, dk, dv)
    S_prev = rng.standard_normal((dk, dv))
    _, S = step(S_prev, c["q"][0], c["k"][0], c["v"][0], c["g"][0], c["b"][0], c["w"][0])
    k, e, z = c["k"][0], c["b"][0] * c["k"][0], c["w"][0] * c["v"][0]
    S_bar = np.exp(c["g"][0])[:, None] * S_prev
    y = z - S_bar.T @ e

    def F(X):
        return np.sum((X - S_bar) ** 2) - 2.0 * (k @ X @ y)

    grad = 2.0 * (S - S_bar) - 2.0 * np.outer(k, y)
    _close(grad, np.zeros_like(grad), 1e-12)
    f0 = F(S)
    for _ in range(8):
        assert F(S + 1e-3 * rng.standard_normal(S.shape)) > f0


def pin_kda(step, dk, dv, seed=2):
    """P2. b = w = beta*1 gives KDA: S_t = (I - beta k k^T) Diag(alpha) S + beta k v^T
    (GDN-2 abstract; note §2 reductions)."""
    rng = np.random.default_rng(seed)
    c = _case(rng, 12, dk, dv)
    beta = rng.uniform(0.05, 1.0, size=12)
    c["b"] = beta[:, None] * np.ones((12, dk))
    c["w"] = beta[:, None] * np.ones((12, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    R = S0.copy()
    for t in range(12):
        k = c["k"][t]
        R = (np.eye(dk) - beta[t] * np.outer(k, k)) @ np.diag(np.exp(c["g"][t])) @ R \
            + beta[t] * np.outer(k, c["v"][t])
        _close(o[t], R.T @ c["q"][t])
    _close(S, R)


def pin_gated_deltanet(step, dk, dv, seed=3):
    """P3. With scalar decay as well, Gated DeltaNet in the review's d_v x d_k layout:
    M_t = alpha_t M_{t-1} (I - beta_t k k^T) + beta_t v k^T, o_t = M_t q_t, M = S^T
    ("Gated Delta Net" review §1.1)."""
    rng = np.random.default_rng(seed)
    c = _case(rng, 12, dk, dv)
    beta = rng.uniform(0.05, 1.0, size=12)
    a = rng.uniform(0.3, 1.0, size=12)
    c["g"] = np.log(a)[:, None] * np.ones((12, dk))
    c["b"] = beta[:, None] * np.ones((12, dk))
    c["w"] = beta[:, None] * np.ones((12, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    M = S0.T.copy()
    for t in range(12):
        k = c["k"][t]
        M = a[t] * M @ (np.eye(dk) - beta[t] * np.outer(k, k)) + beta[t] * np.outer(c["v"][t], k)
        _close(o[t], M @ c["q"][t])
    _close(S, M.T)


def pin_deltanet(step, dk, dv, seed=4):
    """P4. alpha = 1, b = w = beta*1: DeltaNet, both forms of the review's §1.1:
    M_t = M(I - beta k k^T) + beta v k^T = M + beta (v - M k) k^T."""
    rng = np.random.default_rng(seed)
    c = _case(rng, 10, dk, dv)
    beta = rng.uniform(0.05, 1.0, size=10)
    c["g"] = np.zeros((10, dk))
    c["b"] = beta[:, None] * np.ones((10, dk))
    c["w"] = beta[:, None] * np.ones((10, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    M1 = S0.T.copy()
    M2 = S0.T.copy()
    for t in range(10):
        k, v = c["k"][t], c["v"][t]
        M1 = M1 @ (np.eye(dk) - beta[t] * np.outer(k, k)) + beta[t] * np.outer(v, k)
        M2 = M2 + beta[t] * np.outer(v - M2 @ k, k)
        _close(o[t], M1 @ c["q"][t])
    _close(S, M1.T)
    _close(M1, M2)


def pin_linear_attention(step, dk, dv, seed=5):
    """P5. alpha = 1, b = 0, w = 1: linear attention S_t = S_{t-1} + k v^T (review
    §1.1), so o_t = S0^T q_t + sum_{i<=t} (q_t . k_i) v_i  (current token included)."""
    rng = np.random.default_rng(seed)
    L = 9
    c = _case(rng, L, dk, dv)
    c["g"] = np.zeros((L, dk))
    c["b"] = np.zeros((L, dk))
    c["w"] = np.ones((L, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    for t in range(L):
        ref = S0.T @ c["q"][t]
        for i in range(t + 1):
            ref = ref + (c["q"][t] @ c["k"][i]) * c["v"][i]
        _close(o[t], ref)
    _close(S, S0 + c["k"].T @ c["v"])


def pin_mamba2(step, dk, dv, seed=6):
    """P6. Scalar alpha, b = 0, w = 1: S_t = alpha_t S_{t-1} + k v^T (review §1.1), so
    o_t = (prod_{j<=t} a_j) S0^T q_t + sum_i (prod_{i<j<=t} a_j)(q_t . k_i) v_i."""
    rng = np.random.default_rng(seed)
    L = 9
    c = _case(rng, L, dk, dv)
    a = rng.uniform(0.2, 1.0, size=L)
    c["g"] = np.log(a)[:, None] * np.ones((L, dk))
    c["b"] = np.zeros((L, dk))
    c["w"] = np.ones((L, dv))
    S0 = rng.standard_normal((dk, dv))
    o, _ = _run(step, S0, c)
    for t in range(L):
        ref = np.prod(a[: t + 1]) * (S0.T @ c["q"][t])
        for i in range(t + 1):
            ref = ref + np.prod(a[i + 1: t + 1]) * (c["q"][t] @ c["k"][i]) * c["v"][i]
        _close(o[t], ref)


def pin_one_hot_slots(step, dk, dv, seed=7):
    """P7. One-hot key k = e_c (the visual reading's memory-slot simulation): every row
    decays by its own alpha, and only row c is edited:
    row c -> (1 - b_c) alpha_c S[c,:] + w*v; row j != c -> alpha_j S[j,:]."""
    rng = np.random.default_rng(seed)
    S_prev = rng.standard_normal((dk, dv))
    for cidx in (0, dk - 1, dk // 2):
        c = _case(rng, 1, dk, dv)
        k = np.zeros(dk)
        k[cidx] = 1.0
        _, S = step(S_prev, c["q"][0], k, c["v"][0], c["g"][0], c["b"][0], c["w"][0])
        alpha = np.exp(c["g"][0])
        ref = alpha[:, None] * S_prev
        ref[cidx] = (1.0 - c["b"][0][cidx]) * alpha[cidx] * S_prev[cidx] + c["w"][0] * c["v"][0]
        _close(S, ref)


def pin_read_back(step, dk, dv, seed=8):
    """P8. For unit k, reading the new state with k gives
    S_t^T k = S_bar^T ((1 - b) * k) + w * v; with b = w = 1 it returns v exactly
    (the delta rule writes the target along k, review §1.1)."""
    rng = np.random.default_rng(seed)
    S_prev = rng.standard_normal((dk, dv))
    c = _case(rng, 1, dk, dv)
    k, b, w, v = c["k"][0], c["b"][0], c["w"][0], c["v"][0]
    _, S = step(S_prev, c["q"][0], k, v, c["g"][0], b, w)
    S_bar = np.exp(c["g"][0])[:, None] * S_prev
    _close(S.T @ k, S_bar.T @ ((1.0 - b) * k) + w * v)
    _, S1 = step(S_prev, c["q"][0], k, v, c["g"][0], np.ones(dk), np.ones(dv))
    _close(S1.T @ k, v)


def pin_no_erase_closed_form(step, dk, dv, seed=9):
    """P9. b = 0 with per-channel decay: O(T^2) brute force
    o_t = S0^T (q_t * e^{G_t}) + sum_{i<=t} sum_c q_tc k_ic e^{G_tc - G_ic} (w_i * v_i),
    G = cumsum(g): pins the per-key-channel placement of the decay."""
    rng = np.random.default_rng(seed)
    L = 11
    c = _case(rng, L, dk, dv)
    c["b"] = np.zeros((L, dk))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    G = np.cumsum(c["g"], axis=0)
    for t in range(L):
        ref = S0.T @ (c["q"][t] * np.exp(G[t]))
        for i in range(t + 1):
            s = np.sum(c["q"][t] * c["k"][i] * np.exp(G[t] - G[i]))
            ref = ref + s * (c["w"][i] * c["v"][i])
        _close(o[t], ref)


def pin_pure_decay(step, dk, dv, seed=10):
    """P10. b = w = 0: no edit at all, S_T = Diag(exp(sum_t g_t)) S0 and
    o_t = S0^T (q_t * e^{G_t})."""
    rng = np.random.default_rng(seed)
    L = 7
    c = _case(rng, L, dk, dv)
    c["b"] = np.zeros((L, dk))
    c["w"] = np.zeros((L, dv))
    S0 = rng.standard_normal((dk, dv))
    o, S = _run(step, S0, c)
    G = np.cumsum(c["g"], axis=0)
    _close(S, np.exp(G[-1])[:, None] * S0)
    for t in range(L):
        _close(o[t], S0.T @ (c["q"][t] * np.exp(G[t])))


PINS = [pin_objective, pin_kda, pin_gated_deltanet, pin_deltanet, pin_linear_attention,
        pin_mamba2, pin_one_hot_slots, pin_read_back, pin_no_erase_closed_form,
        pin_pure_decay]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("dims", DIMS, ids=lambda d: f"dk{d[0]}_dv{d[1]}")
def test_oracle_pins(pin, dims):
    pin(gdn2_step, *dims)


# ------------------------------------------------- planted mistakes must be caught
def _mk_mutant(kind):
    def step(S, q, k, v, g, b, w):
        alpha = np.exp(g)
        e, z = b * k, w * v
        if kind == "write_gate_on_key":
            e, z = w * k, b * v
        S_bar = alpha[:, None] * S
        if kind == "decay_on_value_axis":
            S_bar = S * alpha[None, :]
        r = (S if kind == "read_before_decay" else S_bar).T @ e
        if kind == "erase_along_e":
            S_new = S_bar - np.outer(e, r) + np.outer(k, z)
        elif kind == "erase_sign":
            S_new = S_bar + np.outer(k, z + r)
        elif kind == "no_write_gate":
            S_new = S_bar + np.outer(k, v - r)
        elif kind == "decay_after_edit":
            S_new = alpha[:, None] * (S + np.outer(k, z - S.T @ e))
        else:
            S_new = S_bar + np.outer(k, z - r)
        if kind == "readout_pre_update":
            o = S_bar.T @ q
        elif kind == "readout_transposed":
            o = S_new @ q
        else:
            o = S_new.T @ q
        return o, S_new
    return step


MUTANTS = ["erase_along_e", "erase_sign", "no_write_gate", "read_before_decay",
           "decay_after_edit", "readout_pre_update", "readout_transposed",
           "decay_on_value_axis", "write_gate_on_key"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    step = _mk_mutant(kind)
    caught = []
    for pin in PINS:
        for dims in DIMS:
            try:
                pin(step, *dims)
            except (AssertionError, ValueError, IndexError):
                caught.append((pin.__name__, dims))
    assert caught, f"planted mistake {kind!r} passed every pin"


def test_unmutated_copy_passes():
    step = _mk_mutant("none")
    for pin in PINS:
        for dims in DIMS:
            pin(step, *dims)


# ------------------------------------------------------------- P11, P12 structure
@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("L", [37, 130])
def test_chunked_equals_sequential(C, L):
    """P11. The chunkwise WY/UT form (note §3 chunk paragraph; visual reading's UT
    transform) equals the token loop, for ragged lengths and several chunk sizes,
    including near-reset tokens (g = -5 on every channel)."""
    rng = np.random.default_rng(100 + C + L)
    dk, dv = 8, 6
    c = _case(rng, L, dk, dv)
    c["g"][::7] = -5.0
    S0 = rng.standard_normal((dk, dv))
    o_ref, S_ref = gdn2_forward(*(c[n][None, :, None, :] for n in "qkvgbw"),
                                s0=S0[None, None])
    o, S = chunked_forward(c["q"], c["k"], c["v"], c["g"], c["b"], c["w"], S0, C)
    _close(o, o_ref[0, :, 0], 1e-11)
    _close(S, S_ref[0, 0], 1e-11)


def test_state_carry():
    """P12a. Running [0, T1) then [T1, T) from the carried state equals one run."""
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 2, 40, 3, 8, 6
    x = {n: rng.standard_normal((B, T, H, dv if n in "vw" else dk)) for n in "qkvgbw"}
    x["g"] = -np.abs(x["g"]) * 0.2
    x["b"] = 1 / (1 + np.exp(-x["b"]))
    x["w"] = 1 / (1 + np.exp(-x["w"]))
    s0 = rng.standard_normal((B, H, dk, dv))
    o, S = gdn2_forward(*(x[n] for n in "qkvgbw"), s0=s0)
    o1, S1 = gdn2_forward(*(x[n][:, :17] for n in "qkvgbw"), s0=s0)
    o2, S2 = gdn2_forward(*(x[n][:, 17:] for n in "qkvgbw"), s0=S1)
    _close(np.concatenate([o1, o2], axis=1), o)
    _close(S2, S)


def test_varlen_equals_separate():
    """P12b. A packed (cu_seqlens) batch equals separate runs per sequence."""
    rng = np.random.default_rng(13)
    lens = [5, 1, 23, 64, 9]
    T, H, dk, dv = sum(lens), 2, 6, 8
    x = {n: rng.standard_normal((1, T, H, dv if n in "vw" else dk)) for n in "qkvgbw"}
    x["g"] = -np.abs(x["g"]) * 0.2
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, S = gdn2_forward(*(x[n] for n in "qkvgbw"), s0=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = gdn2_forward(*(x[m][:, sl] for m in "qkvgbw"), s0=s0[n:n + 1])
        _close(o[:, sl], on)
        _close(S[n], Sn[0])
