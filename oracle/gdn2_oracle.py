"""Float64 CPU oracle of the Gated Delta Rule-2 (GDN-2) token mixer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import or run this module. The library never routes through it.

It is the plain definition: the token-by-token recurrence, written out in float64 over
inputs upcast exactly from their run dtype. No chunking, no blocking, no reordering.

Sources (the pages this follows):
  [note §2]  "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
             (reading note), §2 Theoretical Framework: the decayed old state
             S_bar = Diag(alpha_t) S_{t-1}, the gated key e_t = b_t*k_t, the gated value
             z_t = w_t*v_t, and the fast-weight objective
             ||S - S_bar||_F^2 - 2 <S^T k_t, z_t - S_bar^T e_t>, whose minimiser is the
             update below.
  [note §3]  same page, §3 Technical Architecture: the forward-pass paragraph gives the
             step order (gate, decay, read r_t = S_bar^T e_t, erase, write); the
             gate-aware backward paragraph names the asymmetric factor (I - k_t e_t^T).
  [abstract] "Gated DeltaNet-2" abstract page: erase is key-side, write is value-side;
             b = w = beta*1 reduces to KDA, and scalar decay further to Gated DeltaNet.

Readings taken where the pages are garbled or silent (each is pinned by a test):
  * The erase outer product runs along k_t (S_bar - k_t r_t^T). The forward-pass
    paragraph prints e_t r_t^T, but that contradicts the objective's minimiser, the
    (I - k_t e_t^T) factor and the KDA reduction; the objective decides.
  * State layout is [d_k, d_v] (Diag(alpha) multiplies from the left, read is S^T e).
  * The readout uses the post-update state: o_t = S_t^T q_t.
  * No query scale; alpha is passed as g = log(alpha) <= 0.
  * Decay is applied before the read (the forward-pass paragraph's order).
  * Varlen: each cu_seqlens segment is an independent sequence with its own state.

Backward ([note §3], gate-aware backward paragraph: the gradient of the state flows through
the asymmetric factor, dS_{t-1} = Diag(alpha_t) (I - e_t k_t^T) dS_t, plus the readout's
q_t do_t^T). gdn2_backward is the reverse token loop: the chain rule applied to the step
above in float64, one token at a time, with the forward states recomputed and kept.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gdn2_step", "gdn2_forward", "gdn2_decode_steps", "gdn2_decode_tokens",
           "gdn2_step_backward", "gdn2_backward"]


def gdn2_step(S, q, k, v, g, b, w):
    """One token of Gated Delta Rule-2 for a batch of independent states.

    S: [..., d_k, d_v] float64 state S_{t-1}; q, k, g, b: [..., d_k]; v, w: [..., d_v].
    Returns (o_t [..., d_v], S_t [..., d_k, d_v]).

    [note §3] forward pass: e = b*k, z = w*v; S_bar = Diag(alpha) S; r = S_bar^T e;
    S_t = S_bar - k r^T + k z^T (erase along k, see module docstring); o_t = S_t^T q.
    """
    S = np.asarray(S, dtype=np.float64)
    alpha = np.exp(np.asarray(g, dtype=np.float64))
    e = np.asarray(b, np.float64) * np.asarray(k, np.float64)
    z = np.asarray(w, np.float64) * np.asarray(v, np.float64)
    k = np.asarray(k, np.float64)
    q = np.asarray(q, np.float64)
    S_bar = alpha[..., :, None] * S
    r = np.einsum("...c,...cv->...v", e, S_bar)
    S_new = S_bar + k[..., :, None] * (z - r)[..., None, :]
    o = np.einsum("...c,...cv->...v", q, S_new)
    return o, S_new


def _run_sequence(q, k, v, g, b, w, S):
    """Token loop over one sequence. q..w: [L, H, d]; S: [H, d_k, d_v]."""
    L = q.shape[0]
    o = np.zeros(v.shape, dtype=np.float64)
    for t in range(L):
        o[t], S = gdn2_step(S, q[t], k[t], v[t], g[t], b[t], w[t])
    return o, S


def gdn2_forward(q, k, v, g, b, w, s0=None, cu_seqlens=None):
    """Gated Delta Rule-2 over whole sequences.

    q, k, g, b: [B, T, H, d_k]; v, w: [B, T, H, d_v] (any float dtype; upcast to float64).
    s0: [N, H, d_k, d_v] initial states, or None for zeros.
    cu_seqlens: None (N = B sequences of length T) or int [N+1] offsets into the token
    axis of a B = 1 packed batch; each segment starts from its own s0[n].
    Returns (o [B, T, H, d_v] float64, S_final [N, H, d_k, d_v] float64).
    """
    q, k, v, g, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(n, 0, T) for n in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        if B != 1:
            raise ValueError("varlen inputs are packed with B == 1")
        bounds = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(bounds)
    if s0 is None:
        s0 = np.zeros((N, H, dk, dv))
    s0 = np.asarray(s0, dtype=np.float64)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_final = np.zeros((N, H, dk, dv), dtype=np.float64)
    for n, (bi, t0, t1) in enumerate(bounds):
        sl = (bi, slice(t0, t1))
        o[sl], S_final[n] = _run_sequence(q[sl], k[sl], v[sl], g[sl], b[sl], w[sl],
                                          s0[n].copy())
    return o, S_final


def gdn2_decode_steps(S, q, k, v, g, b, w):
    """Consecutive single-token steps on a pool of states.

    S: [N, H, d_k, d_v]; q, k, g, b: [steps, N, H, d_k]; v, w: [steps, N, H, d_v].
    Returns (o [steps, N, H, d_v], S after the last step). The decode step is the same
    recurrence as the forward pass, one token at a time ([note §3]).
    """
    S = np.asarray(S, dtype=np.float64).copy()
    steps = q.shape[0]
    o = np.zeros(v.shape, dtype=np.float64)
    for s in range(steps):
        o[s], S = gdn2_step(S, q[s], k[s], v[s], g[s], b[s], w[s])
    return o, S


def gdn2_decode_tokens(pool, q, k, v, g, b, w, indices=None, commit=None):
    """L consecutive tokens per sequence against a pool of states (the per-token procedure of
    [note §3], applied L times; serving use: decode or draft verification, [note §7]).

    pool: [P, H, d_k, d_v]; q, k, g, b: [N, L, H, d_k]; v, w: [N, L, H, d_v].
    indices: [N] pool slot per sequence (None: slot n); a slot outside [0, P) skips the
    sequence (its outputs stay zero). commit: [N] number of leading tokens whose update is
    written back to the slot (clamped to [0, L]; None: L).
    Returns (o [N, L, H, d_v], step_states [N, L, H, d_k, d_v] (the state after every
    token), new_pool); all float64.
    """
    pool = np.asarray(pool, dtype=np.float64)
    q, k, v, g, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, w))
    N, L = q.shape[:2]
    P = pool.shape[0]
    new_pool = pool.copy()
    o = np.zeros(v.shape)
    states = np.zeros((N, L) + pool.shape[1:])
    for n in range(N):
        slot = n if indices is None else int(indices[n])
        if slot < 0 or slot >= P:
            continue
        c = L if commit is None else min(max(int(commit[n]), 0), L)
        S = pool[slot].copy()
        for t in range(L):
            o[n, t], S = gdn2_step(S, q[n, t], k[n, t], v[n, t], g[n, t], b[n, t], w[n, t])
            states[n, t] = S
            if t + 1 == c:
                new_pool[slot] = S
    return o, states, new_pool


def gdn2_step_backward(S_prev, q, k, v, g, b, w, do, dS):
    """Reverse of gdn2_step for one token (one state; no batch axes).

    S_prev: [d_k, d_v] state before the token; q, k, g, b: [d_k]; v, w: [d_v];
    do: [d_v] gradient of o_t; dS: [d_k, d_v] gradient of S_t from later tokens.
    Returns (dq, dk, dv, dg, db, dw, dS_prev).

    With S_bar = Diag(alpha) S_prev, e = b*k, z = w*v, r = S_bar^T e,
    S_t = S_bar + k (z - r)^T and o_t = S_t^T q:
      dS_t   = dS + q do^T            dq = S_t do
      dz     = dS_t^T k               dr = -dz
      dk     = dS_t (z - r) + b * de  de = S_bar dr   (r = S_bar^T e)
      dS_bar = dS_t + e dr^T  = (I - e k^T) dS_t
      dalpha = rowsum(dS_bar * S_prev), dg = alpha * dalpha
      dS_prev = Diag(alpha) dS_bar
      db = de * k,  dw = dz * v,  dv = dz * w
    """
    alpha = np.exp(g)
    e = b * k
    z = w * v
    S_bar = alpha[:, None] * S_prev
    r = S_bar.T @ e
    S_t = S_bar + np.outer(k, z - r)
    dS_t = dS + np.outer(q, do)
    dq = S_t @ do
    dz = dS_t.T @ k
    dr = -dz
    de = S_bar @ dr
    dk = dS_t @ (z - r) + b * de
    dS_bar = dS_t + np.outer(e, dr)
    dg = alpha * np.sum(dS_bar * S_prev, axis=1)
    dS_prev = alpha[:, None] * dS_bar
    return dq, dk, dz * w, dg, de * k, dz * v, dS_prev


def gdn2_backward(q, k, v, g, b, w, do, dS_final=None, s0=None, cu_seqlens=None):
    """Gradients of gdn2_forward for upstream gradients `do` (of o, [B, T, H, d_v]) and
    `dS_final` (of the final states, [N, H, d_k, d_v], or None for zero).

    Same shapes and conventions as gdn2_forward. Returns
    (dq, dk, dv, dg, db, dw, ds0): gradients of q, k, v, g (= log alpha), b, w with the
    inputs' shapes, and of the initial states [N, H, d_k, d_v]; all float64.
    """
    q, k, v, g, b, w, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, w, do))
    B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    if cu_seqlens is None:
        bounds = [(n, 0, T) for n in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        if B != 1:
            raise ValueError("varlen inputs are packed with B == 1")
        bounds = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(bounds)
    s0 = np.zeros((N, H, dk_, dv_)) if s0 is None else np.asarray(s0, np.float64)
    dS_final = np.zeros((N, H, dk_, dv_)) if dS_final is None else np.asarray(dS_final, np.float64)
    grads = [np.zeros_like(x) for x in (q, k, v, g, b, w)]
    ds0 = np.zeros((N, H, dk_, dv_))
    for n, (bi, t0, t1) in enumerate(bounds):
        for h in range(H):
            # forward states before every token of this sequence
            states = [s0[n, h].copy()]
            for t in range(t0, t1):
                _, S = gdn2_step(states[-1], q[bi, t, h], k[bi, t, h], v[bi, t, h],
                                 g[bi, t, h], b[bi, t, h], w[bi, t, h])
                states.append(S)
            dS = dS_final[n, h].copy()
            for t in range(t1 - 1, t0 - 1, -1):
                out = gdn2_step_backward(states[t - t0], q[bi, t, h], k[bi, t, h], v[bi, t, h],
                                         g[bi, t, h], b[bi, t, h], w[bi, t, h], do[bi, t, h], dS)
                for gr, d in zip(grads, out[:6]):
                    gr[bi, t, h] = d
                dS = out[6]
            ds0[n, h] = dS
    return (*grads, ds0)
