"""Float64 chunkwise (WY / UT-transform) form of Gated Delta Rule-2, for the tests.

This is a second, independent derivation used only to pin the algebra that the HIP
chunk kernel follows against the token-by-token oracle (chunked == sequential). It is
not a parity source: GPU results are always compared with the oracle itself.

Within one chunk of n tokens with incoming state S0 ([d_k, d_v]) and G = cumsum(g):
  A[r,i] = sum_c e[r,c] k[i,c] exp(G[r,c] - G[i,c])   for i <  r   ((b*k) Gamma k^T)
  P[r,i] = sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])   for i <= r
  T      = (I + A)^{-1}                                 (UT transform)
  W      = T (E * exp(G)),   U~ = T Z
  U      = U~ - W S0
  O      = (Q * exp(G)) S0 + P U
  S_n    = Diag(exp(G[n-1])) S0 + (K * exp(G[n-1] - G))^T U
The decay-normalised state of the GDN-2 reading note (§3, chunkwise-training
paragraph: S_r = Diag(gamma_r) S^_r) turns the chunk into a pure asymmetric delta
recurrence; the UT transform of the Gated DeltaNet visual reading (chunkwise section)
turns its product of delta factors into the triangular inverse above.
"""
from __future__ import annotations

import numpy as np


def chunk_step(S0, q, k, v, g, b, w):
    """One chunk for one head. q, k, g, b: [n, d_k]; v, w: [n, d_v]; S0: [d_k, d_v]."""
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    E = b * k
    Z = w * v
    D = G[:, None, :] - G[None, :, :]                      # G[r] - G[i]
    incl = np.tril(np.ones((n, n), dtype=bool))
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    decay_incl = np.exp(np.where(incl[:, :, None], D, -np.inf))
    A = np.einsum("rc,ic,ric->ri", E, k, decay_incl) * strict
    P = np.einsum("rc,ic,ric->ri", q, k, decay_incl)
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ (E * np.exp(G))
    Ut = T @ Z
    U = Ut - W @ S0
    O = (q * np.exp(G)) @ S0 + P @ U
    Gn = G[-1]
    S = np.exp(Gn)[:, None] * S0 + (k * np.exp(Gn[None, :] - G)).T @ U
    return O, S


def chunked_forward(q, k, v, g, b, w, s0, C):
    """Whole sequence for one head, chunk size C (last chunk may be shorter)."""
    L = q.shape[0]
    S = np.array(s0, dtype=np.float64)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        o[sl], S = chunk_step(S, q[sl], k[sl], v[sl], g[sl], b[sl], w[sl])
    return o, S


def chunk_step_backward(S0, q, k, v, g, b, w, dO, dSn):
    """Reverse of chunk_step for one chunk of one head.

    S0: [d_k, d_v] state entering the chunk; dO: [n, d_v] gradient of the chunk's output;
    dSn: [d_k, d_v] gradient of the state leaving it. Returns
    (dq, dk, dv, dg, db, dw, dS0). With the chunk quantities of chunk_step and
    Ebar = E exp(G), Qbar = q exp(G), Khat = k exp(-G), Ktil = k exp(G_last - G):
      dU    = P^T dO + Ktil dSn                dQbar = dO S0^T + dP Khat
      dP    = lower_incl(dO U^T)               dKtil = U dSn^T
      dW    = -dU S0^T                         dZ    = T^T dU
      dA    = -strict(dZ U~^T + (T^T dW) W^T)  (T = (I + A)^{-1})
      dEbar = T^T dW + dA Khat                 dKhat = dA^T Ebar + dP^T Qbar
      dS0   = Qbar^T dO + Diag(exp(G_last)) dSn - W^T dU
    and the elementwise chain through exp(+-G), e = b*k, z = w*v and G = cumsum(g).
    """
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Gn = G[-1]
    E = b * k
    Z = w * v
    incl = np.tril(np.ones((n, n)))
    strict = np.tril(np.ones((n, n)), -1)
    Ebar, Qbar, Khat = E * Gam, q * Gam, k / Gam
    Ktil = k * np.exp(Gn[None, :] - G)
    A = (Ebar @ Khat.T) * strict
    P = (Qbar @ Khat.T) * incl
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ Ebar
    Ut = T @ Z
    U = Ut - W @ S0
    dU = P.T @ dO + Ktil @ dSn
    dP = (dO @ U.T) * incl
    dQbar = dO @ S0.T + dP @ Khat
    dKtil = U @ dSn.T
    dW = -dU @ S0.T
    dZ = T.T @ dU
    dEbarT = T.T @ dW
    dA = -(dZ @ Ut.T + dEbarT @ W.T) * strict
    dEbar = dEbarT + dA @ Khat
    dKhat = dA.T @ Ebar + dP.T @ Qbar
    dS0 = Qbar.T @ dO + np.exp(Gn)[:, None] * dSn - W.T @ dU
    dE = dEbar * Gam
    dq = dQbar * Gam
    dk = dKhat / Gam + dKtil * np.exp(Gn[None, :] - G) + dE * b
    dG = dEbar * Ebar + dQbar * Qbar - dKhat * Khat - dKtil * Ktil
    dG[-1] += np.sum(dKtil * Ktil, axis=0) + np.sum(dSn * np.exp(Gn)[:, None] * S0, axis=1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dq, dk, dZ * w, dg, dE * k, dZ * v, dS0


def chunked_backward(q, k, v, g, b, w, s0, dO, dSn, C):
    """Whole-sequence backward for one head with chunk size C: a forward pass keeps the
    state entering every chunk, then the chunks run in reverse carrying dS."""
    L = q.shape[0]
    starts = list(range(0, L, C))
    S = np.array(s0, dtype=np.float64)
    states = []
    for c0 in starts:
        states.append(S)
        sl = slice(c0, min(c0 + C, L))
        _, S = chunk_step(S, q[sl], k[sl], v[sl], g[sl], b[sl], w[sl])
    grads = [np.zeros_like(x) for x in (q, k, v, g, b, w)]
    dS = np.array(dSn, dtype=np.float64)
    for ci in range(len(starts) - 1, -1, -1):
        sl = slice(starts[ci], min(starts[ci] + C, L))
        out = chunk_step_backward(states[ci], q[sl], k[sl], v[sl], g[sl], b[sl], w[sl],
                                  dO[sl], dS)
        for gr, d in zip(grads, out[:6]):
            gr[sl] = d
        dS = out[6]
    return (*grads, dS)


def chunk_backward_parts(S0, q, k, v, g, b, w, dO, dSn):
    """chunk_step_backward regrouped the way the GPU backward computes it:

      recurrence part (sequential over chunks, per value column):
        dU  = P^T dO + Ktil dSn,    dZ = T^T dU,    dv = dZ * w,   dw = dZ * v,
        dS0 = Qbar^T dO + Diag(exp(G_last)) dSn - W^T dU
      local part (per chunk, needs only U = U~ - W S0, S0, dSn, dO, dZ and exp(+-G)):
        M1 = lower_incl(dO U^T),    M2 = -strict(dZ U^T)             (M2 = dA)
        dQbar = dO S0^T + M1 Khat,  dEbar = -dZ S0^T + M2 Khat,   dKhat = M2^T Ebar + M1^T Qbar,
        dKtil = U dSn^T
    The regrouping uses T^T dW = -(T^T dU) S0^T = -dZ S0^T, so that
    dA = -strict(dZ U~^T + (T^T dW) W^T) = -strict(dZ (U~ - W S0)^T) = -strict(dZ U^T):
    one triangular solve per chunk instead of two, and no use of T or A in the local part.
    Returns the same tuple as chunk_step_backward.
    """
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Gn = G[-1]
    E, Z = b * k, w * v
    incl = np.tril(np.ones((n, n)))
    strict = np.tril(np.ones((n, n)), -1)
    Ebar, Qbar, Khat = E * Gam, q * Gam, k / Gam
    Ktil = k * np.exp(Gn[None, :] - G)
    A = (Ebar @ Khat.T) * strict
    P = (Qbar @ Khat.T) * incl
    T = np.linalg.inv(np.eye(n) + A)
    W = T @ Ebar
    U = T @ Z - W @ S0
    # recurrence part
    dU = P.T @ dO + Ktil @ dSn
    dZ = T.T @ dU
    dS0 = Qbar.T @ dO + np.exp(Gn)[:, None] * dSn - W.T @ dU
    # local part
    M1 = (dO @ U.T) * incl
    M2 = -(dZ @ U.T) * strict
    dQbar = dO @ S0.T + M1 @ Khat
    dEbar = -dZ @ S0.T + M2 @ Khat
    dKhat = M2.T @ Ebar + M1.T @ Qbar
    dKtil = U @ dSn.T
    dE = dEbar * Gam
    dk = dKhat / Gam + dKtil * np.exp(Gn[None, :] - G) + dE * b
    dG = dEbar * Ebar + dQbar * Qbar - dKhat * Khat - dKtil * Ktil
    dG[-1] += np.sum(dKtil * Ktil, axis=0) + np.sum(dSn * np.exp(Gn)[:, None] * S0, axis=1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dQbar * Gam, dk, dZ * w, dg, dE * k, dZ * v, dS0
