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
