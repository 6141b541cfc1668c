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
"""
from __future__ import annotations

import numpy as np

__all__ = ["gdn2_step", "gdn2_forward", "gdn2_decode_steps"]


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
