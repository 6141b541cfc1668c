"""Float64 CPU oracle of the GDN-2 block's prologue and epilogue around the token mixer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import or run this module. The library never routes through it.

Source: [note §3] "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention" (reading
note), §3 Technical Architecture, block data-flow paragraph: the query and key branches are
linear -> conv -> SiLU -> L2 norm; the value branch is linear -> conv -> SiLU (no
normalisation); the decay, erase and write gates have branches of their own, per channel; the
output is scaled by an RMSNorm with a SiLU gate. The linear projections are plain GEMMs and
are not part of this module.

Readings where the page is silent:
  * conv: causal depthwise convolution of width 4 over the tokens of each sequence (no bias;
    a sequence starts from zero history, so the convolution never crosses a cu_seqlens
    boundary): y[t, c] = sum_{j=0..3} weight[c, j] * x[t - 3 + j, c].
  * L2 norm over d_k per (token, head): x / sqrt(sum x^2 + eps), eps = 1e-6.
  * decay: g = log alpha = -scale[c] * softplus(x) (alpha in (0, 1]); the workloads draw
    exactly this form with scale 0.1 and x ~ N(0, 1).
  * erase and write gates: b = b_max * sigmoid(x), w = sigmoid(x); b_max = 1 nominally, 2 for
    the widened-range ablation of [note §4].
  * RMSNorm over d_v per (token, head): o / sqrt(mean(o^2) + eps) * weight[c], eps = 1e-6;
    the output gate is SiLU(gate) with the gate from its own projection.
"""
from __future__ import annotations

import numpy as np

__all__ = ["causal_conv", "silu", "l2norm", "softplus", "sigmoid", "prologue", "epilogue",
           "CONV_WIDTH", "EPS"]

CONV_WIDTH = 4
EPS = 1e-6


def sigmoid(x):
    x = np.asarray(x, np.float64)
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))), np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))


def softplus(x):
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def causal_conv(x, weight, cu_seqlens=None):
    """x: [B, T, C]; weight: [C, CONV_WIDTH]. Causal depthwise conv per sequence."""
    x = np.asarray(x, np.float64)
    weight = np.asarray(weight, np.float64)
    B, T, C = x.shape
    if cu_seqlens is None:
        bounds = [(bi, 0, T) for bi in range(B)]
    else:
        cu = [int(v) for v in np.asarray(cu_seqlens)]
        bounds = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    y = np.zeros_like(x)
    for bi, t0, t1 in bounds:
        for t in range(t0, t1):
            for j in range(CONV_WIDTH):
                s = t - (CONV_WIDTH - 1) + j
                if s >= t0:
                    y[bi, t] += weight[:, j] * x[bi, s]
    return y


def l2norm(x, axis=-1):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=axis, keepdims=True) + EPS)


def prologue(xq, xk, xv, xg, xb, xw, wq, wk, wv, decay_scale, b_max=1.0, cu_seqlens=None):
    """Projected branches -> mixer inputs.

    xq, xk, xg, xb: [B, T, H, d_k]; xv, xw: [B, T, H, d_v] (pre-activation projections);
    wq, wk: [H * d_k, CONV_WIDTH]; wv: [H * d_v, CONV_WIDTH]; decay_scale: [H * d_k] (> 0).
    Returns q, k, v, g, b, w with the mixer's shapes (float64).
    """
    B, T, H, dk = np.shape(xq)
    dv = np.shape(xv)[-1]

    def conv(x, wgt, d):
        return causal_conv(np.reshape(x, (B, T, H * d)), wgt, cu_seqlens).reshape(B, T, H, d)
    q = l2norm(silu(conv(xq, wq, dk)))
    k = l2norm(silu(conv(xk, wk, dk)))
    v = silu(conv(xv, wv, dv))
    g = -np.reshape(np.asarray(decay_scale, np.float64), (H, dk)) * softplus(xg)
    b = b_max * sigmoid(xb)
    w = sigmoid(xw)
    return q, k, v, g, b, w


def epilogue(o, gate, weight):
    """o, gate: [B, T, H, d_v]; weight: [d_v]. RMSNorm(o) * weight * SiLU(gate)."""
    o = np.asarray(o, np.float64)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + EPS)
    return r * np.asarray(weight, np.float64) * silu(gate)
