"""Pins of the block prologue / epilogue oracle (oracle/gdn2_block.py) against library
routines and closed forms."""
import numpy as np

from oracle import gdn2_block as BK


def test_activations_closed_forms():
    assert BK.sigmoid(0.0) == 0.5
    assert np.isclose(BK.softplus(0.0), np.log(2.0), rtol=0, atol=1e-15)
    x = np.linspace(-40, 40, 161)
    assert np.allclose(BK.softplus(x), np.log1p(np.exp(x)), rtol=1e-12, atol=1e-300)
    assert np.allclose(BK.sigmoid(x), 1.0 / (1.0 + np.exp(-x)), rtol=1e-12, atol=1e-300)
    xs = np.linspace(-5, 5, 21)  # the tanh identity, where it has no cancellation
    assert np.allclose(BK.sigmoid(xs), 0.5 * (1 + np.tanh(xs / 2)), rtol=1e-12)
    assert np.allclose(BK.silu(x), x / (1 + np.exp(-x)), rtol=1e-12, atol=1e-300)


def test_causal_conv_matches_numpy_convolve():
    rng = np.random.default_rng(1)
    B, T, C = 2, 11, 5
    x = rng.normal(size=(B, T, C))
    w = rng.normal(size=(C, BK.CONV_WIDTH))
    y = BK.causal_conv(x, w)
    for bi in range(B):
        for c in range(C):
            # causal: y[t] = sum_j w[j] x[t - 3 + j]  ==  full convolution with reversed taps
            ref = np.convolve(x[bi, :, c], w[c, ::-1], mode="full")[:T]
            assert np.allclose(y[bi, :, c], ref, rtol=0, atol=1e-12)


def test_causal_conv_respects_sequence_boundaries():
    rng = np.random.default_rng(2)
    lens = [3, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.normal(size=(1, sum(lens), 4))
    w = rng.normal(size=(4, BK.CONV_WIDTH))
    y = BK.causal_conv(x, w, cu_seqlens=cu)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        assert np.allclose(y[:, sl], BK.causal_conv(x[:, sl], w), rtol=0, atol=1e-14)


def test_l2norm_and_rmsnorm():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(7, 16))
    n = BK.l2norm(x)
    assert np.allclose(np.sum(n * n, axis=-1), 1.0, atol=1e-6)
    # RMSNorm of a constant row is sign * weight (up to eps); silu(gate) = 1/2 * gate at 0 slope
    o = np.full((1, 1, 1, 8), -3.0)
    gate = np.full((1, 1, 1, 8), 50.0)  # silu(50) = 50 to double precision
    wgt = np.arange(1, 9, dtype=np.float64)
    y = BK.epilogue(o, gate, wgt)
    assert np.allclose(y[0, 0, 0], -wgt * 50.0, rtol=1e-6)


def test_prologue_gate_ranges_and_shapes():
    rng = np.random.default_rng(4)
    B, T, H, dk, dv = 1, 9, 2, 8, 4
    xs = [rng.normal(size=(B, T, H, d)) * 3 for d in (dk, dk, dv, dk, dk, dv)]
    wq = rng.normal(size=(H * dk, 4))
    wk = rng.normal(size=(H * dk, 4))
    wv = rng.normal(size=(H * dv, 4))
    scale = rng.uniform(0.05, 0.5, size=H * dk)
    q, k, v, g, b, w = BK.prologue(*xs, wq, wk, wv, scale, b_max=2.0)
    assert np.allclose(np.sum(q * q, -1), 1.0, atol=1e-5) and np.allclose(np.sum(k * k, -1), 1.0, atol=1e-5)
    assert np.all(g <= 0) and np.all(b >= 0) and np.all(b <= 2) and np.all((w >= 0) & (w <= 1))
    # g = -scale * softplus(x) element by element
    assert np.allclose(g, -scale.reshape(H, dk) * np.log1p(np.exp(xs[3])), rtol=1e-12)
    assert v.shape == (B, T, H, dv)


# ------------------------------------------------------------------------------------------
# Element-by-element pins of the prologue's composition and the epilogue's normalisation
# axis. The reference below is written per (token, head, channel) with plain loops and
# math.exp, in the order the reading note's block paragraph gives (§3: linear -> conv ->
# SiLU -> L2 norm for q and k; linear -> conv -> SiLU for v; separate gate branches), and
# per (token, head) for the gated RMSNorm over the d_v channels of that head. The pins take
# the function under test as an argument; planted mistakes in copies must each fail.
import math  # noqa: E402

import pytest  # noqa: E402


def _ref_branch(x, taps, t0, t, h, c, d):
    """conv then SiLU for token t of a sequence starting at t0, head h, channel c."""
    y = 0.0
    for j in range(BK.CONV_WIDTH):
        s = t - (BK.CONV_WIDTH - 1) + j
        if s >= t0:
            y += taps[h * d + c, j] * x[0, s, h, c]
    return y / (1.0 + math.exp(-y))


def _ref_prologue(xq, xk, xv, xg, xb, xw, wq, wk, wv, scale, b_max, cu):
    _, T, H, dk = xq.shape
    dv = xv.shape[-1]
    out = {n: np.zeros(a.shape) for n, a in zip("qkvgbw", (xq, xk, xv, xg, xb, xw))}
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1]):
            for h in range(H):
                for name, x, taps, d in (("q", xq, wq, dk), ("k", xk, wk, dk)):
                    s = [_ref_branch(x, taps, cu[n], t, h, c, d) for c in range(d)]
                    nrm = math.sqrt(sum(v * v for v in s) + BK.EPS)
                    for c in range(d):
                        out[name][0, t, h, c] = s[c] / nrm
                for c in range(dv):
                    out["v"][0, t, h, c] = _ref_branch(xv, wv, cu[n], t, h, c, dv)
                    out["w"][0, t, h, c] = 1.0 / (1.0 + math.exp(-xw[0, t, h, c]))
                for c in range(dk):
                    out["g"][0, t, h, c] = -scale[h * dk + c] * math.log1p(math.exp(xg[0, t, h, c]))
                    out["b"][0, t, h, c] = b_max / (1.0 + math.exp(-xb[0, t, h, c]))
    return [out[n] for n in "qkvgbw"]


def _prologue_case(seed=31):
    rng = np.random.default_rng(seed)
    H, dk, dv = 3, 5, 4
    lens = [6, 2, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    # per-head magnitudes differ, so a norm over the wrong axis changes the result
    hs = np.array([0.3, 1.0, 4.0])[None, None, :, None]
    xs = [rng.normal(size=(1, T, H, d)) * hs for d in (dk, dk, dv, dk, dk, dv)]
    wq = rng.normal(size=(H * dk, 4))
    wk = rng.normal(size=(H * dk, 4))
    wv = rng.normal(size=(H * dv, 4))
    scale = rng.uniform(0.05, 0.5, size=H * dk)
    return xs, wq, wk, wv, scale, cu


def pin_prologue(fn):
    xs, wq, wk, wv, scale, cu = _prologue_case()
    got = fn(*xs, wq, wk, wv, scale, b_max=2.0, cu_seqlens=cu)
    ref = _ref_prologue(*xs, wq, wk, wv, scale, 2.0, cu)
    for name, a, r in zip("qkvgbw", got, ref):
        assert a.shape == r.shape, name
        assert np.allclose(a, r, rtol=0, atol=1e-12), f"prologue branch {name}"


def _ref_epilogue(o, gate, weight):
    B, T, H, dv = o.shape
    y = np.zeros(o.shape)
    for bi in range(B):
        for t in range(T):
            for h in range(H):
                ms = sum(o[bi, t, h, c] ** 2 for c in range(dv)) / dv
                inv = 1.0 / math.sqrt(ms + BK.EPS)
                for c in range(dv):
                    gt = gate[bi, t, h, c]
                    y[bi, t, h, c] = o[bi, t, h, c] * inv * weight[c] * gt / (1.0 + math.exp(-gt))
    return y


def pin_epilogue(fn):
    rng = np.random.default_rng(32)
    B, T, H, dv = 2, 3, 3, 6
    o = rng.normal(size=(B, T, H, dv)) * np.array([0.01, 1.0, 30.0])[None, None, :, None]
    gate = rng.normal(size=(B, T, H, dv)) * 2
    weight = 1 + 0.3 * rng.normal(size=dv)
    assert np.allclose(fn(o, gate, weight), _ref_epilogue(o, gate, weight), rtol=1e-12, atol=1e-13)


def test_prologue_elementwise():
    pin_prologue(BK.prologue)


def test_epilogue_elementwise():
    pin_epilogue(BK.epilogue)


def _prologue_mutant(kind):
    def fn(xq, xk, xv, xg, xb, xw, wq, wk, wv, decay_scale, b_max=1.0, cu_seqlens=None):
        B, T, H, dk = np.shape(xq)
        dv = np.shape(xv)[-1]
        cu = None if kind == "conv_crosses_sequences" else cu_seqlens

        def conv(x, wgt, d):
            if kind == "taps_reversed":
                wgt = wgt[:, ::-1]
            return BK.causal_conv(np.reshape(x, (B, T, H * d)), wgt, cu).reshape(B, T, H, d)

        def branch(x, wgt, d):
            if kind == "silu_before_conv":
                return conv(BK.silu(x), wgt, d)
            return BK.silu(conv(x, wgt, d))

        def norm(x):
            if kind == "l2_over_heads":
                return BK.l2norm(x.reshape(B, T, -1)).reshape(x.shape)
            return BK.l2norm(x)
        q = norm(branch(xq, wq, dk))
        k = norm(branch(xk, wk, dk))
        v = branch(xv, wv, dv)
        if kind == "v_normalised":
            v = BK.l2norm(v)
        sc = np.reshape(np.asarray(decay_scale, np.float64), (H, dk))
        if kind == "scale_head_major_swapped":
            sc = np.reshape(np.asarray(decay_scale, np.float64), (dk, H)).T
        g = -sc * BK.softplus(xg)
        b = (1.0 if kind == "b_max_dropped" else b_max) * BK.sigmoid(xb)
        w = BK.sigmoid(xw)
        return q, k, v, g, b, w
    return fn


def _epilogue_mutant(kind):
    def fn(o, gate, weight):
        o = np.asarray(o, np.float64)
        if kind == "rms_over_heads":
            ms = np.mean((o * o).reshape(o.shape[:-2] + (-1,)), axis=-1)[..., None, None]
        elif kind == "rms_sum_not_mean":
            ms = np.sum(o * o, axis=-1, keepdims=True)
        else:
            ms = np.mean(o * o, axis=-1, keepdims=True)
        r = o / np.sqrt(ms + BK.EPS)
        gt = BK.sigmoid(gate) if kind == "sigmoid_gate" else BK.silu(gate)
        wt = 1.0 if kind == "weight_dropped" else np.asarray(weight, np.float64)
        return r * wt * gt
    return fn


PROLOGUE_MUTANTS = ["silu_before_conv", "l2_over_heads", "taps_reversed", "v_normalised",
                    "conv_crosses_sequences", "scale_head_major_swapped", "b_max_dropped"]
EPILOGUE_MUTANTS = ["rms_over_heads", "rms_sum_not_mean", "sigmoid_gate", "weight_dropped"]


@pytest.mark.parametrize("kind", PROLOGUE_MUTANTS)
def test_planted_prologue_mistakes_are_caught(kind):
    with pytest.raises(AssertionError):
        pin_prologue(_prologue_mutant(kind))


@pytest.mark.parametrize("kind", EPILOGUE_MUTANTS)
def test_planted_epilogue_mistakes_are_caught(kind):
    with pytest.raises(AssertionError):
        pin_epilogue(_epilogue_mutant(kind))


def test_unmutated_block_copies_pass():
    pin_prologue(_prologue_mutant("none"))
    pin_epilogue(_epilogue_mutant("none"))
