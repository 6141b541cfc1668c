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
