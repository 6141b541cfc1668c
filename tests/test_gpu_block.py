"""GPU parity of the block prologue and epilogue (gdn2_block_prologue / gdn2_block_epilogue,
through the C ABI) with the oracle's block_prologue / block_epilogue: fixed-length and varlen
batches, both dtypes, every head width, and the widened erase-gate range (b_max = 2)."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_block_inputs, varlen_lengths
from oracle import block_epilogue as ref_epilogue
from oracle import block_prologue as ref_prologue
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu
PROJ = ("xq", "xk", "xv", "xg", "xb", "xw")
OUTS = ("q", "k", "v", "g", "b", "w")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def _run_prologue(x, dt, b_max):
    import gated_delta_rule_36_amd as G
    t = {n: dev_tensor(x[n], dt) for n in PROJ}
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    got = G.block_prologue(*(t[n] for n in PROJ), _f32(x["conv_q"]), _f32(x["conv_k"]),
                           _f32(x["conv_v"]), _f32(x["decay_scale"]), b_max=b_max,
                           cu_seqlens=cu)
    torch.cuda.synchronize()
    ref = ref_prologue(*(x[n] for n in PROJ), x["conv_q"], x["conv_k"], x["conv_v"],
                       x["decay_scale"], b_max=b_max, cu_seqlens=x["cu_seqlens"])
    return got, ref


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_prologue_fixed_length(dt, dk, dv):
    B, T, H = 2, 37, 3
    x = make_block_inputs(B, T, H, dk, dv, dt, seed=dk + 3 * dv + (dt == "bf16"))
    say("block_prologue", dt, dk, dv, f"B{B} T{T} H{H}")
    got, ref = _run_prologue(x, dt, 1.0)
    for n, g_, r_ in zip(OUTS, got, ref):
        assert g_.shape == r_.shape
        assert_close(n, host64(g_), r_, TOL[dt])


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_prologue_varlen_and_wide_erase_range(dt):
    lens = varlen_lengths(9, 1, 40, seed=5)
    lens[2] = 1  # shorter than the conv width
    lens[3] = 2
    T = int(np.sum(lens))
    x = make_block_inputs(1, T, 4, 128, 128, dt, seed=17, lengths=lens)
    say("block_prologue varlen", dt, "lens", list(map(int, lens)))
    got, ref = _run_prologue(x, dt, 2.0)
    for n, g_, r_ in zip(OUTS, got, ref):
        assert_close(n, host64(g_), r_, TOL[dt])
    b = host64(got[4])
    assert b.max() > 1.0 and b.max() <= 2.0  # the widened range is reached, never exceeded


def test_prologue_rows_are_unit_norm_and_gates_in_range():
    x = make_block_inputs(1, 300, 8, 128, 128, "fp32", seed=23)
    say("block_prologue invariants", "T300 H8")
    got, _ = _run_prologue(x, "fp32", 1.0)
    q, k, v, g, b, w = (host64(t) for t in got)
    for y in (q, k):  # ||silu(conv(x))||^2 >> eps here, so rows are unit norm to fp32 rounding
        assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-5)
    assert np.all(g <= 0) and np.all(b >= 0) and np.all(b <= 1) and np.all(w >= 0)
    assert np.all(w <= 1)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("dv", [64, 128])
def test_epilogue(dt, dv):
    import gated_delta_rule_36_amd as G
    x = make_block_inputs(3, 29, 5, 64, dv, dt, seed=dv + (dt == "bf16"))
    say("block_epilogue", dt, dv, "B3 T29 H5")
    y = G.block_epilogue(dev_tensor(x["o"], dt), dev_tensor(x["gate"], dt), _f32(x["norm_weight"]))
    torch.cuda.synchronize()
    ref = ref_epilogue(x["o"], x["gate"], x["norm_weight"])
    assert_close("y", host64(y), ref, TOL[dt])


def test_full_size_prologue_epilogue_sampled():
    """The benchmark's shape (B 8, T 2048, H 16, 128/128, bf16): sampled rows against the
    oracle; the oracle runs on a window of tokens around each sampled row."""
    import gated_delta_rule_36_amd as G
    B, T, H, d = 8, 2048, 16, 128
    x = make_block_inputs(B, T, H, d, d, "bf16", seed=31)
    say("block_prologue/epilogue full size", "B8 T2048 H16 128/128 bf16")
    t = {n: dev_tensor(x[n], "bf16") for n in PROJ}
    got = G.block_prologue(*(t[n] for n in PROJ), _f32(x["conv_q"]), _f32(x["conv_k"]),
                           _f32(x["conv_v"]), _f32(x["decay_scale"]))
    y = G.block_epilogue(dev_tensor(x["o"], "bf16"), dev_tensor(x["gate"], "bf16"),
                         _f32(x["norm_weight"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    picks = [(0, 0), (0, 2), (B - 1, T - 1)] + [(int(rng.integers(B)), int(rng.integers(T)))
                                                for _ in range(6)]
    for bi, ti in picks:
        t0 = max(0, ti - 3)  # the conv reaches 3 tokens back; a window from t0 is exact at ti
        win = {n: x[n][bi:bi + 1, t0:ti + 1] for n in PROJ}
        ref = ref_prologue(*(win[n] for n in PROJ), x["conv_q"], x["conv_k"], x["conv_v"],
                           x["decay_scale"])
        for n, g_, r_ in zip(OUTS, got, ref):
            assert_close(f"{n}[{bi},{ti}]", host64(g_[bi, ti]), r_[0, -1], TOL["bf16"])
    ry = ref_epilogue(x["o"][:, ::97], x["gate"][:, ::97], x["norm_weight"])
    assert_close("y sampled", host64(y[:, ::97]), ry, TOL["bf16"])


def test_preallocated_outputs():
    """out= writes the same values into the caller's tensors as the allocating calls."""
    import gated_delta_rule_36_amd as G
    x = make_block_inputs(2, 70, 3, 128, 64, "bf16", seed=77)
    say("block out= B2 T70 H3 dk128 dv64")
    t = {n: dev_tensor(x[n], "bf16") for n in PROJ}
    args = [t[n] for n in PROJ] + [_f32(x["conv_q"]), _f32(x["conv_k"]), _f32(x["conv_v"]),
                                   _f32(x["decay_scale"])]
    ref = G.block_prologue(*args, b_max=1.5)
    out = [torch.full_like(r, float("nan")) for r in ref]
    got = G.block_prologue(*args, b_max=1.5, out=out)
    o, gate = dev_tensor(x["o"], "bf16"), dev_tensor(x["gate"], "bf16")
    y_ref = G.block_epilogue(o, gate, _f32(x["norm_weight"]))
    y = torch.full_like(y_ref, float("nan"))
    y_got = G.block_epilogue(o, gate, _f32(x["norm_weight"]), out=y)
    torch.cuda.synchronize()
    assert all(g is o_ for g, o_ in zip(got, out)) and y_got is y
    for name, a, b in zip(OUTS, got, ref):
        assert torch.equal(a, b), name
    assert torch.equal(y, y_ref)
    with pytest.raises(ValueError):
        G.block_prologue(*args, out=out[:5])
    with pytest.raises(ValueError):
        G.block_epilogue(o, gate, _f32(x["norm_weight"]), out=y[:1])
