"""GPU parity of the training pair: gdn2_chunk_fwd_train (forward that keeps the backward's
intermediates) and gdn2_chunk_bwd_saved (backward that reuses them), through the C ABI, and
of the autograd wrapper, against the float64 oracle's forward and reverse loop."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_inputs, round_to_bf16
from oracle import gdn2_backward, gdn2_forward
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, rel_err, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "b", "w")
GRADS = ("dq", "dk", "dv", "dg", "db", "dw", "ds0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(dk, dv, lens=None, seed=0):
    if lens is None:
        x = make_inputs(2, 150, 2, dk, dv, "bf16", seed=seed, s0_std=0.02)
    else:
        x = make_inputs(1, int(sum(lens)), 2, dk, dv, "bf16", seed=seed, lengths=lens, s0_std=0.02)
    rng = np.random.default_rng(seed + 1)
    B, T, H, _ = x["q"].shape
    N = x["s0"].shape[0]
    do = round_to_bf16(rng.normal(size=(B, T, H, dv)).astype(np.float32))
    dsn = (rng.normal(size=(N, H, dk, dv)) * 0.1).astype(np.float32)
    return x, do, dsn


def _dev(x):
    t = {n: dev_tensor(x[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    return t, s0, cu


@pytest.mark.parametrize("dk,dv,lens", [(128, 128, None), (64, 128, None), (128, 64, [1, 64, 0, 130, 37])])
def test_train_forward_and_saved_backward(dk, dv, lens):
    import gated_delta_rule_36_amd as G
    x, do, dsn = _case(dk, dv, lens, seed=dk + dv)
    say("train pair", dk, dv, lens)
    t, s0, cu = _dev(x)
    o, sN, saved = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0, cu_seqlens=cu)
    torch.cuda.synchronize()
    o_ref, s_ref = gdn2_forward(*(x[n] for n in NAMES), s0=x["s0"], cu_seqlens=x["cu_seqlens"])
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])
    do_t, dsn_t = dev_tensor(do, "bf16"), torch.from_numpy(dsn).cuda()
    g_saved = G.chunk_bwd(*(t[n] for n in NAMES), do_t, initial_state=s0, d_final_state=dsn_t,
                          cu_seqlens=cu, saved=saved)
    g_full = G.chunk_bwd(*(t[n] for n in NAMES), do_t, initial_state=s0, d_final_state=dsn_t,
                         cu_seqlens=cu)
    torch.cuda.synchronize()
    ref = gdn2_backward(*(x[n] for n in NAMES), do, dS_final=dsn, s0=x["s0"],
                        cu_seqlens=x["cu_seqlens"])
    for name, a, b_, r in zip(GRADS, g_saved, g_full, ref):
        assert_close(name, host64(a), r, TOL["bf16"])
        # the same kernels store the same intermediates either way
        assert rel_err(host64(a), host64(b_)) <= 1e-3, name


def test_saved_from_other_tensors_is_rejected():
    import gated_delta_rule_36_amd as G
    x, do, dsn = _case(128, 128, seed=3)
    t, s0, cu = _dev(x)
    say("train pair mismatch guard")
    _, _, saved = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0)
    other = t["q"].clone()
    with pytest.raises(ValueError):
        G.chunk_bwd(other, *(t[n] for n in NAMES[1:]), dev_tensor(do, "bf16"), initial_state=s0,
                    saved=saved)
    torch.cuda.synchronize()


def test_autograd_wrapper():
    import gated_delta_rule_36_amd as G
    x, do, dsn = _case(128, 128, seed=5)
    say("autograd wrapper")
    t, s0, _ = _dev(x)
    leaves = {n: t[n].clone().requires_grad_(True) for n in NAMES}
    s0l = s0.clone().requires_grad_(True)
    o, sN = G.gated_delta_rule2(*(leaves[n] for n in NAMES), initial_state=s0l)
    loss = (o.float() * dev_tensor(do, "bf16").float()).sum() + (sN * torch.from_numpy(dsn).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = gdn2_backward(*(x[n] for n in NAMES), do, dS_final=dsn, s0=x["s0"])
    for name, n, r in zip(GRADS, NAMES, ref):
        assert_close(name, host64(leaves[n].grad), r, TOL["bf16"])
    assert_close("ds0", host64(s0l.grad), ref[6], TOL["bf16"])
