"""GPU parity of the scalar-gate layouts (one erase and / or write gate value per token and
head, shared by its channels: the scalar-gate configurations of the GDN-2 reading note's §4)
through gdn2_chunk_fwd_ex, gdn2_decode_step_ex and gdn2_decode_tokens_ex, against the oracle
run on the same gate broadcast over the channels."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_decode_inputs, make_inputs, make_scalar_gate, varlen_lengths
from oracle import gdn2_decode_steps, gdn2_decode_tokens, gdn2_forward
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "b", "w")
LAYOUTS = {"b": (True, False), "w": (False, True), "bw": (True, True)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _scalarise(x, layout, lead, seed):
    """Replace b and / or w by scalar gates; returns (gates for the GPU, broadcast for the
    oracle)."""
    sb, sw = LAYOUTS[layout]
    gpu = dict(x)
    ref = dict(x)
    for name, on, d in (("b", sb, x["q"].shape[-1]), ("w", sw, x["v"].shape[-1])):
        if on:
            s = make_scalar_gate(lead, x.get("dtype", "bf16"), seed=seed + (name == "w"))
            gpu[name] = s
            ref[name] = np.repeat(s[..., None], d, axis=-1)
    return gpu, ref


@pytest.mark.parametrize("layout", ["b", "w", "bw"])
@pytest.mark.parametrize("dt,dk,dv,path", [("bf16", 128, 128, "fused"), ("bf16", 64, 128, "fused"),
                                           ("fp32", 64, 64, "fused"), ("fp32", 128, 64, "fused"),
                                           ("bf16", 128, 64, "split"),
                                           ("bf16", 128, 128, "split")])
def test_chunk_forward_scalar_gates(layout, dt, dk, dv, path):
    import gated_delta_rule_36_amd as G
    B, T, H = 2, 200, 3
    x = make_inputs(B, T, H, dk, dv, dt, seed=41 + dk + dv, s0_std=0.05)
    gx, rx = _scalarise(x, layout, (B, T, H), seed=7)
    say("chunk_fwd scalar gates", layout, dt, dk, dv, path)
    t = {n: dev_tensor(gx[n], dt) for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, sN = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0, path=path)
    torch.cuda.synchronize()
    o_ref, s_ref = gdn2_forward(*(rx[n] for n in NAMES), s0=x["s0"])
    assert_close("o", host64(o), o_ref, TOL[dt])
    assert_close("S_final", host64(sN), s_ref, TOL[dt])


@pytest.mark.parametrize("path", ["fused", "split"])
def test_chunk_forward_scalar_gates_varlen(path):
    import gated_delta_rule_36_amd as G
    lens = varlen_lengths(5, 1, 150, seed=3)
    lens[1] = 64
    T = int(np.sum(lens))
    x = make_inputs(1, T, 2, 128, 128, "bf16", seed=5, lengths=lens, s0_std=0.05)
    gx, rx = _scalarise(x, "bw", (1, T, 2), seed=9)
    say("chunk_fwd scalar gates varlen", path, list(map(int, lens)))
    t = {n: dev_tensor(gx[n], "bf16") for n in NAMES}
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    o, sN = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=torch.from_numpy(x["s0"]).cuda(),
                        cu_seqlens=cu, path=path)
    torch.cuda.synchronize()
    o_ref, s_ref = gdn2_forward(*(rx[n] for n in NAMES), s0=x["s0"], cu_seqlens=x["cu_seqlens"])
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])


@pytest.mark.parametrize("layout", ["b", "w", "bw"])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_decode_step_scalar_gates(layout, dt):
    import gated_delta_rule_36_amd as G
    N, H, dk, dv, steps = 5, 3, 128, 64, 4
    x = make_decode_inputs(N, H, dk, dv, steps, dt, seed=13, s0_std=0.05)
    # [steps, N, H, d] per-step inputs; scalar gates are [steps, N, H]
    gx, rx = _scalarise(x, layout, (steps, N, H), seed=17)
    say("decode_step scalar gates", layout, dt)
    st = torch.from_numpy(x["s0"]).cuda()
    outs = []
    for s in range(steps):
        outs.append(G.decode_step(*(dev_tensor(gx[n][s], dt) for n in NAMES), st))
    torch.cuda.synchronize()
    o_ref, s_ref = gdn2_decode_steps(x["s0"], *(rx[n] for n in NAMES))
    assert_close("o", host64(torch.stack(outs)), o_ref, TOL[dt])
    assert_close("state", host64(st), s_ref, TOL[dt])


@pytest.mark.parametrize("layout", ["b", "w", "bw"])
def test_decode_tokens_scalar_gates(layout):
    import gated_delta_rule_36_amd as G
    N, L, H, dk, dv, P = 4, 3, 2, 64, 128, 6
    x = make_decode_inputs(N, H, dk, dv, L, "bf16", seed=19, s0_std=0.05)
    toks = {n: np.ascontiguousarray(np.swapaxes(x[n], 0, 1)) for n in NAMES}  # [N, L, H, d]
    toks["dtype"] = "bf16"
    gx, rx = _scalarise(toks, layout, (N, L, H), seed=23)
    rng = np.random.default_rng(3)
    pool = (rng.normal(size=(P, H, dk, dv)) * 0.05).astype(np.float32)
    idx = np.array([4, 0, 2, 5], np.int32)
    say("decode_tokens scalar gates", layout)
    pool_t = torch.from_numpy(pool).cuda()
    o, _ = G.decode_tokens(*(dev_tensor(gx[n], "bf16") for n in NAMES), pool_t,
                           state_indices=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    o_ref, _, pool_ref = gdn2_decode_tokens(pool, *(rx[n] for n in NAMES), indices=idx)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("pool", host64(pool_t), pool_ref, TOL["bf16"])


@pytest.mark.parametrize("T", [150, 1100])
@pytest.mark.parametrize("layout", ["b", "w", "bw"])
@pytest.mark.parametrize("saved", [False, True])
def test_backward_scalar_gates(layout, saved, T):
    """Gradients with scalar gates: a shared gate's gradient is the channel sum of the
    oracle's per-channel gradient of the broadcast gate; through the recomputing backward
    and through the training forward / saved backward pair. At 1100 tokens (18 chunks, four
    chains) both passes cut each sequence into segments."""
    import gated_delta_rule_36_amd as G
    from gdn2_inputs import round_to_bf16
    from oracle import gdn2_backward
    B, H, dk, dv = 2, 2, 128, 64
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=61, s0_std=0.02)
    gx, rx = _scalarise(x, layout, (B, T, H), seed=63)
    rng = np.random.default_rng(65)
    do = round_to_bf16(rng.normal(size=(B, T, H, dv)).astype(np.float32))
    dsn = (rng.normal(size=(B, H, dk, dv)) * 0.1).astype(np.float32)
    say("backward scalar gates", layout, "saved" if saved else "recompute", "T", T)
    t = {n: dev_tensor(gx[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    do_t, dsn_t = dev_tensor(do, "bf16"), torch.from_numpy(dsn).cuda()
    sv = None
    if saved:
        o, sN, sv = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0)
        torch.cuda.synchronize()
        o_ref, s_ref = gdn2_forward(*(rx[n] for n in NAMES), s0=x["s0"])
        assert_close("o", host64(o), o_ref, TOL["bf16"])
        assert_close("S_final", host64(sN), s_ref, TOL["bf16"])
    grads = G.chunk_bwd(*(t[n] for n in NAMES), do_t, initial_state=s0, d_final_state=dsn_t,
                        saved=sv)
    torch.cuda.synchronize()
    ref = list(gdn2_backward(*(rx[n] for n in NAMES), do, dS_final=dsn, s0=x["s0"]))
    sb, sw = LAYOUTS[layout]
    if sb:
        ref[4] = ref[4].sum(-1)
    if sw:
        ref[5] = ref[5].sum(-1)
    for name, a, r in zip(("dq", "dk", "dv", "dg", "db", "dw", "ds0"), grads, ref):
        assert tuple(a.shape) == r.shape, name
        assert_close(name, host64(a), r, TOL["bf16"])


@pytest.mark.parametrize("strong_decay", [False, True])
def test_backward_scalar_gates_varlen(strong_decay):
    """Packed sequences with both gates scalar; with strong_decay, g = -6 on 70 tokens that
    span the fourth sequence's first chunk (past the local-gradient kernel's factor range,
    so its gradients come from the exact kernel and its scalar-b channel sums)."""
    import gated_delta_rule_36_amd as G
    from gdn2_inputs import round_to_bf16
    from oracle import gdn2_backward
    lens = [1, 64, 0, 100, 33]
    T = sum(lens)
    x = make_inputs(1, T, 2, 64, 128, "bf16", seed=71, lengths=lens, s0_std=0.02)
    if strong_decay:
        x["g"][:, 65:135] = -6.0
    gx, rx = _scalarise(x, "bw", (1, T, 2), seed=73)
    rng = np.random.default_rng(75)
    do = round_to_bf16(rng.normal(size=(1, T, 2, 128)).astype(np.float32))
    say("backward scalar gates varlen", lens)
    t = {n: dev_tensor(gx[n], "bf16") for n in NAMES}
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    grads = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(do, "bf16"),
                        initial_state=torch.from_numpy(x["s0"]).cuda(), cu_seqlens=cu)
    torch.cuda.synchronize()
    ref = list(gdn2_backward(*(rx[n] for n in NAMES), do, s0=x["s0"], cu_seqlens=x["cu_seqlens"]))
    ref[4] = ref[4].sum(-1)
    ref[5] = ref[5].sum(-1)
    for name, a, r in zip(("dq", "dk", "dv", "dg", "db", "dw", "ds0"), grads, ref):
        assert_close(name, host64(a), r, TOL["bf16"])


def test_backward_scalar_gates_many_units_sampled():
    """Scalar b and w through the saved backward with 1024 (chunk, head) units, more than one
    per workgroup of the persistent local-gradient kernel (its cross-wave db sum runs once
    per unit); sampled chains of the later iterations against the oracle."""
    import gated_delta_rule_36_amd as G
    from gdn2_inputs import round_to_bf16
    from oracle import gdn2_backward
    B, T, H, dk, dv = 4, 1000, 16, 128, 128
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=81, s0_std=0.02)
    gx, rx = _scalarise(x, "bw", (B, T, H), seed=83)
    rng = np.random.default_rng(85)
    do = round_to_bf16(rng.normal(size=(B, T, H, dv)).astype(np.float32))
    say("backward scalar gates many units B4 T1000 H16 (sampled chains)")
    t = {n: dev_tensor(gx[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, sN, sv = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0)
    grads = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(do, "bf16"), initial_state=s0, saved=sv)
    torch.cuda.synchronize()
    for (n, h) in [(3, 11), (2, 0)]:
        sel = {m: rx[m][n:n + 1, :, h:h + 1] for m in NAMES}
        ref = list(gdn2_backward(*(sel[m] for m in NAMES), do[n:n + 1, :, h:h + 1],
                                 s0=x["s0"][n:n + 1, h:h + 1]))
        ref[4] = ref[4].sum(-1)
        ref[5] = ref[5].sum(-1)
        print(f" chain (n={n}, h={h})", flush=True)
        for name, a, r in zip(("dq", "dk", "dv", "dg", "db", "dw"), grads[:6], ref[:6]):
            assert_close(name, host64(a[n:n + 1, :, h:h + 1]), r, TOL["bf16"])
        assert_close("ds0", host64(grads[6][n:n + 1, h:h + 1]), ref[6], TOL["bf16"])


@pytest.mark.parametrize("layout", ["b", "bw"])
def test_chunk_forward_scalar_gates_segments(layout):
    """The two-phase forward with scalar gates at a length it cuts into segments (1100
    tokens: 18 chunks, six chains of 64 value columns), against the token loop."""
    import gated_delta_rule_36_amd as G
    B, T, H = 1, 1100, 3
    x = make_inputs(B, T, H, 128, 128, "bf16", seed=43, s0_std=0.05, reset_frac=0.05)
    gx, rx = _scalarise(x, layout, (B, T, H), seed=11)
    say("chunk_fwd scalar gates, segments", layout)
    t = {n: dev_tensor(gx[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, sN = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0, path="split")
    torch.cuda.synchronize()
    o_ref, s_ref = gdn2_forward(*(rx[n] for n in NAMES), s0=x["s0"])
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])
