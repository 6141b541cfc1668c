"""GPU parity of the chunkwise backward (through the C ABI) against the oracle's reverse token
loop (float64). Tolerance: normwise max relative error 2e-2 per gradient (bf16 runs)."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_inputs, round_to_bf16
from oracle import gdn2_backward
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")
GRADS = ("dq", "dk", "dv", "dg", "db", "dw")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _upstream(x, seed, with_dsn=True):
    rng = np.random.default_rng(seed)
    B, T, H, _ = x["q"].shape
    dv = x["v"].shape[-1]
    dk = x["q"].shape[-1]
    N = B if x["cu_seqlens"] is None else len(x["cu_seqlens"]) - 1
    do = round_to_bf16(rng.normal(size=(B, T, H, dv)).astype(np.float32))
    dsn = rng.normal(size=(N, H, dk, dv)).astype(np.float32) * 0.1 if with_dsn else None
    return do, dsn


def run_bwd(x, do, dsn):
    import gated_delta_rule_36_amd as G
    t = {n: dev_tensor(x[n], "bf16") for n in NAMES}
    s0 = None if x["s0"] is None else torch.from_numpy(x["s0"]).cuda()
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    dsn_t = None if dsn is None else torch.from_numpy(dsn).cuda()
    out = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(do, "bf16"), initial_state=s0,
                      d_final_state=dsn_t, cu_seqlens=cu)
    torch.cuda.synchronize()
    return out


def check(x, do, dsn, tol=TOL["bf16"]):
    out = run_bwd(x, do, dsn)
    ref = gdn2_backward(*(x[n] for n in NAMES), do, dS_final=dsn, s0=x["s0"],
                        cu_seqlens=x["cu_seqlens"])
    for name, a, r in zip(GRADS + ("ds0",), out, ref):
        assert_close(name, host64(a), r, tol)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_bwd_ragged_with_state(dk, dv):
    x = make_inputs(2, 200, 2, dk, dv, "bf16", seed=300 + dk + dv, s0_std=0.02)
    do, dsn = _upstream(x, 1 + dk + dv)
    say("bwd ragged B2 T200 H2", dk, dv)
    check(x, do, dsn)


def test_bwd_no_state_grads_in():
    x = make_inputs(1, 130, 3, 128, 128, "bf16", seed=311)
    do, _ = _upstream(x, 7, with_dsn=False)
    say("bwd zero S0, no final-state gradient")
    check(x, do, None)


def test_bwd_varlen():
    lens = [1, 63, 64, 0, 65, 130, 7]
    x = make_inputs(1, sum(lens), 2, 128, 64, "bf16", seed=312, lengths=lens, s0_std=0.02)
    do, dsn = _upstream(x, 8)
    say("bwd varlen", lens)
    check(x, do, dsn)


@pytest.mark.parametrize("case", ["b0", "b1_w1", "b2"])
def test_bwd_gate_cases(case):
    x = make_inputs(1, 160, 2, 128, 128, "bf16", seed=313, s0_std=0.02)
    if case == "b0":
        x["b"][:] = 0.0
    elif case == "b1_w1":
        x["b"][:] = 1.0
        x["w"][:] = 1.0
    elif case == "b2":
        x["b"] = (2.0 * x["b"]).astype(np.float32)
    do, dsn = _upstream(x, 9)
    say("bwd gates", case)
    check(x, do, dsn)


@pytest.mark.parametrize("nats", [100.0, 150.0])
def test_bwd_wide_decay_chunk(nats):
    """A chunk whose total decay is past the chunk-referenced range of the forward (83 nats)
    but inside the backward's mid-referenced range (166 nats): in every key channel of the
    second chunk, and in half of the channels of the third."""
    x = make_inputs(1, 200, 2, 128, 128, "bf16", seed=315, s0_std=0.02)
    per = float(round_to_bf16(np.array([-nats / 64], np.float32))[0])
    x["g"][:, 64:128] = per
    x["g"][:, 128:192, :, ::2] = per
    do, dsn = _upstream(x, 12)
    say("bwd wide-decay chunk", nats)
    check(x, do, dsn)


def test_bwd_decay_concentrated_in_one_block():
    """100 nats over one chunk with 90 of them inside one aligned 16-token block: past any
    per-block referencing of the forward factors, inside the backward's per-chunk range."""
    x = make_inputs(1, 200, 2, 128, 128, "bf16", seed=317, s0_std=0.02)
    x["g"][:, 64:128] = float(round_to_bf16(np.array([-10.0 / 48], np.float32))[0])
    x["g"][:, 80:96] = float(round_to_bf16(np.array([-90.0 / 16], np.float32))[0])
    do, dsn = _upstream(x, 14)
    say("bwd decay concentrated in one block")
    check(x, do, dsn)


def test_bwd_near_resets():
    """Near-resets as in the long-context workload (10% of tokens at log-decay -5) plus one
    chunk with 18 of them (about 95 nats): inside the backward's range."""
    x = make_inputs(1, 640, 2, 128, 128, "bf16", seed=316, reset_frac=0.1, s0_std=0.02)
    x["g"][:, 320:338] = -5.0
    do, dsn = _upstream(x, 13)
    say("bwd near-resets T640")
    check(x, do, dsn)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("case", ["chunk_g-5", "chunk_g-8", "block_g-8", "token_g-300"])
def test_bwd_past_local_range(case, dk, dv):
    """Chunks past the local-gradient kernel's factor range (166 nats per channel over 64
    tokens), recomputed by the exact kernel: g = -5 or -8 on every token of the second chunk
    (320 or 512 nats), g = -8 on one aligned 16-token block plus -3 on the rest of its chunk
    (224 nats), two tokens at -300 (alpha underflows fp32); a ragged last chunk and an
    initial state."""
    x = make_inputs(1, 200, 2, dk, dv, "bf16", seed=318 + dk, s0_std=0.02)
    if case == "chunk_g-5":
        x["g"][:, 64:128] = -5.0
    elif case == "chunk_g-8":
        x["g"][:, 64:128] = -8.0
    elif case == "block_g-8":
        x["g"][:, 64:128] = -3.0
        x["g"][:, 80:96] = -8.0
    else:
        x["g"][:, 100:102] = -300.0
    do, dsn = _upstream(x, 15)
    say("bwd past the local range", case, dk, dv)
    check(x, do, dsn)


def test_bwd_past_local_range_varlen():
    lens = [70, 1, 130, 0, 99]
    x = make_inputs(1, sum(lens), 2, 128, 64, "bf16", seed=319, lengths=lens, s0_std=0.02)
    x["g"][:, 80:140] = -6.0  # spans the third sequence's first chunk
    do, dsn = _upstream(x, 16)
    say("bwd past the local range, varlen")
    check(x, do, dsn)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_bwd_many_units_sampled(dk, dv):
    """1024 (chunk, head) units, more than one per workgroup of the persistent local-gradient
    kernel (which walks units u, u + grid, ...), with a ragged last chunk and an initial
    state; the sampled chains (sequences 1 and 3) are units of the later iterations."""
    from oracle import gdn2_backward as ref_bwd
    x = make_inputs(4, 1000, 16, dk, dv, "bf16", seed=410 + dk + dv, s0_std=0.02)
    do, dsn = _upstream(x, 12 + dk + dv)
    say("bwd many units B4 T1000 H16", dk, dv, "(sampled chains)")
    out = run_bwd(x, do, dsn)
    for (n, h) in [(3, 5), (1, 14)]:
        sel = {m: x[m][n:n + 1, :, h:h + 1] for m in NAMES}
        ref = ref_bwd(*(sel[m] for m in NAMES), do[n:n + 1, :, h:h + 1],
                      dS_final=dsn[n:n + 1, h:h + 1], s0=x["s0"][n:n + 1, h:h + 1])
        print(f" chain (n={n}, h={h})", flush=True)
        for name, a, r in zip(GRADS, out[:6], ref[:6]):
            assert_close(name, host64(a[n:n + 1, :, h:h + 1]), r, TOL["bf16"])
        assert_close("ds0", host64(out[6][n:n + 1, h:h + 1]), ref[6], TOL["bf16"])


# ------------------------------------------- long sequences cut into parallel segments
@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 2048, 2, 128, 128), (2, 1100, 1, 128, 64),
                                         (1, 1500, 1, 64, 128), (1, 4096, 1, 64, 64)])
def test_bwd_segments(B, T, H, dk, dv):
    """Few long chains: the backward cuts each sequence into segments (the forward pass and
    the reverse chain each run a transfer pass per segment, a scan over segments, then the
    segments in parallel); the gradients are the plain reverse loop's."""
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=930 + T + dk, s0_std=0.05)
    do, dsn = _upstream(x, 31 + T)
    say("bwd segments", B, T, H, dk, dv)
    check(x, do, dsn)


def test_bwd_segments_saved_pair():
    """Segments through the training forward and the saved backward, with near-resets."""
    import gated_delta_rule_36_amd as G
    x = make_inputs(1, 3000, 2, 128, 128, "bf16", seed=937, reset_frac=0.1, s0_std=0.05)
    do, dsn = _upstream(x, 38)
    say("bwd segments saved pair T3000 H2, near-resets")
    t = {n: dev_tensor(x[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, sN, sv = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0)
    out = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(do, "bf16"), initial_state=s0,
                      d_final_state=torch.from_numpy(dsn).cuda(), saved=sv)
    torch.cuda.synchronize()
    from oracle import gdn2_forward
    o_ref, s_ref = gdn2_forward(*(x[n] for n in NAMES), s0=x["s0"])
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])
    ref = gdn2_backward(*(x[n] for n in NAMES), do, dS_final=dsn, s0=x["s0"])
    for name, a, r in zip(GRADS + ("ds0",), out, ref):
        assert_close(name, host64(a), r, TOL["bf16"])
    # A second backward on the same saved workspace (the first overwrote only what it may:
    # the segments' linear maps, kept by the training forward, are read again), with the
    # upstream gradients scaled by -2 (exact in bf16 and fp32), so the reference gradients
    # are the oracle's scaled by -2.
    out2 = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(-2.0 * do, "bf16"), initial_state=s0,
                       d_final_state=torch.from_numpy(-2.0 * dsn).cuda(), saved=sv)
    torch.cuda.synchronize()
    for name, a2, r in zip(GRADS + ("ds0",), out2, ref):
        assert_close(name + " (second call)", host64(a2), -2.0 * r, TOL["bf16"])
    # a third with the first call's upstream gradients repeats the first bit for bit
    out3 = G.chunk_bwd(*(t[n] for n in NAMES), dev_tensor(do, "bf16"), initial_state=s0,
                       d_final_state=torch.from_numpy(dsn).cuda(), saved=sv)
    torch.cuda.synchronize()
    for name, a, a3 in zip(GRADS + ("ds0",), out, out3):
        assert torch.equal(a, a3), f"{name}: third call differs from the first"



def test_bwd_layer1p3b_full_size_sampled():
    from gdn2_inputs import make_config_inputs
    from oracle import gdn2_backward as ref_bwd
    x = make_config_inputs("layer1p3b_bf16")
    do, dsn = _upstream(x, 11)
    say("bwd layer1p3b B8 H16 T2048 d128 (sampled chains)")
    out = run_bwd(x, do, dsn)
    for (n, h) in [(0, 0), (5, 9)]:
        sel = {m: x[m][n:n + 1, :, h:h + 1] for m in NAMES}
        ref = ref_bwd(*(sel[m] for m in NAMES), do[n:n + 1, :, h:h + 1],
                      dS_final=dsn[n:n + 1, h:h + 1])
        print(f" chain (n={n}, h={h})", flush=True)
        for name, a, r in zip(GRADS, out[:6], ref[:6]):
            assert_close(name, host64(a[n:n + 1, :, h:h + 1]), r, TOL["bf16"])
        assert_close("ds0", host64(out[6][n:n + 1, h:h + 1]), ref[6], TOL["bf16"])


def test_bwd_longctx_full_size_sampled():
    """The long-context workload (B1 H16 T32768, 10% near-resets): heads 15 and 3 each hold
    a chunk past 83 nats (chunks 13 and 40), inside the backward's mid-referenced range."""
    from gdn2_inputs import make_config_inputs
    from oracle import gdn2_backward as ref_bwd
    x = make_config_inputs("longctx_bf16")
    do, dsn = _upstream(x, 14)
    say("bwd longctx B1 H16 T32768 d128 (sampled heads 15, 3)")
    out = run_bwd(x, do, dsn)
    for h in (15, 3):
        sel = {m: x[m][:, :, h:h + 1] for m in NAMES}
        ref = ref_bwd(*(sel[m] for m in NAMES), do[:, :, h:h + 1], dS_final=dsn[:, h:h + 1])
        print(f" head {h}", flush=True)
        for name, a, r in zip(GRADS, out[:6], ref[:6]):
            assert_close(name, host64(a[:, :, h:h + 1]), r, TOL["bf16"])
        assert_close("ds0", host64(out[6][:, h:h + 1]), ref[6], TOL["bf16"])


def test_bwd_varlen_full_size_sampled():
    """The packed workload (16 sequences of 512..8192 tokens, nonzero initial states)."""
    from gdn2_inputs import make_config_inputs
    from oracle import gdn2_backward as ref_bwd
    x = make_config_inputs("varlen_bf16")
    do, dsn = _upstream(x, 15)
    cu = x["cu_seqlens"]
    lens = np.diff(cu)
    say("bwd varlen 16 seqs", int(lens.sum()), "tokens (sampled chains)")
    out = run_bwd(x, do, dsn)
    for n, h in ((int(np.argmin(lens)), 2), (5, 13)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        sel = {m: x[m][:, sl, h:h + 1] for m in NAMES}
        ref = ref_bwd(*(sel[m] for m in NAMES), do[:, sl, h:h + 1],
                      dS_final=dsn[n:n + 1, h:h + 1], s0=x["s0"][n:n + 1, h:h + 1])
        print(f" chain (n={n}, h={h})", flush=True)
        for name, a, r in zip(GRADS, out[:6], ref[:6]):
            assert_close(name, host64(a[:, sl, h:h + 1]), r, TOL["bf16"])
        assert_close("ds0", host64(out[6][n:n + 1, h:h + 1]), ref[6], TOL["bf16"])
