"""GPU parity of the chunk forwards against the float64 oracle over the whole decay domain
that alpha in (0, 1] allows (reading note §1 gate domains, §2 Diag(alpha_t)).

The pipelined fused forward (gdn2_chunk_fwd without a workspace, bf16): every width pair
on ragged lengths with an initial state, long sequences (many chunks through the double-
buffered pipeline), and strong decay on every token of one chunk, on one aligned 16-token
block, on every token of a sequence, single near-total resets, and decays far below fp32
range (alpha that underflows). The same decay cases also run through every other forward:
the two-phase path (with a workspace), the training forward, the value-sliced fused kernel,
its fp32 build (d_k = 64) and the fp32 token-recurrent kernel (d_k = 128).
Tolerance: normwise max relative error 2e-2 on o and on the final state (1e-4 in fp32)."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_inputs, make_scalar_gate, round_to_bf16
from oracle import gdn2_forward
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "b", "w")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(x, path="fused", scalar_b=None, scalar_w=None):
    """path: "fused" or "split" (chunk_fwd), "train" (chunk_fwd_train) or "sliced"
    (chunk_fwd with 32-wide value slices)."""
    import gated_delta_rule_36_amd as G
    t = {n: dev_tensor(x[n], x["dtype"]) for n in NAMES}
    if scalar_b is not None:
        t["b"] = dev_tensor(scalar_b, x["dtype"])
    if scalar_w is not None:
        t["w"] = dev_tensor(scalar_w, x["dtype"])
    s0 = None if x["s0"] is None else torch.from_numpy(np.ascontiguousarray(x["s0"])).cuda()
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    args = [t[n] for n in NAMES]
    if path == "train":
        o, sN, _ = G.chunk_fwd_train(*args, initial_state=s0, cu_seqlens=cu)
    elif path == "sliced":
        o, sN = G.chunk_fwd(*args, initial_state=s0, cu_seqlens=cu, path="fused", value_slice=32)
    else:
        o, sN = G.chunk_fwd(*args, initial_state=s0, cu_seqlens=cu, path=path)
    torch.cuda.synchronize()
    return host64(o), host64(sN)


def _check(x, path="fused", scalar_b=None, scalar_w=None):
    o, sN = _run(x, path, scalar_b, scalar_w)
    xr = dict(x)
    if scalar_b is not None:
        xr["b"] = np.repeat(scalar_b[..., None], x["q"].shape[-1], axis=-1)
    if scalar_w is not None:
        xr["w"] = np.repeat(scalar_w[..., None], x["v"].shape[-1], axis=-1)
    o_ref, s_ref = gdn2_forward(*(xr[n] for n in NAMES), s0=x["s0"], cu_seqlens=x["cu_seqlens"])
    assert_close("o", o, o_ref, TOL[x["dtype"]])
    assert_close("S", sN, s_ref, TOL[x["dtype"]])


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_widths_ragged_with_state(dk, dv):
    x = make_inputs(2, 200, 3, dk, dv, "bf16", seed=101 + dk + dv, s0_std=0.05)
    say("pipelined fwd B2 T200 H3", dk, dv)
    _check(x)


@pytest.mark.parametrize("dk", [64, 128])
def test_many_chunks(dk):
    x = make_inputs(1, 1000, 2, dk, 128, "bf16", seed=202 + dk, s0_std=0.05)
    say("pipelined fwd B1 T1000 H2", dk)
    _check(x)


def _with_decay(x, tokens, g_nats):
    g = np.array(x["g"])
    g[:, tokens] = round_to_bf16(np.full_like(g[:, tokens], g_nats))
    return dict(x, g=g)


RANGE_CASES = {
    "chunk1_all_tokens_g-8": (slice(64, 128), -8.0),      # 512 nats over one chunk
    "aligned_block_g-8": (slice(80, 96), -8.0),           # 128 nats over one 16-token block
    "all_tokens_g-8": (slice(0, 300), -8.0),              # every chunk on the general path
    "single_reset_g-60": ([150], -60.0),                  # one token, within the fast path
    "single_reset_g-300": ([150, 151], -300.0),           # alpha underflows fp32
    "block_g-40_ragged_tail": (slice(272, 300), -40.0),   # last, ragged chunk
}


@pytest.mark.parametrize("case", list(RANGE_CASES))
@pytest.mark.parametrize("dk", [64, 128])
def test_decay_range(case, dk):
    tokens, gn = RANGE_CASES[case]
    x = _with_decay(make_inputs(2, 300, 2, dk, 128, "bf16", seed=303 + dk, s0_std=0.05),
                    tokens, gn)
    say("pipelined fwd range", case, "dk", dk)
    _check(x)


def test_decay_range_varlen_and_scalar_gates():
    lens = [70, 1, 130, 0, 99]
    x = make_inputs(1, sum(lens), 2, 128, 64, "bf16", seed=404, lengths=lens, s0_std=0.05)
    x = _with_decay(x, slice(16, 48), -9.0)      # inside the first sequence
    x = _with_decay(x, slice(100, 140), -7.0)    # spans the third sequence's chunks
    sb = make_scalar_gate(x["q"].shape[:3], seed=404)
    sw = make_scalar_gate(x["q"].shape[:3], seed=405)
    say("pipelined fwd range varlen + scalar gates")
    _check(x)
    _check(x, scalar_b=sb)
    _check(x, scalar_b=sb, scalar_w=sw)


@pytest.mark.parametrize("case", list(RANGE_CASES))
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("path", ["split", "train", "sliced"])
def test_decay_range_other_paths(path, case, dk):
    tokens, gn = RANGE_CASES[case]
    x = _with_decay(make_inputs(2, 300, 2, dk, 128, "bf16", seed=313 + dk, s0_std=0.05),
                    tokens, gn)
    say("fwd range", path, case, "dk", dk)
    _check(x, path)


@pytest.mark.parametrize("case", list(RANGE_CASES))
@pytest.mark.parametrize("dk", [64, 128])
def test_decay_range_fp32(case, dk):
    tokens, gn = RANGE_CASES[case]
    x = _with_decay(make_inputs(2, 300, 2, dk, 64, "fp32", seed=323 + dk, s0_std=0.05), tokens, gn)
    say("fwd range fp32", case, "dk", dk)
    _check(x)


@pytest.mark.parametrize("path", ["split", "train"])
def test_decay_range_other_paths_varlen_scalar_gates(path):
    lens = [70, 1, 130, 0, 99]
    x = make_inputs(1, sum(lens), 2, 128, 64, "bf16", seed=414, lengths=lens, s0_std=0.05)
    x = _with_decay(x, slice(16, 48), -9.0)
    x = _with_decay(x, slice(100, 140), -7.0)
    sb = make_scalar_gate(x["q"].shape[:3], seed=414)
    say("fwd range varlen + scalar b", path)
    _check(x, path, scalar_b=sb)
