"""GPU parity of the recurrent decode step (through the C ABI) against the oracle."""
import numpy as np
import pytest
import torch

from gdn2_inputs import CONFIGS, make_decode_inputs
from oracle import gdn2_decode_steps
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_steps(x, steps, state):
    from gated_delta_rule_36_amd import decode_step
    dt = x["dtype"]
    t = {n: dev_tensor(x[n][:steps], dt) for n in NAMES}
    outs = []
    for s in range(steps):
        outs.append(decode_step(*(t[n][s] for n in NAMES), state))
    torch.cuda.synchronize()
    return torch.stack(outs)


def test_decode_1000_steps_16x16():
    """1000 consecutive steps of the decode workload's recurrence (bf16 inputs, fp32 state)
    on 16 sequences x 16 heads; every state and output against the oracle."""
    from tests.oracle_pool import decode_errors
    c = CONFIGS["decode_bf16"]
    steps = c["steps"]
    x = make_decode_inputs(16, c["H"], c["dk"], c["dv"], steps, "bf16", seed=c["seed"],
                           s0_std=0.02)
    say("decode 1000 steps N16 H16 d128 bf16")
    state = torch.from_numpy(x["s0"]).cuda()
    o = run_steps(x, steps, state)
    e = decode_errors(x["s0"], x, host64(o), host64(state), seqs_per_shard=1)
    print(f"  all states: o {e['o']:.3e}  S {e['S']:.3e}", flush=True)
    assert e["o"] <= TOL["bf16"] and e["S"] <= TOL["bf16"], e


def test_decode_full_batch_all_states():
    """The decode workload's full batch (256 sequences x 16 heads) over 12 steps; every one
    of the 4096 states and every output against the oracle."""
    from tests.oracle_pool import decode_errors
    c = CONFIGS["decode_bf16"]
    x = make_decode_inputs(c["N"], c["H"], c["dk"], c["dv"], 12, "bf16", seed=c["seed"] + 7,
                           s0_std=0.02)
    say("decode full batch N256 H16, 12 steps")
    state = torch.from_numpy(x["s0"]).cuda()
    o = run_steps(x, 12, state)
    e = decode_errors(x["s0"], x, host64(o), host64(state), seqs_per_shard=8)
    print(f"  all 4096 states: o {e['o']:.3e}  S {e['S']:.3e}", flush=True)
    assert np.all(np.isfinite(host64(state)))
    assert e["o"] <= TOL["bf16"] and e["S"] <= TOL["bf16"], e


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_decode_shapes(dt, dk, dv):
    x = make_decode_inputs(5, 3, dk, dv, 40, dt, seed=dk + dv, s0_std=0.02)
    say("decode", dt, dk, dv)
    state = torch.from_numpy(x["s0"]).cuda()
    o = run_steps(x, 40, state)
    o_ref, s_ref = gdn2_decode_steps(x["s0"], *(x[n] for n in NAMES))
    assert_close("o", host64(o), o_ref, TOL[dt])
    assert_close("S", host64(state), s_ref, TOL[dt])
