"""GPU parity of the multi-token decode against the pool (gdn2_decode_tokens, through the
C ABI) with the oracle's gdn2_decode_tokens: outputs, committed slots, per-token states."""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_decode_inputs
from oracle import gdn2_decode_tokens as ref_tokens
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "b", "w")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(N, L, H, dk, dv, dt, P, seed):
    x = make_decode_inputs(N, H, dk, dv, L, dt, seed=seed, s0_std=0.02)
    # [steps, N, H, d] -> [N, L, H, d]
    toks = {n: np.ascontiguousarray(np.swapaxes(x[n], 0, 1)) for n in NAMES}
    rng = np.random.default_rng(seed)
    pool = (rng.normal(size=(P, H, dk, dv)) * 0.02).astype(np.float32)
    idx = rng.permutation(P)[:N].astype(np.int32)
    idx[1] = -1  # one sequence without a state
    commit = rng.integers(0, L + 1, size=N).astype(np.int32)
    commit[0] = L
    return toks, pool, idx, commit


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_tokens(dt, dk, dv):
    import gated_delta_rule_36_amd as G
    N, L, H, P = 6, 4, 2, 9
    toks, pool, idx, commit = _case(N, L, H, dk, dv, dt, P, seed=dk + dv + (dt == "bf16"))
    say("decode_tokens", dt, dk, dv, "N6 L4 H2 P9")
    pool_t = torch.from_numpy(pool).cuda()
    t = {n: dev_tensor(toks[n], dt) for n in NAMES}
    o, steps = G.decode_tokens(*(t[n] for n in NAMES), pool_t,
                               state_indices=torch.from_numpy(idx).cuda(),
                               commit_len=torch.from_numpy(commit).cuda(),
                               return_step_states=True)
    torch.cuda.synchronize()
    o_ref, st_ref, pool_ref = ref_tokens(pool, *(toks[n] for n in NAMES), indices=idx,
                                         commit=commit)
    valid = idx >= 0
    vt = torch.from_numpy(valid).cuda()  # skipped sequences' outputs are left unwritten
    assert_close("o", host64(o[vt]), o_ref[valid], TOL[dt])
    assert_close("step states", host64(steps[vt]), st_ref[valid], TOL[dt])
    assert_close("pool", host64(pool_t), pool_ref, TOL[dt])
    untouched = [s for s in range(P) if s not in idx[valid]]
    assert np.array_equal(pool_t.cpu().numpy()[untouched], pool[untouched])


def test_decode_tokens_equals_chunk_forward():
    """L tokens from the pool equal the chunk forward over the same L tokens from that state."""
    import gated_delta_rule_36_amd as G
    N, L, H, P = 4, 16, 4, 4
    toks, pool, _, _ = _case(N, L, H, 128, 128, "bf16", P, seed=77)
    say("decode_tokens vs chunk_fwd N4 L16 H4")
    t = {n: dev_tensor(toks[n], "bf16") for n in NAMES}
    pool_t = torch.from_numpy(pool).cuda()
    o_fwd, s_fwd = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=pool_t.clone())
    o, _ = G.decode_tokens(*(t[n] for n in NAMES), pool_t)
    torch.cuda.synchronize()
    assert_close("o", host64(o), host64(o_fwd), TOL["bf16"])
    assert_close("S", host64(pool_t), host64(s_fwd), TOL["bf16"])
