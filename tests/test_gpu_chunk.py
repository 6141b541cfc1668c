"""GPU parity of the chunkwise forward (through the C ABI) against the float64 oracle.

Both paths are covered: "fused" (one kernel per sequence, value-slice widths) and "split"
(two-phase: parallel chunk factors into a workspace, then the per-sequence recurrence).
Tolerances (normwise max relative error per tensor, on o and on the final state):
1e-4 for fp32 runs, 2e-2 for bf16 runs.
"""
import numpy as np
import pytest
import torch

from gdn2_inputs import make_config_inputs, make_inputs
from oracle import gdn2_forward
from tests.gpu_util import TOL, assert_close, dev_tensor, host64, say

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _lib():
    import gated_delta_rule_36_amd as G
    return G


def run_gpu(x, value_slice=0, s0=None, use_s0=True, path="auto"):
    G = _lib()
    dt = x["dtype"]
    t = {n: dev_tensor(x[n], dt) for n in NAMES}
    s0 = x["s0"] if (use_s0 and s0 is None) else s0
    s0_t = None if s0 is None else torch.from_numpy(np.ascontiguousarray(s0, np.float32)).cuda()
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).cuda()
    o, sN = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0_t, cu_seqlens=cu,
                        value_slice=value_slice, path=path)
    torch.cuda.synchronize()
    return o, sN


def run_oracle(x):
    return gdn2_forward(*(x[n] for n in NAMES), s0=x["s0"], cu_seqlens=x["cu_seqlens"])


def slices_for(dt, dk, dv):
    out = []
    for nv in (16, 32, 64, 128):
        if nv > dv:
            continue
        if dt == "bf16" and nv == 16 and dk != 64:
            continue
        if dt == "fp32" and (dk != 64 or nv == 128):
            continue
        out.append(nv)
    return out


# ------------------------------------------------------------------ small, full oracle
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("varlen", [False, True])
def test_fp32_dk128(dv, varlen):
    """fp32 with d_k = 128 (the token-recurrent kernel): ragged lengths spanning several
    16-token blocks, an initial state, fp32 tolerance."""
    if varlen:
        lens = [37, 0, 150, 1, 64]
        x = make_inputs(1, sum(lens), 3, 128, dv, "fp32", seed=61 + dv, lengths=lens, s0_std=0.05)
    else:
        x = make_inputs(2, 130, 3, 128, dv, "fp32", seed=71 + dv, s0_std=0.05)
    say("fp32 d_k=128", "dv", dv, "varlen", varlen)
    o, sN = run_gpu(x, 0)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["fp32"])
    assert_close("S", host64(sN), s_ref, TOL["fp32"])



@pytest.mark.parametrize("nv", [16, 32, 64])
def test_tiny_fp32_config(nv):
    x = make_config_inputs("tiny_fp32")
    say("tiny_fp32 B1 H2 T256 d64", "nv", nv)
    o, sN = run_gpu(x, nv)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["fp32"])
    assert_close("S", host64(sN), s_ref, TOL["fp32"])


CASES = [(dk, dv, nv) for dk in (64, 128) for dv in (64, 128) for nv in slices_for("bf16", dk, dv)]


@pytest.mark.parametrize("dk,dv,nv", CASES)
def test_bf16_ragged_with_state(dk, dv, nv):
    x = make_inputs(2, 200, 2, dk, dv, "bf16", seed=7 + dk + dv + nv, s0_std=0.02)
    say("bf16 ragged B2 T200 H2", dk, dv, "nv", nv)
    o, sN = run_gpu(x, nv)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


@pytest.mark.parametrize("dk,dv", [(dk, dv) for dk in (64, 128) for dv in (64, 128)])
def test_bf16_ragged_split(dk, dv):
    x = make_inputs(2, 200, 2, dk, dv, "bf16", seed=3 + dk + dv, s0_std=0.02)
    say("bf16 ragged B2 T200 H2 split", dk, dv)
    o, sN = run_gpu(x, path="split")
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


def test_split_many_heads_value_slices():
    # 2 x 70 chains: the recurrence kernel takes 64-wide slices (>= 256 workgroups) and
    # the factor kernel loops over many (chunk, head) units per workgroup
    x = make_inputs(2, 130, 70, 128, 128, "bf16", seed=17, s0_std=0.02)
    say("split B2 T130 H70")
    o, sN = run_gpu(x, path="split")
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


@pytest.mark.parametrize("dv,nv", [(128, 16), (128, 32), (128, 64), (64, 32)])
def test_fp32_ragged_with_state(dv, nv):
    x = make_inputs(1, 150, 3, 64, dv, "fp32", seed=31 + nv, s0_std=0.02)
    say("fp32 ragged B1 T150 H3 dk64", dv, "nv", nv)
    o, sN = run_gpu(x, nv)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["fp32"])
    assert_close("S", host64(sN), s_ref, TOL["fp32"])


@pytest.mark.parametrize("dt,path", [("bf16", "fused"), ("bf16", "split"), ("fp32", "fused")])
def test_varlen_small_edges(dt, path):
    lens = [1, 63, 64, 0, 65, 130, 7]
    dk = 128 if dt == "bf16" else 64
    x = make_inputs(1, sum(lens), 2, dk, 64, dt, seed=77, lengths=lens, s0_std=0.02)
    say("varlen small", dt, path, lens)
    o, sN = run_gpu(x, path=path)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL[dt])
    assert_close("S", host64(sN), s_ref, TOL[dt])


@pytest.mark.parametrize("path,nseq", [("split", 150), ("fused", 150), ("fused", 256)])
def test_varlen_many_sequences(path, nseq):
    # 150 or 256 sequences (lengths 0..200, several empty, several of equal length): the factor
    # kernel finds each chunk's sequence with a 64-way search that needs more than one round
    # here; the fused kernel starts them longest first (ties by index; 256 is the most it
    # orders)
    rng = np.random.default_rng(123 + nseq)
    lens = [int(v) for v in rng.integers(0, 200, size=nseq)]
    lens[3] = lens[77] = 0
    lens[10] = lens[11] = lens[140] = 130
    x = make_inputs(1, sum(lens), 1, 64, 64, "bf16", seed=55, lengths=lens, s0_std=0.02)
    say("varlen", nseq, "sequences", path, sum(lens), "tokens")
    o, sN = run_gpu(x, path=path)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


def test_varlen_beyond_ordered_count_fused():
    # more sequences than the fused kernel orders by length (256): natural order
    rng = np.random.default_rng(321)
    lens = [int(v) for v in rng.integers(0, 24, size=300)]
    x = make_inputs(1, sum(lens), 1, 64, 64, "bf16", seed=56, lengths=lens, s0_std=0.02)
    say("varlen 300 sequences fused", sum(lens), "tokens")
    o, sN = run_gpu(x, path="fused")
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


@pytest.mark.parametrize("path", ["fused", "split"])
def test_varlen_equals_separate_runs(path):
    lens = [70, 5, 128, 33]
    x = make_inputs(1, sum(lens), 2, 128, 128, "bf16", seed=91, lengths=lens, s0_std=0.02)
    say("varlen vs separate", path, lens)
    vs = 64 if path == "fused" else 0
    o, sN = run_gpu(x, vs, path=path)
    cu = x["cu_seqlens"]
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        xn = {m: x[m][:, sl] for m in NAMES}
        xn.update(dtype="bf16", cu_seqlens=None, s0=x["s0"][n:n + 1])
        on, sn = run_gpu(xn, vs, path=path)
        assert torch.equal(o[:, sl], on)
        assert torch.equal(sN[n:n + 1], sn)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_deterministic(path):
    x = make_inputs(2, 300, 4, 128, 128, "bf16", seed=5)
    say("determinism", path)
    o1, s1 = run_gpu(x, path=path)
    o2, s2 = run_gpu(x, path=path)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_zero_length_and_alias(path):
    G = _lib()
    x = make_inputs(2, 96, 2, 128, 128, "bf16", seed=3, s0_std=0.02)
    say("T=0 and aliasing", path)
    t = {n: dev_tensor(x[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    # T = 0: final state is the initial state
    empty = {n: t[n][:, :0].contiguous() for n in NAMES}
    _, sN = G.chunk_fwd(*(empty[n] for n in NAMES), initial_state=s0, path=path)
    torch.cuda.synchronize()
    assert torch.equal(sN, s0)
    # final_state aliasing initial_state through the C ABI
    import ctypes
    from gated_delta_rule_36_amd import _lib as L
    o_ref, s_ref = run_gpu(x, path=path)
    st = s0.clone()
    o = torch.empty_like(t["v"])
    p = lambda a: ctypes.c_void_p(a.data_ptr())
    nws = L.lib().gdn2_chunk_fwd_workspace_bytes(2, 96, 2, 128, 128, 2, 0) if path == "split" else 0
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    rc = L.lib().gdn2_chunk_fwd(*(p(t[n]) for n in NAMES), p(st), p(o), p(st), None,
                                2, 96, 2, 128, 128, 2, 0, p(ws) if nws else None, nws,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("case", ["all_g_-5", "b0", "b1_w1", "w0", "b2"])
def test_extreme_gates(case, path):
    x = make_inputs(1, 160, 2, 128, 128, "bf16", seed=13, s0_std=0.02)
    if case == "all_g_-5":
        x["g"][:] = -5.0
    elif case == "b0":
        x["b"][:] = 0.0
    elif case == "b1_w1":
        x["b"][:] = 1.0
        x["w"][:] = 1.0
    elif case == "w0":
        x["w"][:] = 0.0
    elif case == "b2":  # erase gate widened to [0, 2]
        x["b"] = (2.0 * x["b"]).astype(np.float32)
    say("extreme gates", case, path)
    o, sN = run_gpu(x, path=path)
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S", host64(sN), s_ref, TOL["bf16"])


def test_prefill_then_decode():
    G = _lib()
    T, s = 150, 6
    x = make_inputs(2, T, 2, 128, 128, "bf16", seed=21, s0_std=0.02)
    say("prefill then decode")
    t = {n: dev_tensor(x[n], "bf16") for n in NAMES}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o_full, s_full = G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0)
    pre = {n: t[n][:, :T - s].contiguous() for n in NAMES}
    o_pre, st = G.chunk_fwd(*(pre[n] for n in NAMES), initial_state=s0)
    outs = []
    for j in range(T - s, T):
        step = {n: t[n][:, j].contiguous() for n in NAMES}
        outs.append(G.decode_step(*(step[n] for n in NAMES), st))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    assert_close("o prefix", host64(o_pre), host64(o_full[:, :T - s]), 1e-6)
    assert_close("o decoded", host64(o_dec), host64(o_full[:, T - s:]), TOL["bf16"])
    assert_close("S", host64(st), host64(s_full), TOL["bf16"])


# ------------------------------------------------- full-size workloads, every chain
_CACHE = {}


def _full(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = make_config_inputs(name)
    return _CACHE[name]


def _check_all_chains(x, o, sN):
    """Every (sequence, head) chain of the workload against the oracle (host process pool)."""
    from tests.oracle_pool import forward_errors
    e = forward_errors(x, host64(o), host64(sN))
    print(f"  all chains ({e['shards']} shards): o {e['o']:.3e}  S {e['S']:.3e}", flush=True)
    assert np.all(np.isfinite(host64(o))) and np.all(np.isfinite(host64(sN)))
    assert e["o"] <= TOL["bf16"], f"o: normwise max rel err {e['o']:.3e}"
    assert e["S"] <= TOL["bf16"], f"S: normwise max rel err {e['S']:.3e}"


@pytest.mark.parametrize("path", ["fused", "split"])
def test_layer1p3b_full_size_all_chains(path):
    x = _full("layer1p3b_bf16")
    say("layer1p3b B8 H16 T2048 d128 bf16, all 128 chains", path)
    o, sN = run_gpu(x, path=path)
    _check_all_chains(x, o, sN)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_longctx_full_size_all_chains(path):
    x = _full("longctx_bf16")
    say("longctx B1 H16 T32768 d128 bf16, 10% near-resets, all 16 chains", path)
    o, sN = run_gpu(x, path=path)
    _check_all_chains(x, o, sN)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_varlen_full_size_all_chains(path):
    x = _full("varlen_bf16")
    lens = np.diff(x["cu_seqlens"])
    say("varlen 16 seqs", int(lens.sum()), "tokens, all 256 chains", path)
    o, sN = run_gpu(x, path=path)
    _check_all_chains(x, o, sN)


# ------------------------------------------- long sequences cut into parallel segments
@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 2048, 2, 128, 128), (2, 1100, 1, 128, 64),
                                         (1, 1500, 1, 64, 128), (1, 4096, 1, 64, 64)])
def test_split_segments(B, T, H, dk, dv):
    """Few long chains: the two-phase path cuts each sequence into segments (transfer pass,
    start-state scan, outputs per segment); the result is the plain recurrence's."""
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=900 + T + dk, s0_std=0.05)
    say("split segments", B, T, H, dk, dv)
    o, sN = run_gpu(x, path="split")
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])


def test_split_segments_near_resets():
    """Segments with large decays inside (near-resets), as in the long-context workload."""
    x = make_inputs(1, 3000, 2, 128, 128, "bf16", seed=907, reset_frac=0.1, s0_std=0.05)
    say("split segments near-resets T3000 H2")
    o, sN = run_gpu(x, path="split")
    o_ref, s_ref = run_oracle(x)
    assert_close("o", host64(o), o_ref, TOL["bf16"])
    assert_close("S_final", host64(sN), s_ref, TOL["bf16"])
