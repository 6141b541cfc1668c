"""The allocation-free forward (gdn2_chunk_fwd_noalloc, library-held scratch) against the
same two-phase forward with a caller workspace (gdn2_chunk_fwd_ex), through the C ABI: two
calls in a row, the second smaller and packed, so the second runs on the scratch the first
left behind. Also checked against the float64 oracle at the bf16 tolerance."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_36_amd import _lib
from gdn2_inputs import make_inputs
from oracle import gdn2_forward
from tests.gpu_util import TOL, assert_close, host64, say

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "b", "w")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(x, B, T, H, dk, dv, N, layout, cu, s0, noalloc):
    dev = torch.device("cuda")
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n], np.float32)).to(torch.bfloat16).to(dev)
         for n in NAMES}
    cu_t = None if cu is None else torch.tensor(cu, dtype=torch.int32, device=dev)
    s0_t = None if s0 is None else torch.from_numpy(s0.astype(np.float32)).to(dev)
    o = torch.full((B, T, H, dv), float("nan"), dtype=torch.bfloat16, device=dev)
    sN = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    L = _lib.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [_ptr(t[n]) for n in NAMES] + [_ptr(s0_t), _ptr(o), _ptr(sN), _ptr(cu_t),
                                          B, T, H, dk, dv, N, 0, layout]
    if noalloc:
        st = L.gdn2_chunk_fwd_noalloc(*args, stream)
    else:
        need = int(L.gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, 0))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        st = L.gdn2_chunk_fwd_ex(*args, _ptr(ws), need, stream)
    assert st == 0, L.gdn2_status_string(st)
    torch.cuda.synchronize()
    return o, sN


def _case(B, T, H, dk, dv, cu, layout, seed):
    N = B if cu is None else len(cu) - 1
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=seed)
    if layout & 1:
        x["b"] = np.ascontiguousarray(x["b"][..., 0])
    if layout & 2:
        x["w"] = np.ascontiguousarray(x["w"][..., 0])
    s0 = np.random.default_rng(seed).normal(0, 0.02, size=(N, H, dk, dv)).astype(np.float32)
    return x, N, s0


def _check(B, T, H, dk, dv, cu, layout, seed):
    x, N, s0 = _case(B, T, H, dk, dv, cu, layout, seed)
    say(f"noalloc B{B} T{T} H{H} dk{dk} dv{dv} cu={cu} layout={layout} seed={seed}")
    o1, s1 = _run(x, B, T, H, dk, dv, N, layout, cu, s0, noalloc=True)
    o2, s2 = _run(x, B, T, H, dk, dv, N, layout, cu, s0, noalloc=False)
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "noalloc differs from the workspace call"
    xb = dict(x)
    if layout & 1:
        xb["b"] = np.repeat(x["b"][..., None], dk, axis=-1)
    if layout & 2:
        xb["w"] = np.repeat(x["w"][..., None], dv, axis=-1)
    o_ref, s_ref = gdn2_forward(*(xb[n] for n in NAMES), s0=s0, cu_seqlens=cu)
    assert_close("o", host64(o1), o_ref, TOL["bf16"])
    assert_close("S", host64(s1), s_ref, TOL["bf16"])


def test_noalloc_two_calls_second_smaller():
    # first: two sequences of 1000 tokens, cut into segments (few chains)
    _check(2, 1000, 4, 128, 128, None, 0, seed=41)
    # second, smaller, on the scratch the first left: packed, scalar gates, d_v = 64
    _check(1, 200, 2, 128, 64, [0, 5, 70, 200], 3, seed=42)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    L = _lib.lib()
    cap = int(L.gdn2_noalloc_scratch_bytes())
    T = 1 << 20
    need = int(L.gdn2_chunk_fwd_workspace_bytes(1, T, 16, 128, 128, 1, 0))
    assert need > cap
    fake = ctypes.c_void_p(0x100000)
    st = L.gdn2_chunk_fwd_noalloc(*([fake] * 6), None, fake, None, None, 1, T, 16, 128, 128,
                                  1, 0, 0, None)
    assert st == 3 and b"scratch" in L.gdn2_status_string(st)
