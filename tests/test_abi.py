"""Host-only checks of the C ABI: the library loads, exports every declared entry point,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_36_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.lib_path()),
                                reason="libgdn2.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert "gdn2_chunk_fwd" in names and "gdn2_decode_step" in names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    L = _lib.lib()
    assert b"gfx950" in L.gdn2_version()
    for s in (0, 1, 2, 3, 4, 99):
        assert L.gdn2_status_string(s)


FAKE = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced on error paths
MIS = ctypes.c_void_p(0x100004)


def _chunk(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, w=FAKE, s0=None, o=FAKE, sN=None, cu=None,
             B=2, T=64, H=4, dk=128, dv=128, N=2, dtype=0, ws=None, wsz=0)
    a.update(kw)
    return _lib.lib().gdn2_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["b"], a["w"], a["s0"],
                                     a["o"], a["sN"], a["cu"], a["B"], a["T"], a["H"],
                                     a["dk"], a["dv"], a["N"], a["dtype"], a["ws"], a["wsz"],
                                     None)


def test_chunk_fwd_error_paths():
    assert _chunk(dtype=7) == 1
    assert _chunk(N=3) == 1                 # N must equal B without cu_seqlens
    assert _chunk(H=0) == 1
    assert _chunk(T=-1) == 1
    assert _chunk(dk=96) == 2
    assert _chunk(dv=256) == 2
    assert _chunk(q=None) == 1
    assert _chunk(o=None) == 1
    assert _chunk(k=MIS) == 1               # misaligned
    assert _chunk(cu=FAKE, B=2) == 1        # packed batches have B == 1
    assert _chunk(B=0, N=0, q=None, k=None, v=None, g=None, b=None, w=None, o=None) == 0
    # two-phase path: the workspace must be aligned and large enough
    # (sizes just below what this call needs: 2 sequences x 1 chunk x 4 heads x 74240 B, so
    # nothing is launched)
    need = 2 * 1 * 4 * 74240
    assert _chunk(ws=MIS, wsz=need) == 1
    assert _chunk(ws=FAKE, wsz=need - 1) == 3
    assert _chunk(ws=FAKE, wsz=0) == 3
    assert _chunk(ws=FAKE, wsz=need - 1, cu=FAKE, B=1, T=128, N=2) == 3  # packed: 4 slots
    # fp32 has no two-phase path: the workspace is ignored (then the N check still applies)
    assert _chunk(ws=FAKE, wsz=0, dtype=1, dk=64, N=3) == 1


def test_workspace_bytes():
    L = _lib.lib()
    unit128 = 4 * 4 * 1024 * 3 + 8 * 1024 + 8 * 4 * 512 + 512  # -W, Qbar, Kt, P, U~, gamma
    assert unit128 == 74240
    # fixed length: B * ceil(T / 64) slots; packed: floor(T / 64) + N; the larger of the two
    assert L.gdn2_chunk_fwd_workspace_bytes(2, 64, 4, 128, 128, 2, 0) == (2 + 2) * 4 * unit128
    # one long sequence with 32 chains (16 heads x 2 value slices) < 256: 4 segments of 8
    # chunks, whose end states [N | M] and start states follow the factors (fp32)
    seg = 256 + 1 * 16 * 4 * 128 * (2 * 128 + 128) * 4
    assert L.gdn2_chunk_fwd_workspace_bytes(1, 2048, 16, 128, 128, 1, 0) == 32 * 16 * unit128 + seg
    assert L.gdn2_chunk_fwd_workspace_bytes(8, 2048, 16, 128, 128, 8, 0) == (256 + 8) * 16 * unit128
    assert L.gdn2_chunk_fwd_workspace_bytes(64, 100, 1, 128, 128, 64, 0) == (100 + 64) * unit128
    unit64 = 4 * 2 * 1024 * 3 + 8 * 1024 + 4 * 4 * 512 + 256
    assert L.gdn2_chunk_fwd_workspace_bytes(1, 64, 1, 64, 64, 1, 0) == 2 * ((unit64 + 255) // 256 * 256)
    assert L.gdn2_chunk_fwd_workspace_bytes(1, 64, 1, 64, 64, 1, 1) == 0    # fp32: fused only
    assert L.gdn2_chunk_fwd_workspace_bytes(1, 64, 1, 96, 64, 1, 0) == 0
    assert L.gdn2_chunk_fwd_workspace_bytes(1, -1, 1, 64, 64, 1, 0) == 0


def test_chunk_fwd_sliced_error_paths():
    L = _lib.lib()

    def call(nv, dk=128, dv=128, dtype=0):
        return L.gdn2_chunk_fwd_sliced(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                                       1, 64, 2, dk, dv, 1, dtype, nv, None)
    assert call(-1) == 1
    assert call(48) == 2
    assert call(16) == 2                    # 16-wide slices need d_k = 64
    assert call(256) == 2
    assert call(128, dk=64, dv=64) == 2     # wider than d_v
    assert call(128, dk=64, dv=128, dtype=1) == 2
    assert call(64, dk=128, dv=128, dtype=1) == 2  # fp32, d_k = 128: token-recurrent, no slices


def test_decode_error_paths():
    L = _lib.lib()

    def call(**kw):
        a = dict(q=FAKE, state=FAKE, N=4, H=2, dk=128, dv=128, dtype=0)
        a.update(kw)
        return L.gdn2_decode_step(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, a["state"], FAKE,
                                  a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)
    assert call(dtype=2) == 1
    assert call(N=-1) == 1
    assert call(dk=32) == 2
    assert call(q=None) == 1
    assert call(state=MIS) == 1
    assert call(N=0, q=None, state=None) == 0


def _bwd(**kw):
    a = dict(B=2, T=64, H=4, dk=128, dv=128, N=2, dtype=0, ws=None, wsz=0, q=FAKE, flag=None)
    a.update(kw)
    L = _lib.lib()
    return L.gdn2_chunk_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, a["flag"], None,
                            a["B"], a["T"], a["H"], a["dk"], a["dv"], a["N"], a["dtype"],
                            a["ws"], a["wsz"], None)


def test_chunk_bwd_error_paths():
    L = _lib.lib()
    need = 2 * 1 * 4 * 238080  # two sequences x one chunk x 4 heads x the d=128 unit
    assert L.gdn2_chunk_bwd_workspace_bytes(2, 64, 4, 128, 128, 2, 0) == (2 + 2) * 4 * 238080
    assert L.gdn2_chunk_bwd_workspace_bytes(2, 64, 4, 64, 64, 2, 1) == 0      # fp32: not built
    # a long sequence with few chains is cut into segments (4 of 8 chunks here): the segment
    # buffers ([units][d_k][2 d_v + d_k] fp32, 256-byte aligned) follow the per-chunk units
    seg = 256 + 1 * 2 * 4 * 128 * (2 * 128 + 128) * 4
    assert L.gdn2_chunk_bwd_workspace_bytes(1, 2048, 2, 128, 128, 1, 0) == 32 * 2 * 238080 + seg
    assert _bwd(dtype=1, dk=64, dv=64) == 2
    assert _bwd(dtype=7) == 1
    assert _bwd(dk=96) == 2
    assert _bwd(N=3) == 1
    assert _bwd(q=None) == 1
    assert _bwd(q=MIS, ws=FAKE, wsz=need) == 1
    assert _bwd(ws=None, wsz=need) == 3                 # the workspace is required
    assert _bwd(ws=FAKE, wsz=need - 1) == 3
    assert _bwd(ws=MIS, wsz=need) == 1
    assert _bwd(flag=ctypes.c_void_p(0x100002), ws=FAKE, wsz=need) == 1  # misaligned flag
    assert _bwd(B=0, N=0, q=None, ws=FAKE, wsz=0) == 0


def test_decode_tokens_error_paths():
    L = _lib.lib()

    def call(**kw):
        a = dict(N=2, Lt=4, H=2, dk=128, dv=128, P=2, dtype=0, idx=None, pool=FAKE, steps=None)
        a.update(kw)
        return L.gdn2_decode_tokens(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["pool"], a["idx"], None,
                                    FAKE, a["steps"], a["N"], a["Lt"], a["H"], a["dk"], a["dv"],
                                    a["P"], a["dtype"], None)
    assert call(dtype=5) == 1
    assert call(dk=32) == 2
    assert call(P=1) == 1                 # without indices the pool needs a slot per sequence
    assert call(pool=None) == 1
    assert call(pool=MIS) == 1
    assert call(steps=MIS) == 1
    assert call(idx=ctypes.c_void_p(0x100002)) == 1
    assert call(N=0, pool=None) == 0
    assert call(Lt=0, pool=None) == 0


def test_block_prologue_epilogue_error_paths():
    L = _lib.lib()

    def pro(**kw):
        a = dict(x=FAKE, out=FAKE, cu=None, B=2, T=8, H=2, dk=128, dv=64, N=2, dtype=0, taps=FAKE)
        a.update(kw)
        return L.gdn2_block_prologue(a["x"], FAKE, FAKE, FAKE, FAKE, FAKE, a["taps"], FAKE, FAKE,
                                     FAKE, 1.0, a["out"], FAKE, FAKE, FAKE, FAKE, FAKE, a["cu"],
                                     a["B"], a["T"], a["H"], a["dk"], a["dv"], a["N"],
                                     a["dtype"], None)
    assert pro(dtype=3) == 1
    assert pro(N=3) == 1                  # N must equal B without cu_seqlens
    assert pro(cu=FAKE, B=2) == 1         # packed batches have B = 1
    assert pro(dk=96) == 2
    assert pro(x=MIS) == 1
    assert pro(taps=None) == 1
    assert pro(H=0) == 1
    assert pro(T=0, x=None) == 0          # no tokens: nothing to do, nothing touched

    def epi(**kw):
        a = dict(o=FAKE, y=FAKE, rows=16, dv=128, dtype=0)
        a.update(kw)
        return L.gdn2_block_epilogue(a["o"], FAKE, FAKE, a["y"], a["rows"], a["dv"], a["dtype"],
                                     None)
    assert epi(dtype=2) == 1
    assert epi(dv=32) == 2
    assert epi(rows=-1) == 1
    assert epi(y=MIS) == 1
    assert epi(rows=0, o=None) == 0


def test_gate_layout_error_paths():
    L = _lib.lib()
    base = [FAKE] * 6 + [None, FAKE, None, None]
    assert L.gdn2_chunk_fwd_ex(*base, 2, 64, 4, 128, 128, 2, 0, 4, None, 0, None) == 1
    assert L.gdn2_chunk_fwd_ex(*base, 2, 64, 4, 128, 128, 2, 0, -1, None, 0, None) == 1
    assert L.gdn2_chunk_fwd_ex(*base, 2, 64, 4, 96, 128, 2, 0, 3, None, 0, None) == 2
    assert L.gdn2_decode_step_ex(*([FAKE] * 8), 2, 2, 128, 128, 0, 8, None) == 1
    assert L.gdn2_decode_step_ex(*([FAKE] * 8), 0, 2, 128, 128, 0, 3, None) == 0
    assert L.gdn2_decode_tokens_ex(*([FAKE] * 7), None, None, FAKE, None, 2, 2, 2, 64, 64, 2,
                                   0, 5, None) == 1


def test_train_pair_error_paths():
    L = _lib.lib()
    base = [FAKE] * 6 + [None, FAKE, None, None]
    # no workspace / too small
    assert L.gdn2_chunk_fwd_train(*base, 2, 64, 4, 128, 128, 2, 0, 0, None, 0, None) == 3
    assert L.gdn2_chunk_fwd_train(*base, 2, 64, 4, 128, 128, 2, 0, 0, FAKE, 100, None) == 3
    # fp32 is not built for the training pair; o is required; unknown layout bits
    assert L.gdn2_chunk_fwd_train(*base, 2, 64, 4, 128, 128, 2, 1, 0, FAKE, 1 << 40, None) == 2
    nob = [FAKE] * 6 + [None, None, None, None]
    assert L.gdn2_chunk_fwd_train(*nob, 2, 64, 4, 128, 128, 2, 0, 0, FAKE, 1 << 40, None) == 1
    assert L.gdn2_chunk_fwd_train(*base, 2, 64, 4, 128, 128, 2, 0, 4, FAKE, 1 << 40, None) == 1
    args = [FAKE] * 6 + [None, FAKE, None] + [FAKE] * 6 + [None, None, None]
    assert L.gdn2_chunk_bwd_saved(*args, 2, 64, 4, 128, 128, 2, 0, 0, None, 0, None) == 3
    assert L.gdn2_chunk_bwd_saved(*args, 2, 64, 4, 96, 128, 2, 0, 0, FAKE, 1 << 40, None) == 2
    assert L.gdn2_chunk_bwd_ex(*args, 2, 64, 4, 128, 128, 2, 0, 8, FAKE, 1 << 40, None) == 1
    assert L.gdn2_chunk_bwd_ex(*args, 2, 64, 4, 128, 128, 2, 0, 3, None, 0, None) == 3


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """A call whose two-phase workspace exceeds the library-held scratch is refused on the
    host (status 3, nothing launched); fp32 has no two-phase path (status 2)."""
    L = _lib.lib()
    cap = int(L.gdn2_noalloc_scratch_bytes())
    assert cap == 128 << 20
    T = 1 << 20
    assert int(L.gdn2_chunk_fwd_workspace_bytes(1, T, 16, 128, 128, 1, 0)) > cap
    args = [FAKE] * 6 + [None, FAKE, None, None]
    assert L.gdn2_chunk_fwd_noalloc(*args, 1, T, 16, 128, 128, 1, 0, 0, None) == 3
    assert b"scratch" in L.gdn2_status_string(3)
    assert L.gdn2_chunk_fwd_noalloc(*args, 1, 64, 2, 64, 64, 1, 1, 0, None) == 2
    assert L.gdn2_chunk_fwd_noalloc(*args, 1, 64, 0, 64, 64, 1, 0, 0, None) == 1


def test_auto_path_rule():
    # "auto" takes the two-phase path only where the fused kernel's workgroups (sequence x
    # head x 64 value columns) number at most a third of the CUs and sequences are long
    from gated_delta_rule_36_amd import uses_split
    need = 1
    assert uses_split(1, 32768, 1, 16, 128, need)            # 32 workgroups
    assert uses_split(2, 8192, 2, 16, 128, need)             # 64
    assert not uses_split(3, 4096, 3, 16, 128, need)         # 96
    assert not uses_split(8, 2048, 8, 16, 128, need)         # the 1.3B-layer batch
    assert not uses_split(1, 79750, 16, 16, 128, need)       # 16 packed sequences
    assert not uses_split(1, 1024, 1, 16, 128, need)         # short
    assert uses_split(1, 4096, 1, 16, 64, need, cus=48)      # 16 workgroups on 48 CUs
    assert not uses_split(1, 32768, 1, 16, 128, 0)           # two-phase path not built
    assert not uses_split(1, 32768, 1, 16, 128, need, value_slice=64)
    assert uses_split(8, 2048, 8, 16, 128, need, path="split")
    assert not uses_split(1, 32768, 1, 16, 128, need, path="fused")
