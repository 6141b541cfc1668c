"""ctypes binding of libgdn2.so (the C ABI declared in include/gdn2.h).

Argument marshalling only: shapes and dtypes are checked, outputs are allocated with
torch on the inputs' device, and the call is issued on torch's current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn2.so")
_lib = None

GDN2_BF16 = 0
GDN2_F32 = 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "launch failed"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_SPLIT_MIN_AVG_TOKENS = 1024  # "auto" takes the two-phase path only past this average length
_Z = ctypes.c_size_t


class Gdn2Error(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed with status {status} ({lib().gdn2_status_string(status).decode()})")


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libgdn2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                               "(python -m gated_delta_rule_36_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        L.gdn2_chunk_fwd.argtypes = [_P] * 10 + [_I] * 7 + [_P, _Z, _P]
        L.gdn2_chunk_fwd.restype = _I
        L.gdn2_chunk_fwd_workspace_bytes.argtypes = [_I] * 7
        L.gdn2_chunk_fwd_workspace_bytes.restype = _Z
        L.gdn2_chunk_bwd.argtypes = [_P] * 18 + [_I] * 7 + [_P, _Z, _P]
        L.gdn2_chunk_bwd.restype = _I
        L.gdn2_chunk_bwd_saved.argtypes = [_P] * 18 + [_I] * 8 + [_P, _Z, _P]
        L.gdn2_chunk_bwd_saved.restype = _I
        L.gdn2_chunk_bwd_ex.argtypes = [_P] * 18 + [_I] * 8 + [_P, _Z, _P]
        L.gdn2_chunk_bwd_ex.restype = _I
        L.gdn2_chunk_fwd_train.argtypes = [_P] * 10 + [_I] * 8 + [_P, _Z, _P]
        L.gdn2_chunk_fwd_train.restype = _I
        L.gdn2_chunk_bwd_workspace_bytes.argtypes = [_I] * 7
        L.gdn2_chunk_bwd_workspace_bytes.restype = _Z
        L.gdn2_chunk_fwd_sliced.argtypes = [_P] * 10 + [_I] * 8 + [_P]
        L.gdn2_chunk_fwd_sliced.restype = _I
        L.gdn2_decode_step.argtypes = [_P] * 8 + [_I] * 5 + [_P]
        L.gdn2_decode_step.restype = _I
        L.gdn2_decode_tokens.argtypes = [_P] * 11 + [_I] * 7 + [_P]
        L.gdn2_decode_tokens.restype = _I
        L.gdn2_chunk_fwd_ex.argtypes = [_P] * 10 + [_I] * 8 + [_P, _Z, _P]
        L.gdn2_chunk_fwd_ex.restype = _I
        L.gdn2_chunk_fwd_noalloc.argtypes = [_P] * 10 + [_I] * 8 + [_P]
        L.gdn2_chunk_fwd_noalloc.restype = _I
        L.gdn2_noalloc_scratch_bytes.argtypes = []
        L.gdn2_noalloc_scratch_bytes.restype = _Z
        L.gdn2_decode_step_ex.argtypes = [_P] * 8 + [_I] * 6 + [_P]
        L.gdn2_decode_step_ex.restype = _I
        L.gdn2_decode_tokens_ex.argtypes = [_P] * 11 + [_I] * 8 + [_P]
        L.gdn2_decode_tokens_ex.restype = _I
        L.gdn2_block_prologue.argtypes = [_P] * 10 + [ctypes.c_float] + [_P] * 7 + [_I] * 7 + [_P]
        L.gdn2_block_prologue.restype = _I
        L.gdn2_block_epilogue.argtypes = [_P] * 4 + [ctypes.c_long, _I, _I, _P]
        L.gdn2_block_epilogue.restype = _I
        L.gdn2_status_string.argtypes = [_I]
        L.gdn2_status_string.restype = ctypes.c_char_p
        L.gdn2_version.argtypes = []
        L.gdn2_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return GDN2_BF16
    if dt == torch.float32:
        return GDN2_F32
    raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")


def _check(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


GATE_B_SCALAR = 1  # gate layouts (the C header's GDN2_GATE_* bits)
GATE_W_SCALAR = 2


def _gate_layout(b, w, lead, dk, dv, dt, dev):
    """Gate layout bits from the shapes of b and w: lead + (d,) per channel, lead alone for
    one value per token and head (broadcast over the channels by the kernels)."""
    lay = 0
    for name, t, d, bit in (("b", b, dk, GATE_B_SCALAR), ("w", w, dv, GATE_W_SCALAR)):
        if tuple(t.shape) == tuple(lead):
            _check(name, t, tuple(lead), dt, dev)
            lay |= bit
        else:
            _check(name, t, tuple(lead) + (d,), dt, dev)
    return lay


def workspace_bytes(B, T, H, dk, dv, N, dtype=torch.bfloat16):
    """Device workspace the two-phase chunk forward needs (0: that path is not built)."""
    return int(lib().gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, _dtype_code(dtype)))


def uses_split(B, T, N, H, dv, need, path="auto", value_slice=0, cus=256):
    """Whether chunk_fwd runs the two-phase path (`need`: its workspace bytes, 0 if unbuilt;
    `cus`: compute units of the device).

    "auto" takes it when the fused kernel would leave most of the GPU idle: its workgroups
    (one per sequence, head and 64 value columns) number at most a third of the compute
    units, and the sequences average more than 1024 tokens (shorter ones run as fast fused).
    Measured on MI355X (H = 16, d = 128): 64 workgroups (2 x 8192 tokens) 0.33 ms two-phase
    against 0.54 ms fused; 96 (3 x 4096) 0.34 against 0.27; 512 (16 packed sequences,
    79,750 tokens) 1.35 against 0.83."""
    chains = N * H * max(1, dv // 64)
    few_long = N > 0 and 3 * chains <= cus and B * T > N * _SPLIT_MIN_AVG_TOKENS
    return need > 0 and not value_slice and (path == "split" or (path == "auto" and few_long))


_CUS = {}


def _cu_count(dev) -> int:
    i = dev.index if dev.index is not None else torch.cuda.current_device()
    if i not in _CUS:
        _CUS[i] = torch.cuda.get_device_properties(i).multi_processor_count
    return _CUS[i]


def chunk_fwd(q, k, v, g, b, w, initial_state=None, cu_seqlens=None,
              output_final_state=True, path="auto", value_slice=0, workspace=None):
    """Gated Delta Rule-2 chunkwise forward.

    q, k, g, b: [B, T, H, d_k]; v, w: [B, T, H, d_v] (bf16 or fp32, same dtype, on a HIP
    device); g = log(alpha) <= 0. b or w may instead be [B, T, H]: one gate value per token
    and head, shared by its channels. initial_state: [N, H, d_k, d_v] fp32 or None.
    cu_seqlens: int32 [N+1] on the device (packed batch, B == 1) or None (N = B).
    path: "split" (two-phase: parallel chunk factors into a workspace, then the per-sequence
    recurrence), "fused" (one kernel per sequence, no workspace) or "auto" (split for bf16
    when the fused kernel's workgroups would number at most a third of the compute units
    and sequences average more than 1024 tokens, else fused). value_slice selects the fused
    kernel's value-slice width.
    workspace: optional uint8 device tensor reused across calls (allocated when None).
    Returns (o [B, T, H, d_v] in the input dtype, final_state [N, H, d_k, d_v] fp32 or None).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    if path not in ("auto", "split", "fused"):
        raise ValueError(f"unknown path {path!r}")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("v", v, dv)):
        _check(name, t, (B, T, H, d), dt, dev)
    layout = _gate_layout(b, w, (B, T, H), dk, dv, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on the inputs' device")
        if B != 1:
            raise ValueError("packed (cu_seqlens) inputs must have B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _check("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if value_slice and layout:
        raise ValueError("value_slice takes per-channel gates")
    L = lib()
    need = int(L.gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, code))
    if path == "split" and need == 0:
        raise ValueError("the two-phase path is built for bf16 with d_k, d_v in {64, 128}")
    if value_slice and path == "split":
        raise ValueError("value_slice applies to the fused path")
    # auto: the two-phase path pays where a few long sequences would leave most CUs idle
    # under the fused kernel (its segments run in parallel); otherwise the fused kernel is
    # faster and moves less data
    use_split = uses_split(B, T, N, H, dv, need, path, value_slice, _cu_count(dev))
    if use_split:
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        elif workspace.device != dev:
            raise ValueError("workspace must be on the inputs' device")
    else:
        workspace = None
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    sN = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(initial_state), _ptr(o),
            _ptr(sN), _ptr(cu_seqlens), B, T, H, dk, dv, N, code]
    if value_slice:
        st = L.gdn2_chunk_fwd_sliced(*args, int(value_slice), _stream(dev))
        fn = "gdn2_chunk_fwd_sliced"
    else:
        wsz = workspace.numel() if workspace is not None else 0
        st = L.gdn2_chunk_fwd_ex(*args, layout, _ptr(workspace), wsz, _stream(dev))
        fn = "gdn2_chunk_fwd_ex"
    if st != 0:
        raise Gdn2Error(fn, st)
    return o, sN


class SavedForBackward:
    """What chunk_fwd_train keeps for chunk_bwd: the workspace holding the chunk factors,
    every chunk's entering state and U, and the identity of the inputs it was computed from."""

    def __init__(self, workspace, key):
        self.workspace = workspace
        self.key = key


def _inputs_key(tensors, cu_seqlens):
    return tuple((t.data_ptr(), tuple(t.shape)) for t in tensors) + (
        (None if cu_seqlens is None else (cu_seqlens.data_ptr(), cu_seqlens.numel())),)


def chunk_fwd_train(q, k, v, g, b, w, initial_state=None, cu_seqlens=None,
                    output_final_state=True, workspace=None):
    """chunk_fwd for training (bf16): the same (o, final_state), plus a SavedForBackward that
    lets chunk_bwd(..., saved=...) skip its forward recomputation. The saved workspace (about
    232 KiB per 64-token chunk and head at d = 128) must stay untouched until then."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("v", v, dv)):
        _check(name, t, (B, T, H, d), dt, dev)
    layout = _gate_layout(b, w, (B, T, H), dk, dv, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on the inputs' device")
        if B != 1:
            raise ValueError("packed (cu_seqlens) inputs must have B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _check("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    L = lib()
    need = int(L.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, code))
    if need == 0:
        raise ValueError("the training forward is built for bf16 with d_k, d_v in {64, 128}")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    sN = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    st = L.gdn2_chunk_fwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                _ptr(initial_state), _ptr(o), _ptr(sN), _ptr(cu_seqlens), B, T,
                                H, dk, dv, N, code, layout, _ptr(workspace), workspace.numel(),
                                _stream(dev))
    if st != 0:
        raise Gdn2Error("gdn2_chunk_fwd_train", st)
    key = _inputs_key((q, k, v, g, b, w) + ((initial_state,) if initial_state is not None else ()),
                      cu_seqlens) + (layout,)
    return o, sN, SavedForBackward(workspace, key)


def chunk_bwd(q, k, v, g, b, w, do, initial_state=None, d_final_state=None, cu_seqlens=None,
              workspace=None, saved=None):
    """Gradients of chunk_fwd (bf16).

    do: [B, T, H, d_v] gradient of o (input dtype); d_final_state: [N, H, d_k, d_v] fp32 or
    None. b or w may be scalar gates [B, T, H] (their gradients then have that shape: the sum
    over the channels). Returns (dq, dk, dv, dg, db, dw, d_initial_state): the first six in the
    input dtype and shapes, the last fp32 [N, H, d_k, d_v]. Exact for any decay: chunks past the
    local-gradient kernel's factor range are recomputed by the library's exact kernel.
    saved: the SavedForBackward of a chunk_fwd_train call on these same tensors; the
    forward recomputation is then skipped.
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("v", v, dv), ("do", do, dv)):
        _check(name, t, (B, T, H, d), dt, dev)
    layout = _gate_layout(b, w, (B, T, H), dk, dv, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on the inputs' device")
        if B != 1:
            raise ValueError("packed (cu_seqlens) inputs must have B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check(name, t, (N, H, dk, dv), torch.float32, dev)
    L = lib()
    need = int(L.gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, code))
    if need == 0:
        raise ValueError("the backward is built for bf16 with d_k, d_v in {64, 128}")
    fn, call = "gdn2_chunk_bwd_ex", L.gdn2_chunk_bwd_ex
    if saved is not None:
        key = _inputs_key((q, k, v, g, b, w) + ((initial_state,) if initial_state is not None
                                                else ()), cu_seqlens) + (layout,)
        if key != saved.key:
            raise ValueError("saved was computed from other tensors than these")
        workspace = saved.workspace
        fn, call = "gdn2_chunk_bwd_saved", L.gdn2_chunk_bwd_saved
    elif workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(x) for x in (q, k, v, g, b, w)]
    ds0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    st = call(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
              _ptr(initial_state), _ptr(do), _ptr(d_final_state),
              *(_ptr(x) for x in grads), _ptr(ds0), _ptr(flag), _ptr(cu_seqlens),
              B, T, H, dk, dv, N, code, layout, _ptr(workspace), workspace.numel(), _stream(dev))
    if st != 0:
        raise Gdn2Error(fn, st)
    return (*grads, ds0)


def decode_step(q, k, v, g, b, w, state):
    """One recurrent decode step; `state` [N, H, d_k, d_v] fp32 is updated in place.

    q, k, g, b: [N, H, d_k]; v, w: [N, H, d_v] (b or w may be [N, H]: one value per head).
    Returns o [N, H, d_v] (input dtype).
    """
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("v", v, dv)):
        _check(name, t, (N, H, d), dt, dev)
    layout = _gate_layout(b, w, (N, H), dk, dv, dt, dev)
    _check("state", state, (N, H, dk, dv), torch.float32, dev)
    o = torch.empty((N, H, dv), dtype=dt, device=dev)
    st = lib().gdn2_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                   _ptr(state), _ptr(o), N, H, dk, dv, code, layout,
                                   _stream(dev))
    if st != 0:
        raise Gdn2Error("gdn2_decode_step_ex", st)
    return o


def decode_tokens(q, k, v, g, b, w, state_pool, state_indices=None, commit_len=None,
                  return_step_states=False):
    """L consecutive tokens per sequence against a pool of fp32 states (decode of several
    tokens, or verification of draft tokens).

    q, k, g, b: [N, L, H, d_k]; v, w: [N, L, H, d_v] (b or w may be [N, L, H]: one value
    per token and head); state_pool: [P, H, d_k, d_v] fp32,
    updated in place for the committed prefix; state_indices: int32 [N] (slot per sequence,
    negative to skip) or None (slot n); commit_len: int32 [N] or None (all L tokens).
    Returns (o [N, L, H, d_v], step_states [N, L, H, d_k, d_v] fp32 or None).
    """
    if q.dim() != 4:
        raise ValueError("q must be [N, L, H, d_k]")
    N, L, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(dt)
    for name, t, d in (("q", q, dk), ("k", k, dk), ("g", g, dk), ("v", v, dv)):
        _check(name, t, (N, L, H, d), dt, dev)
    layout = _gate_layout(b, w, (N, L, H), dk, dv, dt, dev)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [P, H, d_k, d_v]")
    P = state_pool.shape[0]
    _check("state_pool", state_pool, (P, H, dk, dv), torch.float32, dev)
    for name, t in (("state_indices", state_indices), ("commit_len", commit_len)):
        if t is not None and (t.dtype != torch.int32 or t.device != dev or tuple(t.shape) != (N,)):
            raise ValueError(f"{name} must be an int32 [N] tensor on the inputs' device")
    o = torch.empty((N, L, H, dv), dtype=dt, device=dev)
    steps = (torch.empty((N, L, H, dk, dv), dtype=torch.float32, device=dev)
             if return_step_states else None)
    st = lib().gdn2_decode_tokens_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                     _ptr(state_pool), _ptr(state_indices), _ptr(commit_len),
                                     _ptr(o), _ptr(steps), N, L, H, dk, dv, P, code, layout,
                                     _stream(dev))
    if st != 0:
        raise Gdn2Error("gdn2_decode_tokens_ex", st)
    return o, steps


def block_prologue(xq, xk, xv, xg, xb, xw, conv_q, conv_k, conv_v, decay_scale, b_max=1.0,
                   cu_seqlens=None, out=None):
    """Projections -> mixer inputs (q, k, v, g, b, w): conv/SiLU/L2-norm branches and gate
    activations in one pass. xq, xk, xg, xb: [B, T, H, d_k]; xv, xw: [B, T, H, d_v];
    conv_*: fp32 [H * d, 4]; decay_scale: fp32 [H * d_k]. out: optional six preallocated
    outputs shaped like xq, xk, xv, xg, xb, xw (written and returned)."""
    B, T, H, dk = xq.shape
    dv = xv.shape[-1]
    dev, dt = xq.device, xq.dtype
    code = _dtype_code(dt)
    for name, t, d in (("xq", xq, dk), ("xk", xk, dk), ("xg", xg, dk), ("xb", xb, dk),
                       ("xv", xv, dv), ("xw", xw, dv)):
        _check(name, t, (B, T, H, d), dt, dev)
    for name, t, shape in (("conv_q", conv_q, (H * dk, 4)), ("conv_k", conv_k, (H * dk, 4)),
                           ("conv_v", conv_v, (H * dv, 4)), ("decay_scale", decay_scale, (H * dk,))):
        _check(name, t, shape, torch.float32, dev)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    ins = (xq, xk, xv, xg, xb, xw)
    if out is None:
        outs = [torch.empty_like(x) for x in ins]
    else:
        outs = list(out)
        if len(outs) != 6:
            raise ValueError("out must hold six tensors (q, k, v, log_alpha, b, w)")
        for name, t, x in zip(("q", "k", "v", "log_alpha", "b", "w"), outs, ins):
            _check(name, t, tuple(x.shape), dt, dev)
    st = lib().gdn2_block_prologue(*(_ptr(x) for x in (xq, xk, xv, xg, xb, xw)), _ptr(conv_q),
                                   _ptr(conv_k), _ptr(conv_v), _ptr(decay_scale), float(b_max),
                                   *(_ptr(x) for x in outs), _ptr(cu_seqlens), B, T, H, dk, dv,
                                   N, code, _stream(dev))
    if st != 0:
        raise Gdn2Error("gdn2_block_prologue", st)
    return tuple(outs)


def block_epilogue(o, gate, weight, out=None):
    """y = RMSNorm(o) * weight * SiLU(gate) over the last axis (d_v); weight fp32 [d_v].
    out: optional preallocated y shaped like o (written and returned)."""
    dv = o.shape[-1]
    _check("gate", gate, tuple(o.shape), o.dtype, o.device)
    _check("weight", weight, (dv,), torch.float32, o.device)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    if out is None:
        y = torch.empty_like(o)
    else:
        _check("out", out, tuple(o.shape), o.dtype, o.device)
        y = out
    st = lib().gdn2_block_epilogue(_ptr(o), _ptr(gate), _ptr(weight), _ptr(y), o.numel() // dv,
                                   dv, _dtype_code(o.dtype), _stream(o.device))
    if st != 0:
        raise Gdn2Error("gdn2_block_epilogue", st)
    return y


class _GatedDeltaRule2(torch.autograd.Function):
    """Autograd wrapper: the training forward keeps the backward's intermediates; the
    backward consumes them (bf16)."""

    @staticmethod
    def forward(ctx, q, k, v, g, b, w, initial_state, cu_seqlens):
        o, sN, saved = chunk_fwd_train(q, k, v, g, b, w, initial_state=initial_state,
                                       cu_seqlens=cu_seqlens)
        ctx.saved = saved
        ctx.has_s0 = initial_state is not None
        ctx.save_for_backward(q, k, v, g, b, w, initial_state, cu_seqlens)
        return o, sN

    @staticmethod
    def backward(ctx, do, dsN):
        q, k, v, g, b, w, s0, cu = ctx.saved_tensors
        do = do.contiguous() if do is not None else torch.zeros_like(v)
        dsN = None if dsN is None else dsN.contiguous()
        dq, dk, dv, dg, db, dw, ds0 = chunk_bwd(q, k, v, g, b, w, do, initial_state=s0,
                                                d_final_state=dsN, cu_seqlens=cu,
                                                saved=ctx.saved)
        ctx.saved = None
        return dq, dk, dv, dg, db, dw, (ds0 if ctx.has_s0 else None), None


def gated_delta_rule2(q, k, v, g, b, w, initial_state=None, cu_seqlens=None):
    """Differentiable GDN-2 mixer (bf16): returns (o, final_state); gradients flow to q, k,
    v, g, b, w and the initial state through the library's backward."""
    return _GatedDeltaRule2.apply(q, k, v, g, b, w, initial_state, cu_seqlens)
