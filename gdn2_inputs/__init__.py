"""Seeded synthetic inputs for the Gated Delta Rule-2 token mixer.

This module only draws random numbers and rounds them to the run dtype. It holds
none of the recurrence's arithmetic, so both the float64 oracle (through the tests)
and the HIP path consume exactly the same tensors.

Distributions (per (token, head)):
  q, k  ~ N(0, 1), then L2-normalised over the key width and rounded once;
  v     ~ N(0, 1);
  g     = log(alpha) = -0.1 * softplus(N(0, 1)) per key channel (alpha in (0, 1]);
  b, w  = sigmoid(N(0, 1)) per key / value channel;
  optional near-reset tokens: with probability `reset_frac`, every key channel of g
  is set to `reset_logdecay` (-5);
  optional initial state S0 ~ N(0, s0_std^2) in fp32, layout [N, H, d_k, d_v].

Gate domains follow the GDN-2 reading note ("Gated DeltaNet-2: Decoupling Erase and
Write in Linear Attention", §1 summary): alpha in (0,1]^{d_k}, b in [0,1]^{d_k},
w in [0,1]^{d_v}.

Every floating-point array is returned as float32 holding values that are exactly
representable in the run dtype ("bf16" or "fp32"), so that converting to a torch
bfloat16 tensor is exact and the oracle can upcast to float64 exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "CONFIGS",
    "make_scalar_gate",
    "make_block_inputs",
    "round_to_bf16",
    "make_inputs",
    "make_config_inputs",
    "make_decode_inputs",
]

# Named workloads. Seeds are 1000 + position in this table.
CONFIGS = {
    "tiny_fp32": dict(B=1, H=2, T=256, dk=64, dv=64, dtype="fp32", seed=1000),
    "layer1p3b_bf16": dict(B=8, H=16, T=2048, dk=128, dv=128, dtype="bf16", seed=1001),
    "longctx_bf16": dict(B=1, H=16, T=32768, dk=128, dv=128, dtype="bf16", seed=1002,
                         reset_frac=0.1),
    "varlen_bf16": dict(N=16, len_lo=512, len_hi=8192, H=16, dk=128, dv=128, dtype="bf16",
                        seed=1003, s0_std=0.02),
    "decode_bf16": dict(N=256, H=16, dk=128, dv=128, dtype="bf16", seed=1004, steps=1000),
}

RESET_LOGDECAY = -5.0


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 holding the values.

    Works on the IEEE-754 bit pattern: bfloat16 keeps the upper 16 bits of a float32.
    Inputs are finite (no NaN handling needed for the generator's draws).
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32).reshape(f.shape)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def _l2norm_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def _draw_tensors(rng, shape_k, shape_v, dtype, reset_frac):
    """Draw q, k, v, g, b, w in that fixed order (float64), then round once."""
    q = _l2norm_last(rng.standard_normal(shape_k))
    k = _l2norm_last(rng.standard_normal(shape_k))
    v = rng.standard_normal(shape_v)
    g = -0.1 * _softplus(rng.standard_normal(shape_k))
    b = _sigmoid(rng.standard_normal(shape_k))
    w = _sigmoid(rng.standard_normal(shape_v))
    if reset_frac > 0.0:
        mask = rng.random(shape_k[:-1]) < reset_frac  # one draw per (batch, token, head)
        g[mask] = RESET_LOGDECAY
    out = {}
    for name, arr in (("q", q), ("k", k), ("v", v), ("g", g), ("b", b), ("w", w)):
        out[name] = _to_dtype(arr, dtype)
    return out


def make_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, reset_frac=0.0, lengths=None,
                s0_std=None):
    """Inputs for one forward call.

    Fixed-length layout: q, k, g, b are [B, T, H, dk]; v, w are [B, T, H, dv].
    If `lengths` is given (varlen), B must be 1 and T == sum(lengths); the sequences
    are packed back to back and `cu_seqlens` (int32, [N+1]) is returned.
    If `s0_std` is given, an fp32 initial state [N, H, dk, dv] ~ N(0, s0_std^2) is drawn
    after the token tensors; otherwise `s0` is None (zero initial state).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert B == 1 and T == int(lengths.sum())
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
    out = _draw_tensors(rng, (B, T, H, dk), (B, T, H, dv), dtype, reset_frac)
    n_seq = B if lengths is None else len(lengths)
    out["s0"] = None
    if s0_std is not None:
        out["s0"] = (s0_std * rng.standard_normal((n_seq, H, dk, dv))).astype(np.float32)
    out["cu_seqlens"] = cu
    out["dtype"] = dtype
    return out


def varlen_lengths(n, lo, hi, seed):
    """Sequence lengths uniform in [lo, hi], drawn from their own stream (seed, 1)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    return rng.integers(lo, hi + 1, size=n)


def make_config_inputs(name, **overrides):
    """Inputs for one of the named workloads in CONFIGS (forward configs only)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    if "N" in c and "len_lo" in c:
        lengths = varlen_lengths(c["N"], c["len_lo"], c["len_hi"], c["seed"])
        return make_inputs(1, int(lengths.sum()), c["H"], c["dk"], c["dv"], c["dtype"],
                           c["seed"], lengths=lengths, s0_std=c.get("s0_std"))
    return make_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], c["seed"],
                       reset_frac=c.get("reset_frac", 0.0), s0_std=c.get("s0_std"))


def make_decode_inputs(N, H, dk, dv, steps, dtype="bf16", seed=0, s0_std=None):
    """Per-step decode inputs: q, k, g, b are [steps, N, H, dk]; v, w [steps, N, H, dv].

    Same distributions as the forward inputs. `s0` ([N, H, dk, dv] fp32) is drawn last
    when `s0_std` is given.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = _draw_tensors(rng, (steps, N, H, dk), (steps, N, H, dv), dtype, 0.0)
    out["s0"] = None
    if s0_std is not None:
        out["s0"] = (s0_std * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    out["dtype"] = dtype
    return out


def make_block_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, lengths=None):
    """Inputs of the block prologue and epilogue around the mixer.

    Projections xq, xk, xg, xb: [B, T, H, d_k] and xv, xw, o, gate: [B, T, H, d_v], all
    N(0, 1) rounded to the run dtype; conv taps N(0, 1/4) in fp32, [H * d, 4]; decay scale
    0.1 * U(0.5, 1.5) per key channel (fp32); norm weight 1 + 0.1 * N(0, 1) (fp32, [d_v]).
    With `lengths`, B must be 1 and T = sum(lengths); cu_seqlens is returned (else None).
    """
    rng = np.random.default_rng(seed)
    if lengths is not None:
        assert B == 1 and T == int(np.sum(lengths))
    out = {}
    for n, d in (("xq", dk), ("xk", dk), ("xv", dv), ("xg", dk), ("xb", dk), ("xw", dv),
                 ("o", dv), ("gate", dv)):
        out[n] = _to_dtype(rng.normal(size=(B, T, H, d)), dtype)
    for n, d in (("conv_q", dk), ("conv_k", dk), ("conv_v", dv)):
        out[n] = (rng.normal(size=(H * d, 4)) * 0.5).astype(np.float32)
    out["decay_scale"] = (0.1 * rng.uniform(0.5, 1.5, size=H * dk)).astype(np.float32)
    out["norm_weight"] = (1.0 + 0.1 * rng.normal(size=dv)).astype(np.float32)
    out["cu_seqlens"] = (None if lengths is None else
                         np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return out


def make_scalar_gate(shape, dtype="bf16", seed=0):
    """A gate with one value per (token, head): sigmoid(N(0, 1)) of the given leading shape
    (e.g. [B, T, H]), rounded to the run dtype; its own stream (seed, 2)."""
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    return _to_dtype(_sigmoid(rng.standard_normal(shape)), dtype)
