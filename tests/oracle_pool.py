"""Whole-workload parity for the GPU tests: the float64 oracle over every (sequence, head)
chain of a workload, or every decode state, sharded over a pool of host processes and
compared with the GPU's results shard by shard.

The pool is spawned (the test process has initialised the GPU, so no fork) once per test
session and sized to the host's share of cores (at most 16); a worker that dies breaks the
pool with an error rather than a hang. Errors are combined the way
the single-call tests measure them: the normwise max relative error of a tensor is the
largest |gpu - oracle| over all of its shards divided by the largest |oracle|.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

NAMES = ("q", "k", "v", "g", "b", "w")
_POOL = None
_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ProcessPoolExecutor(_WORKERS, mp_context=mp.get_context("spawn"))
        atexit.register(_POOL.shutdown, cancel_futures=True)
    return _POOL


def _forward_shard(job):
    from oracle import gdn2_forward
    arrays, s0, o_gpu, s_gpu = job
    o_ref, s_ref = gdn2_forward(*arrays, s0=s0)
    return (float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0,
            float(np.max(np.abs(o_ref))) if o_ref.size else 0.0,
            float(np.max(np.abs(s_gpu - s_ref))), float(np.max(np.abs(s_ref))))


def _decode_shard(job):
    from oracle import gdn2_decode_steps
    s0, arrays, o_gpu, s_gpu = job
    o_ref, s_ref = gdn2_decode_steps(s0, *arrays)
    return (float(np.max(np.abs(o_gpu - o_ref))), float(np.max(np.abs(o_ref))),
            float(np.max(np.abs(s_gpu - s_ref))), float(np.max(np.abs(s_ref))))


def _combine(errs):
    eo = max(e[0] for e in errs) / max(max(e[1] for e in errs), 1e-30)
    es = max(e[2] for e in errs) / max(max(e[3] for e in errs), 1e-30)
    return {"o": eo, "S": es, "shards": len(errs)}


def forward_errors(x, o_gpu, s_gpu):
    """x: an input dict as make_inputs / make_config_inputs build it ([B, T, H, d] arrays,
    optional cu_seqlens and s0); o_gpu [B, T, H, d_v] and s_gpu [N, H, d_k, d_v] the GPU's
    results on the host. Every chain of every sequence is run by the oracle."""
    B, T, H, dk = x["q"].shape
    cu = x["cu_seqlens"]
    seqs = ([(bi, 0, T) for bi in range(B)] if cu is None
            else [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)])
    hsplit = min(H, max(1, -(-2 * _WORKERS // len(seqs))))
    hb = -(-H // hsplit)
    jobs = []
    for n, (bi, t0, t1) in enumerate(seqs):
        for h0 in range(0, H, hb):
            hs = slice(h0, h0 + hb)
            arrays = tuple(np.ascontiguousarray(x[m][bi:bi + 1, t0:t1, hs]) for m in NAMES)
            s0 = None if x["s0"] is None else np.ascontiguousarray(x["s0"][n:n + 1, hs])
            jobs.append((arrays, s0, np.ascontiguousarray(o_gpu[bi:bi + 1, t0:t1, hs]),
                         np.ascontiguousarray(s_gpu[n:n + 1, hs])))
    # longest shards first so the pool's tail is short
    jobs.sort(key=lambda j: -j[0][0].shape[1] * j[0][0].shape[2])
    return _combine(list(_pool().map(_forward_shard, jobs)))


def decode_errors(s0, x, o_gpu, s_gpu, seqs_per_shard=8):
    """s0 [N, H, d_k, d_v]; x: [steps, N, H, d] step inputs; o_gpu [steps, N, H, d_v] and
    s_gpu (the states after the last step) from the GPU. Every state is run by the oracle."""
    N = s0.shape[0]
    jobs = []
    for n0 in range(0, N, seqs_per_shard):
        ns = slice(n0, n0 + seqs_per_shard)
        jobs.append((np.ascontiguousarray(s0[ns]),
                     tuple(np.ascontiguousarray(x[m][:, ns]) for m in NAMES),
                     np.ascontiguousarray(o_gpu[:, ns]), np.ascontiguousarray(s_gpu[ns])))
    return _combine(list(_pool().map(_decode_shard, jobs)))
