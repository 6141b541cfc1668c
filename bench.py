"""Benchmark: GDN-2 chunkwise forward tokens/s on one MI355X, with roofline fractions.

A step is one gdn2_chunk_fwd call over the 1.3B-layer workload (B=8, H=16, T=2048,
d_k = d_v = 128, bf16 inputs, fp32 state, zero initial state), inputs resident in HBM;
with the path chunk_fwd's "auto" picks (the pipelined kernel at this shape; where the two-phase
path is picked, its two launches are timed together as one call).
Prints ONE JSON line. Also reports (as extra fields) the recurrent decode step on the
decode workload (256 sequences x 16 heads, fp32 128x128 states) and a CPU baseline: the
float64 oracle timed on a bounded sample of the forward workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-block]
                    [--path auto|split|fused] [--workload layer1p3b|longctx|varlen]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN-2 chunk-fwd tokens/s (H=16,d=128,bf16) + % MFMA/HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
NAMES = ("q", "k", "v", "g", "b", "w")


def measured_record(key):
    """The committed rocprofv3 counter record of a workload (profiles/counters.json), or None
    when a kernel's sources changed since the counters were taken (digest mismatch) or no
    record exists."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            rec = json.load(f)[key]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    h = hashlib.sha256()
    for name in rec["sources"]:
        with open(os.path.join(ROOT, "gated_delta_rule_36_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return rec if h.hexdigest() == rec["source_sha256"] else None


def measured_traffic(key):
    """HBM bytes per call from the committed counter record (summed over the call's
    kernels), or None (see measured_record)."""
    rec = measured_record(key)
    return None if rec is None else rec["traffic_bytes"]


def fwd_bytes(B, T, H, dk, dv, N, elt=2, read_s0=False):
    """Algorithmic HBM bytes of one forward call: read q,k,g,b,v,w once, write o once,
    write the fp32 final state (and read the initial one if given)."""
    tok = B * T * H
    b = tok * (4 * dk + 2 * dv) * elt + tok * dv * elt + N * H * dk * dv * 4
    if read_s0:
        b += N * H * dk * dv * 4
    return b


def fwd_flops(B, T, H, dk, dv, C=64):
    """Useful dense flops of the chunk form per call (triangular halves counted once):
    A, P, W (d_k wide) and U~, P U (d_v wide) over the causal C x C half; W S, Q S, K^T U
    (d_k x d_v per token); the UT transform ~C^2/3 per token."""
    tok = B * T * H
    tri = (C + 1) / 2.0  # average causal row length
    per_tok = 2 * tri * dk * 3 + 2 * tri * dv * 2 + 2 * dk * dv * 3 + C * C / 3.0
    return tok * per_tok


def bwd_bytes(B, T, H, dk, dv, N, elt=2):
    """Algorithmic HBM bytes of one backward call: read q, k, g, b, v, w and do once, write
    the six input gradients once, and the fp32 initial-state gradient."""
    tok = B * T * H
    return tok * (4 * dk + 3 * dv) * elt + tok * (4 * dk + 2 * dv) * elt + N * H * dk * dv * 4


def decode_bytes(N, H, dk, dv, elt=2):
    return N * H * (2 * dk * dv * 4 + (4 * dk + 2 * dv) * elt + dv * elt)


def _oracle_shard(arrays):
    """One worker's share of the CPU baseline: the oracle over a block of sequences x heads.
    Returns the token-heads it covered (a shard holds only some of the heads of its tokens,
    so tokens are counted by dividing the sum over shards by H)."""
    from oracle import gdn2_forward
    gdn2_forward(*arrays)
    return arrays[0].shape[0] * arrays[0].shape[1] * arrays[0].shape[2]


def _oracle_shard_errors(args):
    """Parity of one shard: the oracle over it against the GPU's o and final state for the
    same (sequence, heads); returns (max|o - ref|, max|ref o|, max|S - ref|, max|ref S|)."""
    from oracle import gdn2_forward
    arrays, o_gpu, s_gpu = args
    o_ref, s_ref = gdn2_forward(*arrays)
    return (float(np.max(np.abs(o_gpu - o_ref))), float(np.max(np.abs(o_ref))),
            float(np.max(np.abs(s_gpu - s_ref))), float(np.max(np.abs(s_ref))))


def cpu_baseline(x, workers=None, gpu_out=None):
    """The float64 oracle (gdn2_forward, unchanged) over the whole forward workload, sharded
    by (sequence, block of heads) over a process pool of up to 16 host cores; the pool is
    started and warmed before the timed region."""
    import multiprocessing as mp
    B, T, H, dk = x["q"].shape
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    hsplit = max(1, min(H, workers // B)) if workers > B else 1
    hb = (H + hsplit - 1) // hsplit
    shards = [tuple(np.ascontiguousarray(x[n][bi:bi + 1, :, h0:h0 + hb]) for n in NAMES)
              for bi in range(B) for h0 in range(0, H, hb)]
    ctx = mp.get_context("spawn")  # the parent has initialised the GPU: no fork
    with ctx.Pool(min(workers, len(shards))) as pool:
        pool.map(_oracle_shard, [tuple(a[:, :4] for a in sh) for sh in shards])  # warm-up
        t0 = time.perf_counter()
        token_heads = sum(pool.map(_oracle_shard, shards))
        dt = time.perf_counter() - t0
        used = min(workers, len(shards))
        parity = None
        if gpu_out is not None:  # untimed: the same shards again, against the GPU's results
            o_gpu, s_gpu = gpu_out
            jobs = [(sh, o_gpu[bi:bi + 1, :, h0:h0 + hb], s_gpu[bi:bi + 1, h0:h0 + hb])
                    for sh, (bi, h0) in zip(shards, [(bi, h0) for bi in range(B)
                                                     for h0 in range(0, H, hb)])]
            errs = pool.map(_oracle_shard_errors, jobs)
            parity = {"max_rel_err_o": max(e[0] for e in errs) / max(e[1] for e in errs),
                      "max_rel_err_S": max(e[2] for e in errs) / max(e[3] for e in errs)}
        pool.close()  # the workers exit on their own (no SIGTERM from the context's exit)
        pool.join()
    done = token_heads / H  # tokens: every shard holds hb of the H heads of its tokens
    res = {"value": round(done / dt, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
            "tokens": int(round(done)), "seconds": round(dt, 3),
            "sample": f"the whole workload ({B} sequences x {T} tokens x {H} heads) in "
                      f"{len(shards)} shards of {hb} heads (float64 token loop, {dt:.1f} s "
                      f"wall on {used} processes)",
            "cpu": platform.processor() or platform.machine()}
    return res, parity


def provenance():
    """The git commit of the tree, and a digest of the library's sources and header, which
    identifies the build either way. Where the tree is not a checkout (a copy without its git
    metadata), the commit is the one the library was built from, taken only while that build
    record's source digest still matches the sources."""
    import subprocess
    from gated_delta_rule_36_amd.build import BUILD_INFO, source_digest
    digest = source_digest()
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        sha = r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        sha = None
    out = {"git_sha": sha or None, "source_sha256": digest}
    if not sha:
        try:
            with open(BUILD_INFO) as f:
                info = json.load(f)
        except (OSError, ValueError):
            info = None
        if info and info.get("source_sha256") == digest and info.get("git_sha"):
            out["git_sha"] = info["git_sha"]
            out["git_sha_from"] = "build record"
            out["library_sources_committed"] = info.get("library_sources_committed")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # untimed calls first: the GPU's clocks need about 100 ms of sustained work to settle
    # (10 warm-up calls left the forward about 5% slower than 400 did)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context forward measurement")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length forward measurement")
    ap.add_argument("--no-scalar-gates", action="store_true",
                    help="skip the scalar-gate forward measurement")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the block prologue / epilogue measurement")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--path", choices=("auto", "split", "fused"), default="auto",
                    help="chunk-forward path: two-phase (split), single fused kernel, or auto "
                         "(as chunk_fwd chooses)")
    ap.add_argument("--workload", choices=("layer1p3b", "longctx", "varlen"),
                    default="layer1p3b",
                    help="layer1p3b (the reported metric), or one of the other synthetic "
                         "workloads for information: B1 H16 T32768 with 10%% near-resets, or "
                         "16 packed sequences of 512..8192 tokens")
    ap.add_argument("--value-slice", type=int, default=0)
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="before the timed region, run a plain device copy of this many MiB "
                         "(3 times) so hardware byte counters can be calibrated against it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on exactly one GPU (got --gpus {args.gpus}); the chunk "
              "forward shards by sequence/head/value-column with no exchange, but multi-GPU "
              "runs are not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_36_amd as G
    from gdn2_inputs import CONFIGS, make_config_inputs, make_decode_inputs

    dev = torch.device("cuda:0")

    def settle(fn, seconds=0.1):
        """Untimed calls of fn (at least 3) for about `seconds` of wall time, so that the
        timed calls after them run at the GPU's settled clocks."""
        n, t_end = 0, time.perf_counter() + seconds
        while n < 3 or time.perf_counter() < t_end:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    cfg = args.workload + "_bf16"
    x = make_config_inputs(cfg)
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    t = {n: torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in NAMES}
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"]).to(dev)
    s0 = None if x["s0"] is None else torch.from_numpy(x["s0"]).to(dev)
    N = B if cu is None else cu.numel() - 1
    torch.cuda.synchronize()

    if args.copy_calib_mb > 0:
        src = torch.empty(args.copy_calib_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ws_bytes = G.workspace_bytes(B, T, H, dk, dv, N)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    use_split = G.uses_split(B, T, N, H, dv, ws_bytes, args.path, args.value_slice, cus)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if use_split else None

    def step():
        return G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0, cu_seqlens=cu,
                           value_slice=args.value_slice,
                           path="split" if use_split else "fused", workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # then untimed calls for at least 100 ms of sustained work, whatever W is: a few warm-up
    # calls leave the clocks still ramping (5 of them timed the forward about 30% slower)
    t_settle = time.perf_counter()
    settle(step)
    settle_s = time.perf_counter() - t_settle
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_per_step = wall * 1e3 / K
    tokens = B * T
    value = tokens * K / wall
    nbytes = fwd_bytes(B, T, H, dk, dv, N, read_s0=s0 is not None)
    flops = fwd_flops(B, T, H, dk, dv)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    if use_split:
        kernel = (f"gdn2_prep_kernel<{dk},{dv}> + gdn2_state_kernel<{dk},{dv},NV> "
                  "(the launches of one call; a sequence cut into segments adds the "
                  "transfer pass and the combine kernel between them)")
        tkey = f"chunk_fwd_split_{cfg}"
    elif args.value_slice:
        kernel = f"gdn2_chunk_kernel<bf16,{dk},{args.value_slice},0>"
        tkey = None
    else:
        kernel = f"gdn2_fwd_kernel<{dk},0>"
        tkey = f"chunk_fwd_{cfg}"
    path_name = ("two-phase" if use_split else
                 "fused (value slice %d)" % args.value_slice if args.value_slice else "pipelined")
    workloads = {
        "layer1p3b": "GDN-2 chunk forward, 1.3B-layer shape: B=8 H=16 T=2048 d_k=d_v=128 "
                     "C=64, bf16 in/out, fp32 state, zero S0",
        "longctx": "GDN-2 chunk forward, long context: B=1 H=16 T=32768 d_k=d_v=128 C=64, "
                   "10% of (token, head) decays at g=-5, bf16, zero S0",
        "varlen": "GDN-2 chunk forward, packed: 16 sequences of 512..8192 tokens, H=16 "
                  "d_k=d_v=128 C=64, bf16, S0 ~ N(0, 0.02^2)",
    }
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "log-alpha=-0.1*softplus(N(0,1)), b,w=sigmoid(N(0,1)))",
        "config": {"workload": workloads[args.workload], "global_batch": B, "seq_len": T,
                   "sequences": N, "path": path_name,
                   "parallelism": "single GPU"},
        "clock_settle_s": round(settle_s, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(tkey),
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel_ms": round(kern_ms, 4)},
        "mfma": {"useful_flops_per_launch": round(flops),
                 "achieved_tflops": round(flops / (kern_ms * 1e-3) / 1e12, 2),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    rec = measured_record(tkey)
    if rec is not None and "derived" in rec:
        # rocprofv3 counters of the same kernel (profiles/): SQ_VALU_MFMA_BUSY_CYCLES over
        # the GRBM active cycles of the 1024 SIMDs, and the MFMA work the hardware executed
        out["mfma"]["counter_busy_frac"] = round(rec["derived"]["mfma_busy_frac"], 4)
        out["mfma"]["counter_executed_flops_per_launch"] = rec["derived"]["mfma_bf16_flops_executed"]

    if args.workload == "layer1p3b" and not args.no_scalar_gates:
        # the scalar-gate configuration (one b and one w value per token and head), timed
        # right after the headline, at the same clocks
        gen = torch.Generator(device=dev).manual_seed(5)
        sb = torch.sigmoid(torch.randn(B, T, H, generator=gen, device=dev)).to(t["b"].dtype)
        sw = torch.sigmoid(torch.randn(B, T, H, generator=gen, device=dev)).to(t["w"].dtype)
        sg = dict(t, b=sb, w=sw)

        def sstep():
            return G.chunk_fwd(*(sg[n] for n in NAMES), initial_state=s0, cu_seqlens=cu,
                               path="fused")
        settle(sstep)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        for a, b2 in evs:
            a.record()
            sstep()
            b2.record()
        torch.cuda.synchronize()
        sms = float(np.mean([a.elapsed_time(b2) for a, b2 in evs]))
        sbytes = B * T * H * ((3 * dk + dv + dv) * 2 + 2 * 2) + N * H * dk * dv * 4
        out["scalar_gates"] = {
            "workload": "the same forward with scalar b and w ([B, T, H]), pipelined kernel",
            "ms_per_call": round(sms, 4), "tokens_per_s": round(B * T / (sms * 1e-3), 1),
            "algorithmic_bytes": sbytes,
            "hbm_frac": round(sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("chunk_fwd_scalar_gates_layer1p3b_bf16")}

    if not args.no_backward:
        rng = np.random.default_rng(7)
        do = torch.from_numpy(rng.normal(size=(B, T, H, dv)).astype(np.float32)).to(dev)
        do = do.to(torch.bfloat16)
        bws = torch.empty(int(G.lib().gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, 0)),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return G.chunk_bwd(*(t[n] for n in NAMES), do, initial_state=s0, cu_seqlens=cu,
                               workspace=bws)
        bstep()
        settle(bstep)
        KB = max(5, K // 5)
        evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(KB)]
        for a, b2 in evb:
            a.record()
            bstep()
            b2.record()
        torch.cuda.synchronize()
        bms = float(np.mean([a.elapsed_time(b2) for a, b2 in evb]))
        bb = bwd_bytes(B, T, H, dk, dv, N)
        out["backward"] = {
            "workload": "chunk backward on the same workload (gradients of q, k, v, g, b, w "
                        "and the initial state for a random bf16 gradient of o)",
            "ms_per_call": round(bms, 4), "tokens_per_s": round(B * T / (bms * 1e-3), 1),
            "kernels": "factor kernel (backward layout) + forward chain + reverse chain + "
                       "local gradients", "calls_timed": KB,
            "algorithmic_bytes": bb, "achieved_GBs": round(bb / (bms * 1e-3) / 1e9, 1),
            "hbm_frac": round(bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": (measured_traffic("chunk_bwd_layer1p3b_bf16")
                        if args.workload == "layer1p3b" else None)}

        # a training step (on the headline workload): forward then backward. Either the fused
        # forward and a backward that recomputes the forward, or the training forward (keeps
        # the intermediates) and the backward that reuses them.
        def pair_recompute():
            G.chunk_fwd(*(t[n] for n in NAMES), initial_state=s0, cu_seqlens=cu, path="fused")
            bstep()

        def pair_saved():
            _, _, sv = G.chunk_fwd_train(*(t[n] for n in NAMES), initial_state=s0, cu_seqlens=cu,
                                         workspace=bws)
            G.chunk_bwd(*(t[n] for n in NAMES), do, initial_state=s0, cu_seqlens=cu, saved=sv)
        res_t = {}
        pairs = (("recompute", pair_recompute), ("saved", pair_saved))
        for name, fn in (pairs if args.workload == "layer1p3b" else ()):
            settle(fn)
            evt = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(KB)]
            for a, b2 in evt:
                a.record()
                fn()
                b2.record()
            torch.cuda.synchronize()
            res_t[name] = round(float(np.mean([a.elapsed_time(b2) for a, b2 in evt])), 4)
        if res_t:
            out["train_step"] = {
                "workload": "forward + backward on the same workload",
                "ms_fused_forward_then_recomputing_backward": res_t["recompute"],
                "ms_training_forward_then_saved_backward": res_t["saved"],
                "tokens_per_s_saved": round(B * T / (res_t["saved"] * 1e-3), 1)}
        del bws

    if args.workload == "layer1p3b" and not args.no_long:
        # the long-context shape beside the headline (one 32K-token sequence, 16 heads, 10%
        # near-resets; inputs drawn on the device with the same recipe), with the path
        # chunk_fwd's "auto" picks for it: the throughput should stay near the headline's
        gen = torch.Generator(device=dev).manual_seed(3)
        TL = 32768

        def l2n(t):
            return t / t.norm(dim=-1, keepdim=True)
        lq = l2n(torch.randn(1, TL, H, dk, generator=gen, device=dev)).to(torch.bfloat16)
        lk = l2n(torch.randn(1, TL, H, dk, generator=gen, device=dev)).to(torch.bfloat16)
        lv = torch.randn(1, TL, H, dv, generator=gen, device=dev).to(torch.bfloat16)
        lg = -0.1 * torch.nn.functional.softplus(torch.randn(1, TL, H, dk, generator=gen, device=dev))
        reset = torch.rand(1, TL, H, 1, generator=gen, device=dev) < 0.1
        lg = torch.where(reset, torch.full_like(lg, -5.0), lg).to(torch.bfloat16)
        lb = torch.sigmoid(torch.randn(1, TL, H, dk, generator=gen, device=dev)).to(torch.bfloat16)
        lw = torch.sigmoid(torch.randn(1, TL, H, dv, generator=gen, device=dev)).to(torch.bfloat16)
        lws = torch.empty(G.workspace_bytes(1, TL, H, dk, dv, 1), dtype=torch.uint8, device=dev)

        def lstep():
            return G.chunk_fwd(lq, lk, lv, lg, lb, lw, workspace=lws)
        settle(lstep)
        evl = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(10)]
        for a, b2 in evl:
            a.record()
            lstep()
            b2.record()
        torch.cuda.synchronize()
        lms = float(np.mean([a.elapsed_time(b2) for a, b2 in evl]))
        lbytes = fwd_bytes(1, TL, H, dk, dv, 1)
        lbwd_ms = None
        if not args.no_backward:  # the backward on the same sequence (cut into segments too)
            ldo = torch.randn(1, TL, H, dv, generator=gen, device=dev).to(torch.bfloat16)
            lbws = torch.empty(int(G.lib().gdn2_chunk_bwd_workspace_bytes(1, TL, H, dk, dv, 1, 0)),
                               dtype=torch.uint8, device=dev)

            def lbstep():
                return G.chunk_bwd(lq, lk, lv, lg, lb, lw, ldo, workspace=lbws)
            lbstep()
            settle(lbstep)
            evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(5)]
            for a, b2 in evb:
                a.record()
                lbstep()
                b2.record()
            torch.cuda.synchronize()
            lbwd_ms = round(float(np.mean([a.elapsed_time(b2) for a, b2 in evb])), 4)
            del ldo, lbws
        out["long_context"] = {
            "workload": "one sequence of 32768 tokens, H=16, d_k=d_v=128, bf16, 10% near-resets "
                        "(log-alpha=-5); path auto (two-phase, cut into segments)",
            "ms_per_call": round(lms, 4), "tokens_per_s": round(TL / (lms * 1e-3), 1),
            "vs_headline_tokens_per_s": round(TL / (lms * 1e-3) / out["value"], 3),
            "algorithmic_bytes": lbytes,
            "hbm_frac": round(lbytes / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "backward_ms_per_call": lbwd_ms}
        del lq, lk, lv, lg, lb, lw, lws

    if args.workload == "layer1p3b" and not args.no_varlen:
        # the packed workload: 16 sequences of 512..8192 tokens, nonzero initial states,
        # drawn on the device (seeded)
        lens = np.random.default_rng(7).integers(512, 8193, size=16)
        cu_v = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
        TV, NV_ = int(lens.sum()), len(lens)
        gen = torch.Generator(device=dev).manual_seed(7)

        def unit_rows(d):
            x = torch.randn(1, TV, H, d, generator=gen, device=dev)
            return x / x.norm(dim=-1, keepdim=True)
        vq, vk = unit_rows(dk).to(torch.bfloat16), unit_rows(dk).to(torch.bfloat16)
        vv = torch.randn(1, TV, H, dv, generator=gen, device=dev).to(torch.bfloat16)
        vg = (-0.1 * torch.nn.functional.softplus(torch.randn(1, TV, H, dk, generator=gen, device=dev))
              ).to(torch.bfloat16)
        vb = torch.sigmoid(torch.randn(1, TV, H, dk, generator=gen, device=dev)).to(torch.bfloat16)
        vw = torch.sigmoid(torch.randn(1, TV, H, dv, generator=gen, device=dev)).to(torch.bfloat16)
        vs0 = 0.02 * torch.randn(NV_, H, dk, dv, generator=gen, device=dev)
        vws = torch.empty(G.workspace_bytes(1, TV, H, dk, dv, NV_), dtype=torch.uint8, device=dev)

        def vstep():
            return G.chunk_fwd(vq, vk, vv, vg, vb, vw, initial_state=vs0, cu_seqlens=cu_v,
                               workspace=vws)
        settle(vstep)
        evv = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(10)]
        for a, b2 in evv:
            a.record()
            vstep()
            b2.record()
        torch.cuda.synchronize()
        vms = float(np.mean([a.elapsed_time(b2) for a, b2 in evv]))
        vbytes = fwd_bytes(1, TV, H, dk, dv, NV_, read_s0=True)
        out["varlen"] = {
            "workload": f"{NV_} packed sequences of 512..8192 tokens ({TV} in all), H=16, "
                        "d_k=d_v=128, bf16, initial states N(0, 0.02^2); path auto ("
                        + ("two-phase" if G.uses_split(1, TV, NV_, H, dv, 1, "auto", 0, cus)
                           else "fused, longest sequences first") + ")",
            "ms_per_call": round(vms, 4), "tokens_per_s": round(TV / (vms * 1e-3), 1),
            "vs_headline_tokens_per_s": round(TV / (vms * 1e-3) / out["value"], 3),
            "algorithmic_bytes": vbytes,
            "hbm_frac": round(vbytes / (vms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del vq, vk, vv, vg, vb, vw, vs0, vws

    if not args.no_block and args.workload == "layer1p3b":
        # prologue (projections -> q, k, v, g, b, w) and epilogue (gated RMSNorm) at this shape
        gen = torch.Generator(device=dev).manual_seed(11)
        shp = {"xq": dk, "xk": dk, "xv": dv, "xg": dk, "xb": dk, "xw": dv}
        px = {n: torch.randn(B, T, H, d, generator=gen, device=dev).to(torch.bfloat16)
              for n, d in shp.items()}
        taps = [torch.randn(H * d, 4, generator=gen, device=dev) * 0.5 for d in (dk, dk, dv)]
        dsc = torch.full((H * dk,), 0.1, device=dev)
        og = [torch.randn(B, T, H, dv, generator=gen, device=dev).to(torch.bfloat16)
              for _ in range(2)]
        nw = torch.ones(dv, device=dev)

        def timed(fn, reps=20):
            settle(fn)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for a, b2 in ev:
                a.record()
                fn()
                b2.record()
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b2) for a, b2 in ev])) * 1e3
        pout = [torch.empty_like(x) for x in px.values()]  # outputs allocated once, outside
        yout = torch.empty_like(og[0])                       # the timed calls
        pus = timed(lambda: G.block_prologue(*px.values(), *taps, dsc, out=pout))
        eus = timed(lambda: G.block_epilogue(og[0], og[1], nw, out=yout))
        rows = B * T * H
        pbytes = rows * (4 * dk + 2 * dv) * 2 * 2  # each projection read once, each input written
        ebytes = rows * dv * 2 * 3
        out["block"] = {
            "workload": "block prologue (conv/SiLU/L2 norm branches and gate activations) and "
                        "epilogue (RMSNorm with SiLU gate) on the same tokens, bf16",
            "prologue": {"us_per_call": round(pus, 2), "algorithmic_bytes": pbytes,
                         "traffic": measured_traffic("block_prologue_layer1p3b_bf16"),
                         "achieved_GBs": round(pbytes / (pus * 1e-6) / 1e9, 1),
                         "hbm_frac": round(pbytes / (pus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "epilogue": {"us_per_call": round(eus, 2), "algorithmic_bytes": ebytes,
                         "traffic": measured_traffic("block_epilogue_layer1p3b_bf16"),
                         "achieved_GBs": round(ebytes / (eus * 1e-6) / 1e9, 1),
                         "hbm_frac": round(ebytes / (eus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
        del px, og, pout, yout

    if not args.no_decode and args.workload == "layer1p3b":
        cd = CONFIGS["decode_bf16"]
        N, Hd, dkd, dvd = cd["N"], cd["H"], cd["dk"], cd["dv"]
        pool = 8
        d = make_decode_inputs(N, Hd, dkd, dvd, pool, "bf16", seed=cd["seed"], s0_std=0.02)
        td = {n: torch.from_numpy(d[n]).to(dev).to(torch.bfloat16) for n in NAMES}
        states = [torch.from_numpy(d["s0"]).to(dev), torch.from_numpy(d["s0"]).to(dev)]
        res = {}
        for mode in ("one_pool", "two_pools"):
            st = states[0]
            settle(lambda: G.decode_step(*(td[n][0] for n in NAMES), st))
            # one event pair around the consecutive steps: the per-step figure is the
            # stream's throughput, not one launch's latency
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s in range(cd["steps"]):
                st = states[s & 1] if mode == "two_pools" else states[0]
                G.decode_step(*(td[n][s % pool] for n in NAMES), st)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / cd["steps"] * 1e3
            gbs = decode_bytes(N, Hd, dkd, dvd) / (us * 1e-6) / 1e9
            res[mode] = {"us_per_step": round(us, 2), "achieved_GBs": round(gbs, 1),
                         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        out["decode"] = {"workload": f"decode step: N={N} sequences x H={Hd}, d_k=d_v={dkd}, "
                                     f"fp32 state in place, {cd['steps']} consecutive steps",
                         "bytes_per_step": decode_bytes(N, Hd, dkd, dvd),
                         "traffic": measured_traffic("decode_step_n256_h16_bf16"), **res}
        # several tokens per call against the pool (draft verification / multi-token decode)
        Lv = 4
        vt = {n: torch.stack([td[n][s % pool] for s in range(Lv)], dim=1).contiguous()
              for n in NAMES}
        vstate = states[0]
        settle(lambda: G.decode_tokens(*(vt[n] for n in NAMES), vstate))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            G.decode_tokens(*(vt[n] for n in NAMES), vstate)
        e1.record()
        torch.cuda.synchronize()
        vus = e0.elapsed_time(e1) / 50 * 1e3
        vbytes = N * Hd * (2 * dkd * dvd * 4 + Lv * ((4 * dkd + 2 * dvd) * 2 + dvd * 2))
        out["decode"]["tokens_per_call_L4"] = {
            "us_per_call": round(vus, 2), "tokens_per_s": round(N * Lv / (vus * 1e-6), 1),
            "bytes_per_call": vbytes, "achieved_GBs": round(vbytes / (vus * 1e-6) / 1e9, 1),
            "traffic": measured_traffic("decode_tokens_n256_l4_h16_bf16"),
            "hbm_frac": round(vbytes / (vus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "vs_four_single_steps": round(4 * res["one_pool"]["us_per_step"] / vus, 3)}

    if not args.no_cpu and args.workload == "layer1p3b":
        o_last, s_last = step()  # one more call: its outputs are checked against the oracle
        torch.cuda.synchronize()
        gpu_out = (o_last.float().cpu().numpy().astype(np.float64),
                   s_last.cpu().numpy().astype(np.float64))
        out["cpu_baseline"], parity = cpu_baseline(x, gpu_out=gpu_out)
        out["parity"] = {**{k: float(f"{v:.3e}") for k, v in parity.items()},
                         "tolerance": 2e-2, "norm": "normwise: max|x - ref| / max|ref| over "
                         "the whole call's o and final states, float64 oracle"}
    out["provenance"] = provenance()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
