"""Throughput of the fused head + CTC loss forward and backward on one MI355X.

One step = pcx_forward + pcx_backward (dX, dW, db; dX only for the frozen LLM
head) over one synthetic batch already resident in HBM.  The default workload
is the large-vocabulary head-and-loss point of "Pruned CTC for
Memory-Efficient Large-Vocabulary ASR Training" (App. C.2 / Sec. 5.1: M =
16,000 frames, V = 180,000 classes, D = 512, chunk 4096), here with seeded
synthetic inputs of that shape.

Prints one JSON line: frames/s (value), ms per step, the fraction of the
matrix peak reached by the GEMM FLOPs of a step, a roofline entry for the
dominant kernel family (its launches event-timed inside the timed region,
where no other launch carries events), the per-family times and the HBM
rates of the DP and normalizer passes (from one untimed step with every
family event-timed, which picks the dominant one), the library workspace,
and the CPU FP64 oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"f32": 157.3e12, "bf16": 2.5e15}  # MI355X dense matrix peaks, FLOP/s
HBM_PEAK = 8.0e12
PROFILES = os.path.join(ROOT, "profiles")
GEMM_SRC = os.path.join(ROOT, "vocabulary_ctc_loss_amd", "csrc", "pcx_gemm.hip")

# Kernel families whose work is a slice of the head GEMMs: FLOPs per step.
GEMM_KERNELS = ("fwd_gemm_lse", "bwd_recompute_dz", "dx_gemm", "dw_gemm")
# The CTC recursions: per (frame, extended-label state) each writes its FP64
# value (alpha, beta: 2 x 8 B) and reads one fp32 emission (2 x 4 B).
DP_KERNEL = "ctc_alpha_beta"
DP_BYTES_PER_STATE = 24
# Memory-bound passes beside the GEMMs, with their algorithmic bytes per step:
#   ctc_alpha_beta  24 B per (frame, extended-label state), as above;
#   lambda          the M x (vocabulary spans) FP64 (max, sum) partials read
#                   (16 B each), lambda written in FP64 and fp32 (12 B/frame);
#   scores          Zsel read and S written in place (K x M fp32 each), lambda
#                   read (8 B/frame);
#   occupancy       alpha and beta read (16 B/state), S read (4 B/state), the
#                   occupancy written (4 B/state), g written (8 B/frame).
def pass_bytes(bt, K, nspan):
    L = np.diff(bt.tgt_off).astype(np.int64)
    states = int(np.sum(bt.frame_counts.astype(np.int64) * (2 * L + 1)))
    return {
        DP_KERNEL: DP_BYTES_PER_STATE * states,
        "lambda": bt.M * (16 * nspan + 12),
        "scores": bt.M * (8 * K + 8),
        "occupancy": 24 * states + 8 * bt.M,
    }


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="v180k",
                   choices=["tiny", "v500", "v5k", "v180k", "llm152k"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-utts", type=int, default=3)
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain device copy of known size (HBM counter calibration)")
    return p.parse_args()


def copy_probe():
    """A plain 1 GiB device-to-device copy, repeated, as the reference for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 28  # fp32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))


def gemm_flops_per_step(bt):
    # forward projection + backward recompute + dX (+ dW): 2 M V D each
    n = 3 if not bt.want_dW else 4
    return n * 2.0 * bt.M * bt.V * bt.D


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source."""
    path = os.path.join(PROFILES, "%s_%s_pmc.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if d.get("source_sha256") != sha:
            return None
        return d.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(bt, n_utts):
    import oracle
    import workloads
    idx = list(range(min(n_utts, bt.N)))
    sb = workloads.sample_utterances(bt, idx)
    t0 = time.perf_counter()
    oracle.pcx(sb.X, sb.W, sb.b, sb.frame_counts, sb.tgt_off, sb.tgt, sb.blank, grad=1.0,
               want_dW=sb.want_dW, want_db=sb.want_db)
    dt = time.perf_counter() - t0
    return {"value": sb.M / dt, "unit": "frames/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d utterance(s) of %s (%d frames) through the full V=%d, D=%d head; "
                      "loss + dX%s in FP64, %.1f s wall" % (
                          len(idx), bt.name, sb.M, bt.V, bt.D,
                          " + dW + db" if sb.want_dW else "", dt)}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: pcx has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads
    from vocabulary_ctc_loss_amd import Context

    dev = torch.device("cuda:0")
    bt = workloads.make(args.workload, seed=args.seed)
    dt = torch.float32 if bt.dtype == "f32" else torch.bfloat16
    X = torch.from_numpy(bt.X).to(dev).to(dt)
    W = torch.from_numpy(bt.W).to(dev).to(dt)
    b = torch.from_numpy(bt.b).to(dev).to(dt) if bt.b is not None else None
    off = torch.from_numpy(bt.tgt_off).to(dev)
    tgt = torch.from_numpy(bt.tgt).to(dev)
    fc = torch.from_numpy(bt.frame_counts).to(dev)
    dX = torch.empty_like(X)
    dW = torch.empty_like(W) if bt.want_dW else None
    db = torch.empty_like(b) if (bt.want_db and b is not None) else None
    stream = torch.cuda.current_stream()
    ctx = Context()

    def step():
        ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk, stream=stream)
        ctx.backward(1.0, dX, dW, db, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # One untimed step with every kernel family bracketed by events: the
    # per-family breakdown, and the dominant family.
    ctx.profile_enable(True)
    ctx.profile_mask(None)
    ctx.profile_reset()
    step()
    torch.cuda.synchronize()
    breakdown = ctx.profile_read()
    dom = max(breakdown, key=lambda k: breakdown[k][0])
    # Timed region: only the dominant family's launches carry events (two
    # event records per launch; bracketing every launch would add about 2%).
    ctx.profile_mask([dom])
    ctx.profile_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    prof = ctx.profile_read()
    ctx.profile_enable(False)
    info = ctx.info

    ms = 1e3 * t / args.steps
    frames_per_s = bt.M * args.steps / t
    peak = PEAK[bt.dtype]
    fused_frac = gemm_flops_per_step(bt) / (t / args.steps) / peak
    # the dominant kernel's event time over the timed region
    dom_ms, dom_n = prof[dom]
    if dom in GEMM_KERNELS:
        flops_per_launch = 2.0 * bt.M * bt.V * bt.D * args.steps / max(dom_n, 1)
        achieved = flops_per_launch / (dom_ms / dom_n / 1e3)
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": traffic_from_profiles(dom, bt.name)}
    elif dom == DP_KERNEL:
        L = np.diff(bt.tgt_off).astype(np.int64)
        states = int(np.sum(bt.frame_counts.astype(np.int64) * (2 * L + 1)))
        achieved = DP_BYTES_PER_STATE * states * args.steps / (dom_ms / 1e3)
        roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": achieved / HBM_PEAK,
                "traffic": traffic_from_profiles(dom, bt.name)}
    else:
        roof = {"bound": "alu", "achieved": None, "peak": None, "unit": None, "frac": None,
                "traffic": None}
    # per-family times of the profiled (untimed) step
    kernels = {k: {"ms_per_step": v[0], "launches_per_step": v[1]}
               for k, v in breakdown.items() if v[1]}
    # achieved HBM rate of the DP and normalizer passes (same step)
    hbm_passes = {}
    for k, nbytes in pass_bytes(bt, info["K"], info["lse_spans"]).items():
        if k in breakdown and breakdown[k][1]:
            sec = breakdown[k][0] / 1e3
            hbm_passes[k] = {"bytes_per_step": nbytes, "ms_per_step": 1e3 * sec,
                             "achieved_GBps": nbytes / sec / 1e9,
                             "frac": nbytes / sec / HBM_PEAK}
    out = {
        "metric": "frames/s fused head+CTC fwd+bwd (V=180k,M=16k,D=512); % MFMA peak",
        "value": frames_per_s,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": bt.dtype,
        "data": "synthetic",
        "config": {"workload": bt.name, "M": bt.M, "V": bt.V, "D": bt.D, "N": bt.N,
                   "chunk": bt.chunk, "K": info["K"], "blank": bt.blank,
                   "grads": "dX" + (",dW,db" if bt.want_dW else "")},
        "pct_mfma_peak": 100.0 * fused_frac,
        "gemm_flops_per_step": gemm_flops_per_step(bt),
        "workspace_GiB": info["workspace_bytes"] / 2**30,
        "roofline": dict(kernel=dom, **roof),
        "kernels": kernels,
        "hbm_passes": hbm_passes,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(bt, args.cpu_sample_utts)
    ctx.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
