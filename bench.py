"""Throughput of the fused head + CTC loss forward and backward on one MI355X.

One step = pcx_forward + pcx_backward (dX, dW, db; dX only for the frozen LLM
head) over one synthetic batch already resident in HBM.  The default workload
is the large-vocabulary head-and-loss point of "Pruned CTC for
Memory-Efficient Large-Vocabulary ASR Training" (App. C.2 / Sec. 5.1: M =
16,000 frames, V = 180,000 classes, D = 512, chunk 4096), here with seeded
synthetic inputs of that shape.

Prints one JSON line: frames/s (value), ms per step (mean over the timed
steps, and their median / min / max from per-step device events), the
fraction of the matrix peak reached by the GEMM FLOPs of a step, a roofline
entry for the dominant kernel family (its launches event-timed inside the
timed region, where no other launch carries events), the per-family times
and the HBM rates of the DP and normalizer passes (from one untimed step with
every family event-timed, which picks the dominant one; with the counter
bytes of the committed rocprofv3 summaries beside the algorithmic ones), the
library workspace, and the CPU FP64 oracle timed on a bounded sample of the
same workload.  The other workloads (V = 500, 5000 and the bf16 LLM head)
follow in `extra_workloads`, each with its own steps, peak fraction and
dominant-kernel roofline, and `beam` times the finite-beam objective at the
pages' training beam (100) beside the exact one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
CSRC = os.path.join(ROOT, "vocabulary_ctc_loss_amd", "csrc")
GEMM_SRC = os.path.join(CSRC, "pcx_gemm.hip")
CTC_SRC = os.path.join(CSRC, "pcx_ctc.hip")
# source file of each kernel family (counter summaries are valid while it
# is unchanged)
KERNEL_SRC = {"fwd_gemm_lse": GEMM_SRC, "bwd_recompute_dz": GEMM_SRC, "dx_gemm": GEMM_SRC,
              "dw_gemm": GEMM_SRC, "lambda": GEMM_SRC, "scores": GEMM_SRC,
              "ctc_alpha_beta": CTC_SRC, "occupancy": CTC_SRC, "ctc_viterbi": CTC_SRC,
              "beam_mask": CTC_SRC}

# Kernel families whose work is a slice of the head GEMMs: FLOPs per step.
GEMM_KERNELS = ("fwd_gemm_lse", "bwd_recompute_dz", "dx_gemm", "dw_gemm")
# The CTC recursions: per (frame, extended-label state) each writes its value
# (alpha, beta: 2 x 8 B, an fp32 mantissa and an int32 exponent); per (frame,
# distinct class of the utterance, blank included) each reads the fp32
# emission once (2 x 4 B: the states of one class share it).
DP_KERNEL = "ctc_alpha_beta"
DP_BYTES_PER_STATE = 16
DP_BYTES_PER_CLASS = 8


# Memory-bound passes beside the GEMMs, with their algorithmic bytes per step:
#   ctc_alpha_beta  24 B per (frame, extended-label state), as above (with a
#                   finite beam one more byte per state: the arc mask read);
#   lambda          the M x (vocabulary spans) FP64 (max, sum) partials read
#                   (16 B each), lambda written in FP64 and fp32 (12 B/frame);
#   scores          Zsel read and S written in place (K x M fp32 each), lambda
#                   read (8 B/frame);
#   occupancy       alpha and beta read (16 B/state), the occupancy written
#                   (4 B per frame and distinct class of the utterance, blank
#                   included), g written (8 B/frame);
#   ctc_viterbi     as ctc_alpha_beta (best prefix / suffix scores);
#   beam_mask       the two best-score tables read (16 B/state), the emission
#                   (4 B per frame and class), the arc mask written (1 B/state).
def pass_bytes(bt, K, nspan, pruned=False):
    L = np.diff(bt.tgt_off).astype(np.int64)
    states = int(np.sum(bt.frame_counts.astype(np.int64) * (2 * L + 1)))
    classes = sum(int(t) * (len(np.unique(bt.tgt[bt.tgt_off[n]:bt.tgt_off[n + 1]])) + 1)
                  for n, t in enumerate(bt.frame_counts))
    out = {
        DP_KERNEL: (DP_BYTES_PER_STATE + (2 if pruned else 0)) * states
                   + DP_BYTES_PER_CLASS * classes,
        "lambda": bt.M * (16 * nspan + 12),
        "scores": bt.M * (8 * K + 8),
        "occupancy": 16 * states + 4 * classes + 8 * bt.M,
    }
    if pruned:
        out["ctc_viterbi"] = DP_BYTES_PER_STATE * states + DP_BYTES_PER_CLASS * classes
        out["beam_mask"] = 17 * states + 4 * classes
    return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="v180k",
                   choices=["tiny", "v500", "v5k", "v180k", "llm152k"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--beam", type=float, default=math.inf,
                   help="alignment beam of the headline workload (default: exact)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="headline workload only (no extra workloads, no beam block)")
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


def counters_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source."""
    path = os.path.join(PROFILES, "%s_%s_pmc.json" % (kernel, workload))
    src = KERNEL_SRC.get(kernel)
    if not os.path.exists(path) or src is None:
        return None
    try:
        d = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if d.get("source_sha256") != sha:
            return None
        return d.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
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
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d utterance(s) of %s (%d frames) through the full V=%d, D=%d head; "
                      "loss + dX%s in FP64, %.1f s wall" % (
                          len(idx), bt.name, sb.M, bt.V, bt.D,
                          " + dW + db" if sb.want_dW else "", dt)}


class Run:
    """One workload resident on the GPU, with its own context."""

    def __init__(self, name, seed):
        import torch

        import workloads
        from vocabulary_ctc_loss_amd import Context
        dev = torch.device("cuda:0")
        self.bt = bt = workloads.make(name, seed=seed)
        dt = torch.float32 if bt.dtype == "f32" else torch.bfloat16
        self.X = torch.from_numpy(bt.X).to(dev).to(dt)
        self.W = torch.from_numpy(bt.W).to(dev).to(dt)
        self.b = torch.from_numpy(bt.b).to(dev).to(dt) if bt.b is not None else None
        self.off = torch.from_numpy(bt.tgt_off).to(dev)
        self.tgt = torch.from_numpy(bt.tgt).to(dev)
        self.fc = torch.from_numpy(bt.frame_counts).to(dev)
        self.dX = torch.empty_like(self.X)
        self.dW = torch.empty_like(self.W) if bt.want_dW else None
        self.db = torch.empty_like(self.b) if (bt.want_db and self.b is not None) else None
        self.stream = torch.cuda.current_stream()
        self.ctx = Context()

    def step(self):
        c, bt = self.ctx, self.bt
        c.forward(self.X, self.W, self.b, self.off, self.tgt, self.fc, bt.blank, bt.chunk,
                  stream=self.stream)
        c.backward(1.0, self.dX, self.dW, self.db, stream=self.stream)

    def step_times(self, steps, warmup):
        """Per-step times (ms) of `steps` steps after `warmup` untimed ones,
        one event pair around each step, nothing else timed."""
        import torch
        for _ in range(warmup):
            self.step()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for a, e in evs:
            a.record(self.stream)
            self.step()
            e.record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(e) for a, e in evs]

    def measure(self, steps, warmup, beam=math.inf):
        """Warm-up, one untimed profiled step (per-family breakdown, dominant
        family), then `steps` timed steps with only the dominant family's
        launches event-timed and one event pair around each step."""
        import torch
        bt, ctx = self.bt, self.ctx
        ctx.set_beam(beam)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ctx.profile_enable(True)
        ctx.profile_mask(None)
        ctx.profile_reset()
        self.step()
        torch.cuda.synchronize()
        breakdown = ctx.profile_read()
        dom = max(breakdown, key=lambda k: breakdown[k][0])
        ctx.profile_mask([dom])
        ctx.profile_reset()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, e in evs:
            a.record(self.stream)
            self.step()
            e.record(self.stream)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        prof = ctx.profile_read()
        ctx.profile_enable(False)
        per_step = sorted(a.elapsed_time(e) for a, e in evs)
        info = ctx.info
        peak = PEAK[bt.dtype]
        dom_ms, dom_n = prof[dom]
        if dom in GEMM_KERNELS:
            flops_per_launch = 2.0 * bt.M * bt.V * bt.D * steps / max(dom_n, 1)
            achieved = flops_per_launch / (dom_ms / dom_n / 1e3)
            roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                    "unit": "TFLOP/s", "frac": achieved / peak,
                    "traffic": counters_from_profiles(dom, bt.name)}
        elif dom == DP_KERNEL:
            nbytes = pass_bytes(bt, info["K"], info["lse_spans"], not math.isinf(beam))[dom]
            achieved = nbytes * steps / (dom_ms / 1e3)
            roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK,
                    "traffic": counters_from_profiles(dom, bt.name)}
        else:
            roof = {"bound": "alu", "achieved": None, "peak": None, "unit": None,
                    "frac": None, "traffic": None}
        kernels = {k: {"ms_per_step": v[0], "launches_per_step": v[1]}
                   for k, v in breakdown.items() if v[1]}
        hbm_passes = {}
        for k, nbytes in pass_bytes(bt, info["K"], info["lse_spans"],
                                    not math.isinf(beam)).items():
            if k in breakdown and breakdown[k][1]:
                sec = breakdown[k][0] / 1e3
                hbm_passes[k] = {"bytes_per_step": nbytes, "ms_per_step": 1e3 * sec,
                                 "achieved_GBps": nbytes / sec / 1e9,
                                 "frac": nbytes / sec / HBM_PEAK}
                cb = counters_from_profiles(k, bt.name) if math.isinf(beam) else None
                if cb is not None:
                    hbm_passes[k]["counter_bytes_per_step"] = cb * breakdown[k][1]
        return {
            "t": t, "steps": steps, "info": info, "dom": dom, "roof": roof,
            "kernels": kernels, "hbm_passes": hbm_passes,
            "ms_per_step": 1e3 * t / steps,
            "ms_per_step_stats": {"median": float(np.median(per_step)),
                                  "min": per_step[0], "max": per_step[-1]},
            "pct_mfma_peak": 100.0 * gemm_flops_per_step(bt) / (t / steps) / peak,
        }

    def close(self):
        self.ctx.close()


def config_of(bt, info):
    return {"workload": bt.name, "M": bt.M, "V": bt.V, "D": bt.D, "N": bt.N,
            "chunk": bt.chunk, "K": info["K"], "blank": bt.blank,
            "grads": "dX" + (",dW,db" if bt.want_dW else "")}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: pcx has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    head = Run(args.workload, args.seed)
    bt = head.bt
    r = head.measure(args.steps, args.warmup, beam=args.beam)
    info = r["info"]
    out = {
        "metric": "frames/s fused head+CTC fwd+bwd (V=180k,M=16k,D=512); % MFMA peak",
        "value": bt.M * args.steps / r["t"],
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "ms_per_step_stats": r["ms_per_step_stats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": bt.dtype,
        "data": "synthetic",
        "config": dict(config_of(bt, info),
                       beam=None if math.isinf(args.beam) else args.beam),
        "pct_mfma_peak": r["pct_mfma_peak"],
        "gemm_flops_per_step": gemm_flops_per_step(bt),
        "workspace_GiB": info["workspace_bytes"] / 2**30,
        "roofline": dict(kernel=r["dom"], **r["roof"]),
        "kernels": r["kernels"],
        "hbm_passes": r["hbm_passes"],
    }
    if not args.no_extra:
        # the finite-beam objective at the pages' training beam, beside the
        # exact headline: the extra Viterbi and arc-mask passes
        rb = head.measure(max(3, min(args.steps, 10)), 1, beam=100.0)
        out["beam"] = {"workload": bt.name, "beam": 100.0,
                       "ms_per_step": rb["ms_per_step"],
                       "ms_per_step_stats": rb["ms_per_step_stats"],
                       "value": bt.M / (rb["ms_per_step"] / 1e3),
                       "extra_ms_vs_exact": rb["ms_per_step"] - r["ms_per_step"],
                       "kernels": {k: v for k, v in rb["kernels"].items()
                                   if k in ("ctc_viterbi", "beam_mask", DP_KERNEL,
                                            "occupancy")},
                       "hbm_passes": rb["hbm_passes"]}
        # the pages' timing protocol: 3 runs of 5 warm-up and 50 measured
        # steps, the mean of the three run medians
        head.ctx.set_beam(math.inf)
        meds = [float(np.median(head.step_times(50, 5))) for _ in range(3)]
        out["protocol_3x50"] = {"runs": 3, "warmup": 5, "measured": 50,
                                "run_medians_ms": meds,
                                "mean_of_medians_ms": float(np.mean(meds)),
                                "frames_per_s": bt.M / (float(np.mean(meds)) / 1e3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(bt, args.cpu_sample_utts)
    head.close()
    del head
    if not args.no_extra:
        extra = {}
        for name in ("v500", "v5k", "llm152k"):
            if name == args.workload:
                continue
            run = Run(name, args.seed)
            steps = max(3, min(args.steps, 10))
            e = run.measure(steps, 2)
            extra[name] = {
                "config": config_of(run.bt, e["info"]), "dtype": run.bt.dtype,
                "steps": steps, "value": run.bt.M / (e["ms_per_step"] / 1e3),
                "unit": "frames/s", "ms_per_step": e["ms_per_step"],
                "ms_per_step_stats": e["ms_per_step_stats"],
                "pct_mfma_peak": e["pct_mfma_peak"],
                "workspace_GiB": e["info"]["workspace_bytes"] / 2**30,
                "roofline": dict(kernel=e["dom"], **e["roof"]),
                "kernels": e["kernels"], "hbm_passes": e["hbm_passes"],
            }
            if name == "v500":
                # the small vocabulary is where the recursions matter: the
                # finite beam's cost there
                rb = run.measure(steps, 1, beam=100.0)
                extra[name]["beam100_ms_per_step"] = rb["ms_per_step"]
                extra[name]["beam100_kernels"] = {
                    k: v for k, v in rb["kernels"].items()
                    if k in ("ctc_viterbi", "beam_mask", DP_KERNEL, "occupancy")}
            run.close()
            del run
        out["extra_workloads"] = extra
    print(json.dumps(out))


if __name__ == "__main__":
    main()
