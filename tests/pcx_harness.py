"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
the CPU oracle on the same seeded batch, and compare."""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def to_device(bt: workloads.Batch, dev="cuda:0"):
    import torch
    # "f32_bf16w": fp32 encoder states with a bf16-stored head
    xt = torch.bfloat16 if bt.dtype == "bf16" else torch.float32
    wt = torch.float32 if bt.dtype == "f32" else torch.bfloat16
    X = torch.from_numpy(bt.X).to(dev).to(xt)
    W = torch.from_numpy(bt.W).to(dev).to(wt)
    b = None if bt.b is None else torch.from_numpy(bt.b).to(dev).to(wt)
    off = torch.from_numpy(np.ascontiguousarray(bt.tgt_off, np.int32)).to(dev)
    tgt = torch.from_numpy(np.ascontiguousarray(bt.tgt, np.int32)).to(dev)
    fc = torch.from_numpy(np.ascontiguousarray(bt.frame_counts, np.int32)).to(dev)
    return X, W, b, off, tgt, fc


def run_pcx(bt: workloads.Batch, grad=1.0, want_dX=True, want_dW=True, want_db=True,
            getters=True, ctx=None, grouped=False):
    import torch
    from vocabulary_ctc_loss_amd import Context
    X, W, b, off, tgt, fc = to_device(bt)
    own = ctx is None
    c = Context() if own else ctx
    c.set_formulation(grouped)
    loss, info = c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
    dX = torch.full_like(X, float("nan")) if want_dX else None
    dW = torch.full_like(W, float("nan")) if want_dW else None
    db = torch.full_like(b, float("nan")) if (want_db and b is not None) else None
    c.backward(grad, dX, dW, db)
    torch.cuda.synchronize()
    out = {"loss": loss, "info": info}
    if getters:
        out.update(U=c.selected(), rel=c.relabeled(), flags=c.alignable(),
                   utt_loss=c.utt_losses(), status=c.utt_status())
        if getters != "light":
            out.update(lam=c.normalizer(), S=c.scores(), Gam=c.occupancy())
        if grouped:
            out["other"] = c.other()
    for k, t in (("dX", dX), ("dW", dW), ("db", db)):
        out[k] = None if t is None else t.double().cpu().numpy()
    if own:
        c.close()
    return out


def run_oracle(bt: workloads.Batch, grad=1.0, cols=None, want_gamma=False, want_dW=True,
               want_db=True):
    return oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                      grad=grad, cols=cols, want_gamma=want_gamma, want_dW=want_dW,
                      want_db=want_db)


def rel_fro(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / den


def tolerance(bt: workloads.Batch) -> float:
    # fp32 products (fp32 inputs, or fp32 states with a bf16-stored head whose
    # values both sides see exactly): 1e-5 on loss and gradients; bf16: 2e-2.
    return 2e-2 if bt.dtype == "bf16" else 1e-5
