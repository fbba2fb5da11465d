"""pcx_backward inside a HIP graph.  The backward makes no host
synchronisation and, once a first call has sized the context's workspace,
no allocation (the workspace only grows), so it can be captured and
replayed.  Each replay, with eager work between the replays, must give the
eager call's outputs bit for bit (the backward is deterministic)."""
import numpy as np
import pytest

import workloads
from pcx_harness import to_device

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "f32_all":   # fp32, dX dW db, several chunks and tiles
        return workloads.make_random(1, N=6, T_lo=40, T_hi=130, V=700, D=72, chunk=200), True
    # bf16 on the 256 x 256 core, dX alone: frames in two parts, chunks in pairs
    return workloads.make_random(25, N=6, T_lo=100, T_hi=140, V=900, D=64, chunk=128,
                                 dtype="bf16"), False


@pytest.mark.parametrize("name", ["f32_all", "bf16_dx_parts"])
def test_backward_replays_from_a_graph(name):
    import torch
    from vocabulary_ctc_loss_amd import Context
    bt, grads = _case(name)
    print("case", name, "M", bt.M, "V", bt.V, bt.dtype, flush=True)
    X, W, b, off, tgt, fc = to_device(bt)
    ctx = Context()
    try:
        ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        outs = [torch.empty_like(X), torch.empty_like(W) if grads else None,
                torch.empty_like(b) if grads and b is not None else None]
        ctx.backward(0.8, *outs)  # sizes the workspace
        torch.cuda.synchronize()
        ref = [None if t is None else t.clone() for t in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ctx.backward(0.8, *outs)
        for rep in range(3):
            for t in outs:
                if t is not None:
                    t.fill_(float("nan"))
            # unrelated eager work between the replays
            _ = (X[:64].float() @ W[:64].float().t().contiguous()).sum().item()
            g.replay()
            torch.cuda.synchronize()
            for k, (got, want) in enumerate(zip(outs, ref)):
                if want is None:
                    continue
                assert torch.equal(got, want), (rep, k)
        del g
    finally:
        ctx.close()
    assert np.isfinite(ref[0].double().cpu().numpy()).all()
