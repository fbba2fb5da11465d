"""The workspace lives in the caller's allocator (pcx_create's callbacks).

The Python binding hands the library torch's caching allocator, so the
workspace of a forward and backward shows in torch.cuda.memory_allocated and
max_memory_allocated, the counters the pages measure head-and-loss memory
with ("Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", App.
C.1).  Results do not depend on where the workspace comes from: a context on
the library's own hipMalloc gives the same bits.  pcx_destroy hands every
byte back.
"""
import pytest

import workloads
from pcx_harness import to_device

pytestmark = pytest.mark.gpu


def _grads(X, W, b):
    import torch
    return (torch.full_like(X, float("nan")), torch.full_like(W, float("nan")),
            torch.full_like(b, float("nan")))


def test_workspace_in_torch_allocator_counters():
    import torch
    from vocabulary_ctc_loss_amd import Context
    bt = workloads.make_random(3, N=8, T_lo=60, T_hi=200, V=3000, D=128, chunk=512)
    X, W, b, off, tgt, fc = to_device(bt)
    dX, dW, db = _grads(X, W, b)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    print("case alloc-counters M", bt.M, "V", bt.V, flush=True)
    ctx = Context()  # torch's caching allocator
    loss, info = ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
    after_fwd = torch.cuda.memory_allocated()
    fwd_ws = info["workspace_bytes"]
    assert fwd_ws > 0
    # the caching allocator rounds each block up to 512 bytes
    assert fwd_ws <= after_fwd - base <= fwd_ws + 512 * 40
    ctx.backward(1.0, dX, dW, db)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    held = torch.cuda.memory_allocated() - base
    # the backward adds occupancies, the M x C block and the split partials
    assert held > after_fwd - base
    assert peak >= held
    ctx.close()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base

    # the same calls on the library's own hipMalloc workspace: identical bits,
    # and nothing of it in torch's counters
    ref = Context(allocator=None)
    rX, rW, rb = _grads(X, W, b)
    torch.cuda.synchronize()
    base2 = torch.cuda.memory_allocated()
    rloss, rinfo = ref.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
    ref.backward(1.0, rX, rW, rb)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base2
    assert rloss == loss and rinfo["K"] == info["K"]
    for got, want in ((dX, rX), (dW, rW), (db, rb)):
        assert torch.equal(got, want)
    ref.close()


def test_workspace_growth_on_the_callers_stream():
    """A second, larger forward on the same stream grows the workspace through
    the allocator (release then allocate on that stream, no device-wide
    wait); results match a fresh context, and the first batch's results are
    reproduced after the growth."""
    import torch
    from vocabulary_ctc_loss_amd import Context
    small = workloads.make_random(4, N=3, T_lo=30, T_hi=60, V=500, D=64, chunk=256)
    large = workloads.make_random(5, N=7, T_lo=100, T_hi=220, V=2500, D=64, chunk=256)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ctx = Context()
    outs = []
    with torch.cuda.stream(s):
        for bt in (small, large, small):
            print("case growth M", bt.M, "V", bt.V, flush=True)
            X, W, b, off, tgt, fc = to_device(bt)
            g = _grads(X, W, b)
            loss, info = ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk, stream=s)
            ctx.backward(1.0, *g, stream=s)
            outs.append((loss, info["workspace_bytes"], [t.clone() for t in g]))
    torch.cuda.synchronize()
    assert outs[1][1] > outs[0][1]          # the workspace grew
    assert outs[2][1] >= outs[1][1]         # and is kept (the backward may add more)
    assert outs[2][0] == outs[0][0]
    for a, c in zip(outs[0][2], outs[2][2]):
        assert torch.equal(a, c)
    fresh = Context()
    X, W, b, off, tgt, fc = to_device(large)
    g = _grads(X, W, b)
    loss, _ = fresh.forward(X, W, b, off, tgt, fc, large.blank, large.chunk)
    fresh.backward(1.0, *g)
    torch.cuda.synchronize()
    assert loss == outs[1][0]
    for a, c in zip(g, outs[1][2]):
        assert torch.equal(a, c)
    ctx.close()
    fresh.close()
