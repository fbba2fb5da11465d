"""The library works on the stream it is handed.  Two contexts on two side
streams (default priority), each with its own batch, their backward calls
issued back to back so that the work of the two can overlap on the GPU,
give the results of the same calls made one after the other on the default
stream, bit for bit (everything is deterministic and the contexts share no
device state)."""
import pytest

import workloads
from pcx_harness import to_device

pytestmark = pytest.mark.gpu


def _batches():
    a = workloads.make_random(1, N=6, T_lo=40, T_hi=130, V=700, D=72, chunk=200)
    b = workloads.make_random(25, N=6, T_lo=100, T_hi=140, V=900, D=64, chunk=128,
                              dtype="bf16")
    return [(a, True), (b, False)]


def _run(ctx, bt, dev, grads, stream):
    import torch
    X, W, b, off, tgt, fc = dev
    loss, _ = ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk, stream=stream)
    outs = [torch.full_like(X, float("nan")),
            torch.full_like(W, float("nan")) if grads else None,
            torch.full_like(b, float("nan")) if grads and b is not None else None]
    return loss, outs


def test_two_contexts_on_two_streams():
    import torch
    from vocabulary_ctc_loss_amd import Context
    jobs = []
    for bt, grads in _batches():
        jobs.append((Context(), bt, to_device(bt), grads))
    torch.cuda.synchronize()
    try:
        # one after the other on the default stream
        ref = []
        for c, bt, dev, grads in jobs:
            loss, outs = _run(c, bt, dev, grads, None)
            c.backward(0.6, *outs)
            torch.cuda.synchronize()
            ref.append((loss, [None if t is None else t.clone() for t in outs]))
        # side streams: both forwards, then both backwards back to back
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        runs = []
        for (c, bt, dev, grads), s in zip(jobs, streams):
            with torch.cuda.stream(s):
                runs.append(_run(c, bt, dev, grads, s))
        for (c, _, _, _), s, (_, outs) in zip(jobs, streams, runs):
            with torch.cuda.stream(s):
                c.backward(0.6, *outs, stream=s)
        torch.cuda.synchronize()
        for (loss, outs), (rloss, routs) in zip(runs, ref):
            assert loss == rloss
            for k, (got, want) in enumerate(zip(outs, routs)):
                if want is not None:
                    assert torch.equal(got, want), k
    finally:
        for c, _, _, _ in jobs:
            c.close()


def test_one_context_across_streams_with_growth():
    """One context, a small batch on one side stream (its backward left in
    flight), then a larger one on another stream: the workspace grows while
    the first stream may still be working, and both results equal their
    default-stream references bit for bit."""
    import torch
    from vocabulary_ctc_loss_amd import Context
    small = workloads.make_random(30, N=2, T_lo=20, T_hi=40, V=300, D=64, chunk=64,
                                  dtype="bf16")
    large = _batches()[0][0]  # fp32 with all gradients: most buffers grow
    jobs = [(small, False), (large, True)]
    devs = [to_device(bt) for bt, _ in jobs]
    torch.cuda.synchronize()
    ref = []
    for (bt, grads), dev in zip(jobs, devs):
        c = Context()
        loss, outs = _run(c, bt, dev, grads, None)
        c.backward(0.6, *outs)
        torch.cuda.synchronize()
        ref.append((loss, [None if t is None else t.clone() for t in outs]))
        c.close()
    c = Context()
    try:
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        got = []
        for (bt, grads), dev, s in zip(jobs, devs, streams):
            with torch.cuda.stream(s):
                loss, outs = _run(c, bt, dev, grads, s)
                c.backward(0.6, *outs, stream=s)
                got.append((loss, outs))
        torch.cuda.synchronize()
        for (loss, outs), (rloss, routs) in zip(got, ref):
            assert loss == rloss
            for k, (a, b) in enumerate(zip(outs, routs)):
                if b is not None:
                    assert torch.equal(a, b), k
    finally:
        c.close()


def test_one_context_across_streams_same_shapes():
    """One context, the same shapes twice (so the workspace does not grow)
    with different inputs, on two streams: the second call's forward must
    not overwrite the scores, normalizer and recursions the first call's
    backward, still in flight on the other stream, reads.  Calls on one
    context follow each other across streams; both results equal their
    default-stream references bit for bit."""
    import torch
    from vocabulary_ctc_loss_amd import Context
    bt = _batches()[0][0]
    dev1 = to_device(bt)
    X2 = dev1[0] * 0.5
    dev2 = (X2,) + tuple(dev1[1:])
    torch.cuda.synchronize()
    ref = []
    for dev in (dev1, dev2):
        c = Context()
        loss, outs = _run(c, bt, dev, True, None)
        c.backward(0.6, *outs)
        torch.cuda.synchronize()
        ref.append((loss, [t.clone() for t in outs]))
        c.close()
    c = Context()
    try:
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        got = []
        for dev, st in zip((dev1, dev2), streams):
            with torch.cuda.stream(st):
                loss, outs = _run(c, bt, dev, True, st)
                c.backward(0.6, *outs, stream=st)
                got.append((loss, outs))
        torch.cuda.synchronize()
        for (loss, outs), (rloss, routs) in zip(got, ref):
            assert loss == rloss
            for k, (a, b) in enumerate(zip(outs, routs)):
                assert torch.equal(a, b), k
    finally:
        c.close()

