"""Finite alignment beam (pcx_set_beam): the pages' pruned objective L_beta.

"Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", App. B.1
(finite-beam computation) and the finite-beam gap analysis; the PrunedCTC
README's output_beam.  An arc of an utterance's alignment lattice is kept
when the best complete alignment through it scores within beta of the best
alignment; the loss sums the alignments whose arcs are all kept, and the
gradient holds the kept arcs fixed.

Whether an arc is kept is a comparison of sums of log-probabilities, and the
library sums the FP32 scores S while the oracle sums its FP64 log-softmax, so
an arc whose score lies within rounding of the threshold could go either way.
The beam of each case is therefore chosen on the CPU, by the oracle alone,
among a set of candidates: the one whose nearest arc lies furthest from the
threshold (at least 1e-3 nats; the two sides' alignment scores differ by
about 1e-5 here), among those that do discard some mass.  With
the retained lattice then unique, loss, gradients, occupancies and the
discarded mass delta_n are held to the oracle's bar.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro, to_device, tolerance

pytestmark = pytest.mark.gpu

# candidate beams: 0.5, 0.75, ..., 20
CANDIDATES = [0.5 + 0.25 * i for i in range(79)]


def _case(name):
    if name == "tiles":
        return workloads.make_random(1, N=6, T_lo=40, T_hi=130, V=700, D=72, chunk=200)
    if name == "sharp":       # larger logits: alignment scores spread wider
        bt = workloads.make_random(31, N=5, T_lo=30, T_hi=90, V=300, D=64, chunk=128)
        bt.W = (bt.W * 12.0).astype(np.float32)
        return bt
    if name == "blank_last":
        return workloads.make_random(3, N=5, T_lo=20, T_hi=90, V=300, D=64, blank=299, chunk=64)
    if name == "unalignable_mix":
        T = [5, 3, 4, 9, 40]
        ys = [[1, 1, 2, 2], [3, 4, 5], [6, 6, 6], [7], list(range(8, 20))]
        return workloads.make_random(8, N=5, T_lo=0, T_hi=0, V=60, D=24, chunk=32,
                                     frame_counts=T, target_lengths=[len(y) for y in ys],
                                     labels=np.concatenate(ys).astype(np.int32))
    if name == "empty_and_short":
        T = [7, 20, 1, 33, 2]
        ys = [[], [3, 5, 5, 9, 2], [], [4, 4, 1, 8, 8, 8, 2, 6], [7]]
        return workloads.make_random(10, N=5, T_lo=0, T_hi=0, V=30, D=16, chunk=8,
                                     frame_counts=T, target_lengths=[len(y) for y in ys],
                                     labels=np.concatenate([np.asarray(y, np.int32)
                                                            for y in ys if y]))
    if name == "long_targets":   # several states per thread in the recursions
        bt = workloads.make_random(11, N=2, T_lo=0, T_hi=0, V=500, D=32, chunk=256,
                                   frame_counts=[1300, 700], target_lengths=[600, 300])
        bt.W = (bt.W * 6.0).astype(np.float32)
        return bt
    if name == "bf16_head":
        return workloads.make_random(14, N=3, T_lo=30, T_hi=90, V=900, D=136, chunk=256,
                                     dtype="bf16")
    raise KeyError(name)


def _pick_beam(bt):
    """The candidate beam whose pruning decisions are furthest from ties (by
    the oracle), among those that discard some posterior mass."""
    best = None
    for beam in CANDIDATES:
        r = oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                       want_dX=False, want_dW=False, want_db=False, want_lambda=False,
                       beam=beam)
        ok = r["status"] == 0
        if not np.any(ok):
            continue
        margin = float(np.min(r["margin"][ok]))
        dmax = float(np.nanmax(r["delta"]))
        if dmax > 1e-7 and (best is None or margin > best[1]):
            best = (beam, margin)
    return best


def _run(bt, beam, grouped=False):
    import torch
    from vocabulary_ctc_loss_amd import Context
    X, W, b, off, tgt, fc = to_device(bt)
    c = Context()
    try:
        c.set_formulation(grouped)
        c.set_beam(beam)
        loss, info = c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        dX = torch.full_like(X, float("nan"))
        dW = torch.full_like(W, float("nan"))
        db = torch.full_like(b, float("nan")) if b is not None else None
        c.backward(1.0, dX, dW, db)
        torch.cuda.synchronize()
        out = dict(loss=loss, info=info, utt_loss=c.utt_losses(), status=c.utt_status(),
                   U=c.selected(), Gam=c.occupancy(), delta=c.discarded_mass())
        for k, t in (("dX", dX), ("dW", dW), ("db", db)):
            out[k] = None if t is None else t.double().cpu().numpy()
    finally:
        c.close()
    return out


@pytest.mark.parametrize("name,grouped", [
    ("tiles", False), ("sharp", False), ("sharp", True), ("blank_last", False),
    ("unalignable_mix", False), ("empty_and_short", False), ("long_targets", False),
    ("bf16_head", False)])
def test_beam_matches_oracle(name, grouped):
    bt = _case(name)
    picked = _pick_beam(bt)
    assert picked is not None, "no candidate beam prunes this case"
    beam, margin = picked
    print("case", name, "grouped", grouped, "beam", beam, "margin %.3g" % margin, flush=True)
    assert margin >= 1e-3, "pruning decisions too close to ties for a parity check"
    got = _run(bt, beam, grouped)
    ref = oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                     cols=got["U"].tolist(), want_gamma=True, beam=beam)
    tol = tolerance(bt)
    assert got["status"].tolist() == ref["status"].tolist()
    assert abs(got["loss"] - ref["loss"]) <= tol * abs(ref["loss"])
    ok = ref["status"] == 0
    np.testing.assert_allclose(got["utt_loss"][ok], ref["utt_loss"][ok], rtol=tol)
    assert np.all(got["utt_loss"][~ok] == 0.0)
    for k in ("dX", "dW", "db"):
        if got[k] is None:
            continue
        e = rel_fro(got[k], ref[k])
        assert e <= tol, (k, e)
    # occupancies over the retained alignments, on the selected classes
    gam_tol = 2e-2 if bt.dtype == "bf16" else 1e-5
    np.testing.assert_allclose(got["Gam"], ref["gamma_cols"].T, atol=gam_tol)
    # discarded posterior mass per utterance
    d_ref, d_got = ref["delta"], got["delta"]
    assert np.array_equal(np.isnan(d_got), np.isnan(d_ref))
    fin = ~np.isnan(d_ref)
    dtol = (5e-2 if bt.dtype == "bf16" else 2e-3) * d_ref[fin] + 1e-10
    assert np.all(np.abs(d_got[fin] - d_ref[fin]) <= dtol), (d_got, d_ref)
    assert np.nanmax(d_got) > 1e-7
    assert np.all(d_got[fin] >= 0.0) and np.all(d_got[fin] <= 1.0)  # 1 - exp(-gap) rounds to 1


def test_unbounded_beam_is_the_exact_path_bit_for_bit():
    """An infinite beam is the default path; a beam wider than every score
    spread keeps every arc, so the pruned recursions reproduce the exact
    ones bit for bit, and nothing is discarded."""
    bt = _case("tiles")
    inf = _run(bt, math.inf)
    wide = _run(bt, 1e30)
    assert wide["loss"] == inf["loss"]
    for k in ("dX", "dW", "db", "Gam", "utt_loss"):
        assert np.array_equal(wide[k], inf[k]), k
    assert np.all(inf["delta"] == 0.0) and np.all(wide["delta"] == 0.0)


def test_narrow_beam_keeps_the_best_alignment():
    """A beam of 1e-9 keeps the best alignment alone (unique for these
    random scores): each utterance's occupancy is one-hot per frame and the
    loss is minus the best alignment's score, which the oracle's enumeration
    pins at small sizes and its lattice recursion gives here."""
    bt = workloads.make_random(41, N=4, T_lo=20, T_hi=60, V=200, D=32, chunk=64)
    got = _run(bt, 1e-9)
    ref = oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                     want_dX=False, want_dW=False, want_db=False, beam=1e-9)
    assert got["status"].tolist() == ref["status"].tolist() == [0, 0, 0, 0]
    np.testing.assert_allclose(got["utt_loss"], ref["utt_loss"], rtol=1e-5)
    G = got["Gam"]
    assert np.all((np.abs(G) < 1e-6) | (np.abs(G - 1.0) < 1e-6))
    np.testing.assert_allclose(G.sum(0), 1.0, atol=1e-6)


def test_beam_argument_checks():
    from vocabulary_ctc_loss_amd import Context, PcxError
    c = Context()
    try:
        for bad in (-1.0, float("nan")):
            with pytest.raises(PcxError):
                c.set_beam(bad)
        c.set_beam(0.0)
        c.set_beam(float("inf"))
    finally:
        c.close()


@pytest.mark.timeout(600)
def test_full_size_training_beam():
    """At the pages' training beam (100) on the V = 180k workload the pruned
    loss of every utterance is at least the exact one and discards almost
    nothing (the pages find beta = 100 at the numerical floor of their
    estimate), and the gradients stay within the fp32 bar of the exact
    path's."""
    bt = workloads.make("v180k", seed=0)
    exact = _run(bt, math.inf)
    pruned = _run(bt, 100.0)
    assert pruned["status"].tolist() == exact["status"].tolist()
    assert np.all(pruned["utt_loss"] >= exact["utt_loss"] * (1 - 1e-12))
    d = pruned["delta"]
    print("beam 100: max delta %.3g" % np.max(d), flush=True)
    assert np.all(d >= 0.0) and np.all(d <= 1e-6)
    assert abs(pruned["loss"] - exact["loss"]) <= 1e-5 * abs(exact["loss"])
    for k in ("dX", "dW", "db"):
        assert rel_fro(pruned[k], exact[k]) <= 1e-5, k
