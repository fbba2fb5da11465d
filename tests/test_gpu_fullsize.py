"""Parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot redo a whole V = 180k or LLM-head batch in seconds, so:
* U, relabelled targets and alignability flags are compared bit-exact on the
  whole batch (cheap set arithmetic in the oracle);
* per-utterance losses and the dX rows of sampled utterances are compared
  with the oracle run on those utterances alone (both depend only on the
  utterance itself);
* dW and db, which mix all utterances, are checked by properties that hold
  at any size: every alignable frame's logit-gradient row sums to zero, so
  sum_v db_v = 0 and sum_v dW[v, :] = 0 up to rounding (and neither is all
  zeros);
* the grouped formulation is held to the same sampled bar and compared with
  the direct one on the whole batch;
* the two small-vocabulary workloads (V = 500 and 5000), where the oracle
  runs the whole batch in seconds, are compared output by output: every
  utterance's loss, and all of dX, dW and db;
* the V = 180k workload is compared output by output too: the oracle runs
  it in five groups of five utterances (about half a minute each), every
  utterance's loss and dX rows are checked per group, and dW and db against
  the sum of the groups' head gradients (utterances contribute additively);
* on the LLM head (dX alone, frames in two parts on the GPU) dX is compared
  on the first and last utterances, on one more utterance wholly inside each
  part, and on the utterance that straddles the part boundary.
"""
import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro, run_pcx, tolerance

pytestmark = pytest.mark.gpu

# GPU results of a full-size workload, computed once per module
_GPU = {}


def _gpu(name):
    if name not in _GPU:
        bt = workloads.make(name, seed=0)
        print("workload", name, "M", bt.M, "V", bt.V, "D", bt.D, "N", bt.N, flush=True)
        _GPU[name] = (bt, run_pcx(bt, want_dW=bt.want_dW, want_db=bt.want_db, getters="light"))
    return _GPU[name]


def _sample(bt):
    # the shortest utterance keeps the oracle's share of the test short; where
    # the oracle is quick enough (D <= 512) the longest one too
    idx = [int(np.argmin(bt.frame_counts))]
    if bt.D <= 512:
        idx.append(int(np.argmax(bt.frame_counts)))
    return idx


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["v500", "v5k", "v180k", "llm152k"])
def test_full_size_sampled(name):
    bt, got = _gpu(name)
    U, rel, flags = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    assert got["U"].tolist() == U.tolist()
    assert got["rel"].tolist() == rel.tolist()
    assert got["flags"].tolist() == flags.tolist()
    assert np.all(got["status"] == 0)
    assert got["loss"] == pytest.approx(float(np.sum(got["utt_loss"])), rel=1e-12)
    tol = tolerance(bt)
    idx = _sample(bt)
    sb = workloads.sample_utterances(bt, idx)
    print("oracle on utterances", idx, "frames", sb.M, flush=True)
    ref = oracle.pcx(sb.X, sb.W, sb.b, sb.frame_counts, sb.tgt_off, sb.tgt, sb.blank,
                     want_dW=False, want_db=False)
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    for j, n in enumerate(idx):
        assert abs(got["utt_loss"][n] - ref["utt_loss"][j]) <= tol * abs(ref["utt_loss"][j])
    rows = np.concatenate([np.arange(row_off[n], row_off[n + 1]) for n in idx])
    assert rel_fro(got["dX"][rows], ref["dX"]) <= tol
    if bt.want_db:
        db = got["db"]
        assert np.abs(db).sum() > 0.0
        assert abs(db.sum()) <= 1e-5 * np.abs(db).sum()
    if bt.want_dW:
        dW = got["dW"]
        colsum = np.abs(dW.sum(0))
        scale = np.abs(dW).sum(0)
        assert np.all(scale > 0.0)
        assert np.all(colsum <= 1e-5 * scale)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["v180k", "llm152k"])
def test_full_size_grouped_matches_oracle_and_direct(name):
    """The grouped ("other" column) formulation at full size: per-utterance
    losses and sampled dX rows against the oracle, and everything against the
    direct formulation on the same inputs (equal up to rounding)."""
    bt = workloads.make(name, seed=0)
    print("workload", name, "grouped", flush=True)
    d = run_pcx(bt, want_dW=bt.want_dW, want_db=bt.want_db, getters="light")
    g = run_pcx(bt, want_dW=bt.want_dW, want_db=bt.want_db, getters="light", grouped=True)
    tol = tolerance(bt)
    assert g["status"].tolist() == d["status"].tolist()
    assert abs(g["loss"] - d["loss"]) <= 1e-6 * abs(d["loss"])
    for k in ("dX", "dW", "db"):
        if d[k] is not None:
            assert rel_fro(g[k], d[k]) <= (1e-6 if bt.dtype == "f32" else 1e-2), k
    idx = _sample(bt)
    sb = workloads.sample_utterances(bt, idx)
    ref = oracle.pcx(sb.X, sb.W, sb.b, sb.frame_counts, sb.tgt_off, sb.tgt, sb.blank,
                     want_dW=False, want_db=False)
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    for j, n in enumerate(idx):
        assert abs(g["utt_loss"][n] - ref["utt_loss"][j]) <= tol * abs(ref["utt_loss"][j])
    rows = np.concatenate([np.arange(row_off[n], row_off[n + 1]) for n in idx])
    assert rel_fro(g["dX"][rows], ref["dX"]) <= tol


# utterance groups of the V = 180k batch (N = 25) for the oracle, and the sum
# of their head gradients
V180K_GROUPS = [list(range(5 * i, 5 * i + 5)) for i in range(5)]
_V180K = {}       # group -> the oracle's per-utterance outputs
_V180K_SUM = {}   # running sums of the groups' dW, db and loss


def _v180k_group(i):
    if i not in _V180K:
        bt, _ = _gpu("v180k")
        sb = workloads.sample_utterances(bt, V180K_GROUPS[i])
        print("oracle on v180k utterances", V180K_GROUPS[i], "frames", sb.M, flush=True)
        ref = oracle.pcx(sb.X, sb.W, sb.b, sb.frame_counts, sb.tgt_off, sb.tgt, sb.blank,
                         want_lambda=False)
        if not _V180K_SUM:
            _V180K_SUM.update(dW=np.zeros_like(ref["dW"]), db=np.zeros_like(ref["db"]), loss=0.0)
        _V180K_SUM["dW"] += ref["dW"]
        _V180K_SUM["db"] += ref["db"]
        _V180K_SUM["loss"] += ref["loss"]
        _V180K[i] = {k: ref[k] for k in ("status", "utt_loss", "dX")}
    return _V180K[i]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("group", range(len(V180K_GROUPS)))
def test_v180k_whole_batch_losses_and_dx(group):
    """V = 180k at full size: the losses and dX rows of five utterances, from
    the one whole-batch GPU run, against the oracle on those utterances."""
    bt, got = _gpu("v180k")
    ref = _v180k_group(group)
    idx = V180K_GROUPS[group]
    tol = tolerance(bt)
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    assert got["status"][idx].tolist() == ref["status"].tolist()
    for j, n in enumerate(idx):
        assert abs(got["utt_loss"][n] - ref["utt_loss"][j]) <= tol * abs(ref["utt_loss"][j])
    rows = np.concatenate([np.arange(row_off[n], row_off[n + 1]) for n in idx])
    e = rel_fro(got["dX"][rows], ref["dX"])
    print("dX rows of", idx, "relative Frobenius error %.3g" % e, flush=True)
    assert e <= tol


@pytest.mark.timeout(900)
def test_v180k_whole_batch_head_gradients():
    """dW and db of the whole V = 180k batch (the split-frame dW reduction and
    the 44 chunk reductions of the timed configuration) against the sum of
    the oracle's per-group head gradients, and the summed loss."""
    bt, got = _gpu("v180k")
    for i in range(len(V180K_GROUPS)):
        _v180k_group(i)
    dW, db, loss = _V180K_SUM["dW"], _V180K_SUM["db"], _V180K_SUM["loss"]
    tol = tolerance(bt)
    assert abs(got["loss"] - loss) <= tol * abs(loss)
    for k, want in (("dW", dW), ("db", db)):
        assert np.linalg.norm(got[k]) > 0.0
        e = rel_fro(got[k], want)
        print(k, "relative Frobenius error %.3g" % e, flush=True)
        assert e <= tol, (k, e)


def _llm_samples(bt):
    """Utterances of the LLM-head batch to check dX on: the first, the last,
    the one holding the first row of the backward's second frame part, and
    the shortest utterance wholly inside each part."""
    M, rtile = bt.M, 256
    split = ((M + 1) // 2 + rtile - 1) // rtile * rtile  # first row of part 2
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    n_split = int(np.searchsorted(row_off, split, side="right")) - 1
    assert row_off[n_split] < split < row_off[n_split + 1]
    part1 = [n for n in range(1, bt.N - 1) if row_off[n + 1] <= split and n != n_split]
    part2 = [n for n in range(1, bt.N - 1) if row_off[n] >= split and n != n_split]
    pick = lambda ns: min(ns, key=lambda n: bt.frame_counts[n])  # noqa: E731
    return {"first": 0, "last": bt.N - 1, "straddle": n_split, "part1": pick(part1),
            "part2": pick(part2)}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("which", ["first", "part1", "straddle", "part2", "last"])
def test_llm152k_dx_across_frame_parts(which):
    bt, got = _gpu("llm152k")
    n = _llm_samples(bt)[which]
    sb = workloads.sample_utterances(bt, [n])
    print("oracle on llm152k utterance", n, which, "frames", sb.M, flush=True)
    ref = oracle.pcx(sb.X, sb.W, sb.b, sb.frame_counts, sb.tgt_off, sb.tgt, sb.blank,
                     want_dW=False, want_db=False, want_lambda=False)
    tol = tolerance(bt)
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    assert abs(got["utt_loss"][n] - ref["utt_loss"][0]) <= tol * abs(ref["utt_loss"][0])
    e = rel_fro(got["dX"][row_off[n]:row_off[n + 1]], ref["dX"])
    print("dX relative Frobenius error %.3g" % e, flush=True)
    assert e <= tol


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["v500", "v5k"])
def test_full_size_whole_batch(name):
    """Full size, no sampling: the oracle on the whole batch; loss and every
    gradient held to the relative Frobenius bar (1e-5 fp32)."""
    bt = workloads.make(name, seed=0)
    print("workload", name, "M", bt.M, "V", bt.V, "D", bt.D, "N", bt.N, flush=True)
    got = run_pcx(bt, want_dW=True, want_db=True, getters="light")
    print("oracle on the whole batch", flush=True)
    ref = oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                     want_lambda=False)
    tol = tolerance(bt)
    assert got["status"].tolist() == ref["status"].tolist()
    assert abs(got["loss"] - ref["loss"]) <= tol * abs(ref["loss"])
    assert rel_fro(got["utt_loss"], ref["utt_loss"]) <= tol
    for k in ("dX", "dW", "db"):
        e = rel_fro(got[k], ref[k])
        print(k, "relative Frobenius error %.3g" % e, flush=True)
        assert e <= tol, (k, e)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["v180k", "llm152k"])
def test_full_size_workspace(name):
    """On the two large-vocabulary heads (V much larger than the chunk C) the
    device workspace a context holds after a forward and a backward (read at
    the following forward; it only grows) has no block of the batch's M x V
    size: it stays under a quarter of one fp32 M x V logits matrix, and at
    the V = 180k, M = 16k point within the 1.29 GiB of head and loss memory
    the pages report for their own implementation ([P] Sec. 5.1, Fig. 4)."""
    from vocabulary_ctc_loss_amd import Context
    bt = workloads.make(name, seed=0)
    c = Context()
    try:
        run_pcx(bt, want_dW=bt.want_dW, want_db=bt.want_db, getters=False, ctx=c)
        got = run_pcx(bt, want_dW=bt.want_dW, want_db=bt.want_db, getters=False, ctx=c)
    finally:
        c.close()
    ws = got["info"]["workspace_bytes"]
    dense = bt.M * bt.V * 4
    print(name, "workspace %.3f GiB, fp32 M x V %.3f GiB" % (ws / 2**30, dense / 2**30),
          flush=True)
    assert ws < dense / 4
    if name == "v180k":
        assert ws <= 1.29 * 2**30

