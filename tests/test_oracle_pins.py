"""Pins for the CPU FP64 oracle, against things other than the oracle itself.

* brute-force enumeration of every frame-level label sequence and the collapse
  map (merge repeats, then drop blanks; "Pruned CTC for Memory-Efficient
  Large-Vocabulary ASR Training", Sec. 3.1) on tiny inputs, for the loss and
  the occupancies;
* the alignment-count closed form C(T + L - r, 2L), checked by brute force and
  then used for uniform logits at sizes brute force cannot reach;
* special cases with a single alignment (T = |y| + r) and the empty target;
* central finite differences of the oracle's own loss for dX, dW and db;
* Proposition 1 (Sec. 3.2): the reduced computation on grouped logits R
  (selected columns plus one "other" column holding the log-sum-exp of the
  complement, Eq. 4) gives the same loss, and, with the other-column gradient
  spread over the complement by the log-sum-exp Jacobian (App. B.1, Eq. 11),
  the same logit gradient;
* invariants: gradient rows sum to zero on alignable frames, unalignable
  utterances give exact zeros, shift of the bias, consistent relabelling of
  classes, utterance permutation and batch additivity;
* the selected-class set and the alignability flags against Python set
  arithmetic and the README example fixture.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def collapse(seq, blank):
    out = []
    prev = None
    for s in seq:
        if s != prev and s != blank:
            out.append(s)
        prev = s
    return out


def brute_force(Z, y, blank):
    """Sum over all V^T label sequences whose collapse is y."""
    T, V = Z.shape
    logp = Z - np.log(np.sum(np.exp(Z - Z.max(1, keepdims=True)), 1, keepdims=True)) \
        - Z.max(1, keepdims=True)
    p = np.exp(logp)
    total = 0.0
    occ = np.zeros((T, V))
    count = 0
    y = list(y)
    for seq in itertools.product(range(V), repeat=T):
        if collapse(seq, blank) == y:
            pr = 1.0
            for t, v in enumerate(seq):
                pr *= p[t, v]
            total += pr
            count += 1
            for t, v in enumerate(seq):
                occ[t, v] += pr
    gamma = occ / total if total > 0 else occ
    return total, gamma, count, p


def repeats(y):
    return sum(1 for i in range(len(y) - 1) if y[i] == y[i + 1])


# ------------------------------------------------------------ brute force
@pytest.mark.parametrize("T,V,y,blank,seed", [
    (5, 4, [1, 2], 0, 0),
    (6, 4, [1, 1], 0, 1),
    (6, 3, [2, 1, 2], 0, 2),
    (7, 4, [3, 3, 3], 0, 3),     # T = L + r: a single alignment
    (6, 4, [], 0, 4),            # empty target
    (6, 4, [0, 2], 3, 5),        # blank is the last class
    (6, 5, [1, 4, 1], 2, 6),     # blank in the middle
    (8, 3, [1, 2, 1, 2], 0, 7),
])
def test_brute_force_loss_and_occupancy(T, V, y, blank, seed):
    rng = np.random.default_rng(seed)
    Z = rng.normal(scale=2.0, size=(T, V))
    total, gamma, count, p = brute_force(Z, y, blank)
    r = oracle.ctc_logits(Z, y, blank, grad=1.0)
    assert count == math.comb(T + len(y) - repeats(y), 2 * len(y))
    assert r["status"] == 0
    assert r["loss"] == pytest.approx(-math.log(total), rel=1e-12, abs=1e-12)
    np.testing.assert_allclose(r["gamma"], gamma, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(r["dZ"], p - gamma, rtol=1e-10, atol=1e-13)


def test_brute_force_unalignable():
    rng = np.random.default_rng(11)
    Z = rng.normal(size=(3, 4))
    y = [1, 1, 2]  # needs 4 frames
    total, _, count, _ = brute_force(Z, y, 0)
    assert count == 0 and total == 0.0
    r = oracle.ctc_logits(Z, y, 0)
    assert r["status"] == oracle.STATUS_UNALIGNABLE
    assert r["loss"] == 0.0
    assert np.all(r["dZ"] == 0.0) and np.all(r["gamma"] == 0.0)


def test_brute_force_through_head():
    """Whole path on a 3-utterance batch against enumeration per utterance."""
    rng = np.random.default_rng(21)
    V, D = 4, 3
    T = [5, 4, 3]
    ys = [[1, 2], [3, 3], [2, 1, 2]]  # last one needs 3 frames: alignable
    M = sum(T)
    X = rng.normal(size=(M, D))
    W = rng.normal(size=(V, D))
    b = rng.normal(size=V)
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate(ys)
    out = oracle.pcx(X, W, b, T, off, tgt, blank=0, grad=1.0)
    row = 0
    expected = 0.0
    for n, y in enumerate(ys):
        Z = X[row:row + T[n]] @ W.T + b
        total, _, _, _ = brute_force(Z, y, 0)
        assert out["utt_loss"][n] == pytest.approx(-math.log(total), rel=1e-12)
        expected += -math.log(total)
        row += T[n]
    assert out["loss"] == pytest.approx(expected, rel=1e-12)


def test_column_gather_at_unsorted_columns():
    """logp_cols / gamma_cols at an unsorted, non-identity column list.

    The scores S and occupancies Gamma of the reduced method are indexed by
    the selected classes U ("Pruned CTC for Memory-Efficient Large-Vocabulary
    ASR Training", Sec. 3.2), so the oracle's per-column outputs must be the
    log-probability and occupancy of class cols[c], not of class c.  Checked
    on a three-utterance batch against numpy's log-softmax of X W^T + b and
    against brute-force occupancies of every utterance.
    """
    rng = np.random.default_rng(31)
    V, D = 5, 3
    T = [6, 5, 4]
    ys = [[1, 3], [4, 4], [2]]
    M = sum(T)
    X = rng.normal(size=(M, D))
    W = rng.normal(size=(V, D))
    b = rng.normal(size=V)
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate(ys)
    cols = [V - 1, 0, 3, 2]
    out = oracle.pcx(X, W, b, T, off, tgt, blank=0, cols=cols, want_gamma=True)
    Z = X @ W.T + b
    zmax = Z.max(1, keepdims=True)
    logp = Z - zmax - np.log(np.sum(np.exp(Z - zmax), 1, keepdims=True))
    np.testing.assert_allclose(out["logp_cols"], logp[:, cols], rtol=1e-13, atol=1e-13)
    row = 0
    for n, y in enumerate(ys):
        rows = slice(row, row + T[n])
        _, gamma, count, _ = brute_force(Z[rows], y, 0)
        assert count > 0
        np.testing.assert_allclose(out["gamma_cols"][rows], gamma[:, cols], rtol=1e-10,
                                   atol=1e-13)
        row += T[n]
    # the gathered columns differ from the first len(cols) classes
    assert not np.allclose(out["logp_cols"], logp[:, :len(cols)])


# ------------------------------------------------------------ finite beam
def node_states(seq, blank):
    """State of each frame of an alignment in the blank-interleaved label
    sequence: 2k on a blank after k emitted labels, 2k - 1 on the k-th label
    (the node of the alignment lattice the frame visits)."""
    out = []
    k = 0
    prev = None
    for v in seq:
        if v != blank and v != prev:
            k += 1
        out.append(2 * k if v == blank else 2 * k - 1)
        prev = v
    return out


def brute_force_beam(Z, y, blank, beam):
    """Retained-alignment sum by enumeration: an alignment is kept when every
    arc it uses (the initial arc into its first node, each frame-to-frame arc,
    the final arc out of its last node) lies on some alignment scoring within
    `beam` of the best one.  Returns (P_beta, gamma_beta, P, B, n_kept)."""
    T, V = Z.shape
    zmax = Z.max(1, keepdims=True)
    logp = Z - zmax - np.log(np.sum(np.exp(Z - zmax), 1, keepdims=True))
    paths = []
    for seq in itertools.product(range(V), repeat=T):
        if collapse(seq, blank) == list(y):
            sc = sum(logp[t, v] for t, v in enumerate(seq))
            st = node_states(seq, blank)
            arcs = [("init", st[0]), ("final", st[-1])] + \
                   [(t, st[t - 1], st[t]) for t in range(1, T)]
            paths.append((seq, sc, arcs))
    best = max(sc for _, sc, _ in paths)
    arc_best = {}
    for _, sc, arcs in paths:
        for a in arcs:
            arc_best[a] = max(arc_best.get(a, -np.inf), sc)
    P = Pb = 0.0
    gam = np.zeros((T, V))
    kept = 0
    for seq, sc, arcs in paths:
        P += math.exp(sc)
        if all(arc_best[a] >= best - beam for a in arcs):
            kept += 1
            Pb += math.exp(sc)
            for t, v in enumerate(seq):
                gam[t, v] += math.exp(sc)
    return Pb, gam / Pb if Pb > 0 else gam, P, best, kept


@pytest.mark.parametrize("T,V,y,blank,seed,beam", [
    (6, 4, [1, 2], 0, 40, 1.0),
    (6, 4, [1, 2], 0, 40, 3.0),
    (7, 3, [1, 1], 0, 41, 2.0),
    (6, 4, [2, 1, 2], 3, 42, 1.5),
    (7, 4, [3], 1, 43, 4.0),
    (6, 4, [], 0, 44, 0.7),
    (8, 3, [1, 2, 1], 0, 45, 2.5),
])
def test_beam_brute_force_retained_alignments(T, V, y, blank, seed, beam):
    """Loss over the retained alignments and their occupancies, against the
    enumeration of every alignment and of the best alignment through each
    lattice arc."""
    rng = np.random.default_rng(seed)
    Z = rng.normal(scale=2.0, size=(T, V))
    Pb, gam, P, best, kept = brute_force_beam(Z, y, blank, beam)
    r = oracle.ctc_beam(Z, y, blank, beam)
    assert r["margin"] > 1e-9          # no arc within rounding of the threshold
    assert r["status"] == 0 and kept > 0
    assert r["loss"] == pytest.approx(-math.log(Pb), rel=1e-12, abs=1e-12)
    assert r["full_loss"] == pytest.approx(-math.log(P), rel=1e-12, abs=1e-12)
    np.testing.assert_allclose(r["gamma"], gam, rtol=1e-10, atol=1e-13)
    p = np.exp(Z - r["lambda"][:, None])
    np.testing.assert_allclose(r["dZ"], p - gam, rtol=1e-10, atol=1e-13)


def test_beam_best_is_over_complete_alignments():
    """With the blank strongly favoured, the best-scoring prefix at the last
    frame ends in an unfinished state (all blanks); the threshold must come
    from the best complete alignment, as the enumeration's does."""
    rng = np.random.default_rng(50)
    T, V, y, beam = 7, 4, [1, 2, 3], 2.0
    Z = rng.normal(size=(T, V))
    Z[:, 0] += 4.0
    Pb, gam, P, best, kept = brute_force_beam(Z, y, 0, beam)
    r = oracle.ctc_beam(Z, y, 0, beam)
    lp = Z - r["lambda"][:, None]
    assert lp[:, 0].sum() > best + beam      # the all-blank prefix beats every alignment
    assert r["status"] == 0 and r["margin"] > 1e-9
    assert r["loss"] == pytest.approx(-math.log(Pb), rel=1e-12)
    np.testing.assert_allclose(r["gamma"], gam, rtol=1e-10, atol=1e-13)


def test_beam_prunes_something_in_the_brute_force_cases():
    """The parameter sets above do prune (retained fewer than all), and keep
    more than the best alignment alone in some."""
    fewer = more = 0
    for T, V, y, blank, seed, beam in [(6, 4, [1, 2], 0, 40, 1.0), (7, 3, [1, 1], 0, 41, 2.0),
                                       (8, 3, [1, 2, 1], 0, 45, 2.5)]:
        Z = np.random.default_rng(seed).normal(scale=2.0, size=(T, V))
        Pb, _, P, _, kept = brute_force_beam(Z, y, blank, beam)
        total = math.comb(T + len(y) - repeats(y), 2 * len(y))
        fewer += kept < total
        more += kept > 1
    assert fewer == 3 and more >= 2


def test_beam_limits():
    """An unbounded beam is the unpruned loss; a beam just above zero (1e-9:
    at exactly zero, rounding of the arc scores can put the best alignment's
    own arcs below its score and empty the lattice) keeps only the best
    alignment (unique here), so the loss is minus its score; the loss never
    increases as the beam widens and never drops below the unpruned one."""
    rng = np.random.default_rng(46)
    T, V, y = 9, 4, [1, 3, 3]
    Z = rng.normal(scale=2.0, size=(T, V))
    full = oracle.ctc_logits(Z, y, 0)
    inf = oracle.ctc_beam(Z, y, 0, math.inf)
    assert inf["loss"] == full["loss"] and inf["full_loss"] == full["loss"]
    np.testing.assert_array_equal(inf["dZ"], full["dZ"])
    Pb, _, _, best, kept = brute_force_beam(Z, y, 0, 1e-9)
    assert kept == 1
    zero = oracle.ctc_beam(Z, y, 0, 1e-9)
    assert zero["status"] == 0
    assert zero["loss"] == pytest.approx(-best, rel=1e-12)
    gam = zero["gamma"]
    assert np.all((gam == 0.0) | (np.abs(gam - 1.0) < 1e-12))  # one path: one-hot
    prev = math.inf
    for beam in [1e-9, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 64.0, math.inf]:
        r = oracle.ctc_beam(Z, y, 0, beam, want_grad=False)
        assert r["loss"] <= prev + 1e-12 and r["loss"] >= full["loss"] - 1e-12
        prev = r["loss"]
    assert prev == full["loss"]


def test_beam_occupancy_mixture_bound():
    """The full occupancy mixes the retained and the discarded ones with
    weight delta, so per frame the L1 distance between gamma and gamma_beta is
    at most 2 delta (the pages' finite-beam gap analysis), with delta = 1 -
    exp(-(L_beta - L)) = 1 - P_beta / P."""
    rng = np.random.default_rng(47)
    T, V, y = 12, 5, [2, 4, 4, 1]
    Z = rng.normal(scale=2.5, size=(T, V))
    full = oracle.ctc_logits(Z, y, 0)
    seen = 0
    for beam in [1.0, 2.0, 3.0, 5.0]:
        r = oracle.ctc_beam(Z, y, 0, beam)
        gap = r["loss"] - full["loss"]
        delta = -math.expm1(-gap)
        assert gap >= -1e-12 and 0.0 <= delta < 1.0
        l1 = np.abs(full["gamma"] - r["gamma"]).sum(1)
        assert np.all(l1 <= 2 * delta + 1e-12)
        seen += delta > 1e-6
    assert seen >= 2


def test_beam_finite_differences():
    """Gradient of L_beta with the retained lattice held fixed (the pages'
    "locally fixed" lattice): central differences of the loss through the
    head, at a beam whose pruning decisions are far from ties."""
    rng = np.random.default_rng(48)
    V, D = 5, 3
    T = [7, 6]
    ys = [[1, 3], [2, 2]]
    M = sum(T)
    X = rng.normal(size=(M, D))
    W = rng.normal(size=(V, D))
    b = rng.normal(size=V)
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate(ys)
    beam = 1.5
    out = oracle.pcx(X, W, b, T, off, tgt, 0, grad=1.0, beam=beam)
    assert out["status"].tolist() == [0, 0]
    assert np.all(out["margin"] > 1e-3) and np.all(out["delta"] > 1e-4)

    def f(X_, W_, b_):
        return oracle.pcx(X_, W_, b_, T, off, tgt, 0, want_dX=False, want_dW=False,
                          want_db=False, beam=beam)["loss"]

    h = 1e-6
    for name, arr, grad in (("X", X, out["dX"]), ("W", W, out["dW"]), ("b", b, out["db"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = arr.copy(); ap[idx] += h
            am = arr.copy(); am[idx] -= h
            args_p = {"X": (ap, W, b), "W": (X, ap, b), "b": (X, W, ap)}[name]
            args_m = {"X": (am, W, b), "W": (X, am, b), "b": (X, W, am)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        err = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert err < 1e-6, (name, err)


def test_beam_batch_matches_per_utterance_and_delta():
    """The batch routine with a beam: per-utterance losses, the discarded mass
    delta_n = 1 - P_beta / P (by enumeration), exclusion of an unalignable
    utterance, and the empty-target utterance (a single alignment, never
    pruned)."""
    rng = np.random.default_rng(49)
    V, D = 4, 3
    T = [6, 2, 5, 6]
    ys = [[1, 2], [3, 3], [], [2, 1]]  # the second needs 3 frames
    M = sum(T)
    X = rng.normal(size=(M, D))
    W = rng.normal(scale=2.0, size=(V, D))
    b = rng.normal(size=V)
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate([np.asarray(y, np.int64) for y in ys])
    beam = 1.2
    out = oracle.pcx(X, W, b, T, off, tgt, 0, beam=beam, cols=[0, 1, 2, 3], want_gamma=True)
    assert out["status"].tolist() == [0, 1, 0, 0]
    assert out["utt_loss"][1] == 0.0 and math.isnan(out["delta"][1])
    assert np.all(out["dX"][6:8] == 0.0)
    row = 0
    total = 0.0
    for n, y in enumerate(ys):
        Zn = X[row:row + T[n]] @ W.T + b
        if n != 1:
            Pb, gam, P, _, _ = brute_force_beam(Zn, y, 0, beam)
            assert out["utt_loss"][n] == pytest.approx(-math.log(Pb), rel=1e-12)
            assert out["delta"][n] == pytest.approx(1.0 - Pb / P, rel=1e-9, abs=1e-15)
            np.testing.assert_allclose(out["gamma_cols"][row:row + T[n]], gam, rtol=1e-10,
                                       atol=1e-13)
            total += -math.log(Pb)
        row += T[n]
    assert out["delta"][2] == 0.0
    assert out["delta"][0] > 1e-6 or out["delta"][3] > 1e-6
    assert out["loss"] == pytest.approx(total, rel=1e-12)


# ----------------------------------------------------------- closed forms
def test_readme_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "readme_example.json")))
    ys = g["targets"]
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate(ys)
    U, rel, flags = oracle.select(g["V"], g["blank"], g["frame_counts"], off, tgt)
    e = g["expected"]
    assert U.tolist() == e["U"] and len(U) == e["K"]
    assert rel.tolist() == e["relabeled"]
    assert flags.tolist() == e["alignable"]
    for n, y in enumerate(ys):
        assert repeats(y) == e["repeat_pairs"][n]
        T = g["frame_counts"][n]
        assert math.comb(T + len(y) - repeats(y), 2 * len(y)) == e["alignment_counts"][n]
    # uniform logits: W = 0, b = 0
    M = sum(g["frame_counts"])
    out = oracle.pcx(np.ones((M, g["D"])), np.zeros((g["V"], g["D"])), np.zeros(g["V"]),
                     g["frame_counts"], off, tgt, g["blank"])
    np.testing.assert_allclose(out["utt_loss"], e["uniform_logit_losses"]["values"],
                               rtol=1e-13)


@pytest.mark.parametrize("T,L,rep,V", [(300, 75, 10, 50), (880, 220, 0, 64),
                                       (1100, 366, 40, 64), (57, 28, 27, 7)])
def test_uniform_logits_closed_form(T, L, rep, V):
    """p = 1/V everywhere, so -log P = T log V - log C(T + L - r, 2L)."""
    rng = np.random.default_rng(T)
    # a target of length L with exactly `rep` adjacent repeats
    y = [1]
    while len(y) < L:
        if repeats(y) < rep:
            y.append(y[-1])
        else:
            nxt = int(rng.integers(1, V))
            while nxt == y[-1]:
                nxt = int(rng.integers(1, V))
            y.append(nxt)
    assert repeats(y) == rep and len(y) == L and L + rep <= T
    Z = np.zeros((T, V))
    r = oracle.ctc_logits(Z, y, 0, want_grad=False)
    lc = math.lgamma(T + L - rep + 1) - math.lgamma(2 * L + 1) - math.lgamma(T - L - rep + 1)
    assert r["loss"] == pytest.approx(T * math.log(V) - lc, rel=1e-12)


def test_single_alignment_forced_path():
    """T = |y| + r: the only alignment is y with one blank between repeats."""
    rng = np.random.default_rng(5)
    y = [2, 2, 5, 1, 1, 1, 3]
    r = repeats(y)
    path = []
    for i, v in enumerate(y):
        if i > 0 and y[i - 1] == v:
            path.append(0)
        path.append(v)
    T = len(path)
    assert T == len(y) + r
    Z = rng.normal(scale=3.0, size=(T, 7))
    out = oracle.ctc_logits(Z, y, 0)
    lam = np.log(np.sum(np.exp(Z), 1))
    lp = Z - lam[:, None]
    assert out["loss"] == pytest.approx(-sum(lp[t, v] for t, v in enumerate(path)), rel=1e-13)
    onehot = np.zeros_like(Z)
    onehot[np.arange(T), path] = 1.0
    np.testing.assert_allclose(out["gamma"], onehot, atol=1e-13)


def test_empty_target():
    rng = np.random.default_rng(6)
    Z = rng.normal(size=(9, 5))
    out = oracle.ctc_logits(Z, [], 2)
    lp = Z - np.log(np.sum(np.exp(Z), 1))[:, None]
    assert out["status"] == 0
    assert out["loss"] == pytest.approx(-lp[:, 2].sum(), rel=1e-13)
    g = np.zeros_like(Z)
    g[:, 2] = 1.0
    np.testing.assert_allclose(out["gamma"], g, atol=1e-14)


# ------------------------------------------------------ finite differences
def test_finite_differences_head_gradients():
    rng = np.random.default_rng(8)
    V, D = 5, 3
    T = [6, 4, 2]
    ys = [[1, 3], [2, 2], [4, 4]]  # last one is unalignable (needs 3 frames)
    M = sum(T)
    X = rng.normal(size=(M, D))
    W = rng.normal(size=(V, D))
    b = rng.normal(size=V)
    off = np.concatenate([[0], np.cumsum([len(y) for y in ys])])
    tgt = np.concatenate(ys)
    g = 0.7
    out = oracle.pcx(X, W, b, T, off, tgt, 0, grad=g)
    assert out["status"].tolist() == [0, 0, 1]

    def f(X_, W_, b_):
        return g * oracle.pcx(X_, W_, b_, T, off, tgt, 0, want_dX=False, want_dW=False,
                              want_db=False)["loss"]

    h = 1e-5
    for name, arr, grad in (("X", X, out["dX"]), ("W", W, out["dW"]), ("b", b, out["db"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap = arr.copy(); ap[idx] += h
            am = arr.copy(); am[idx] -= h
            args_p = {"X": (ap, W, b), "W": (X, ap, b), "b": (X, W, ap)}[name]
            args_m = {"X": (am, W, b), "W": (X, am, b), "b": (X, W, am)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        err = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert err < 1e-7, (name, err)
    # rows of the unalignable utterance receive exactly zero gradient
    assert np.all(out["dX"][10:12] == 0.0)


# -------------------------------------------------------- Proposition 1
@pytest.mark.parametrize("seed,V,blank", [(0, 9, 0), (1, 12, 11), (2, 7, 3)])
def test_proposition1_reduced_equals_full(seed, V, blank):
    rng = np.random.default_rng(seed)
    T = 10
    nonblank = [v for v in range(V) if v != blank]
    y = [int(v) for v in rng.choice(nonblank[:4], size=4)]
    Z = rng.normal(scale=2.0, size=(T, V))
    full = oracle.ctc_logits(Z, y, blank)
    # selected classes: blank first, then ascending distinct labels
    Usel = [blank] + sorted(set(y))
    comp = [v for v in range(V) if v not in Usel]
    assert comp, "test needs a nonempty complement"
    zc = Z[:, comp]
    other = zc.max(1) + np.log(np.sum(np.exp(zc - zc.max(1, keepdims=True)), 1))
    R = np.concatenate([Z[:, Usel], other[:, None]], axis=1)    # Eq. 4
    yr = [Usel.index(v) for v in y]
    red = oracle.ctc_logits(R, yr, 0)
    # pooling preserves the normalizer
    np.testing.assert_allclose(red["lambda"], full["lambda"], rtol=1e-14)
    assert red["loss"] == pytest.approx(full["loss"], rel=1e-13)
    # gradient: selected columns directly; the other column is spread over
    # the complement with weights exp(Z_v - R_other) (Eq. 11)
    dZ = np.zeros_like(Z)
    dZ[:, Usel] = red["dZ"][:, :len(Usel)]
    dZ[:, comp] = red["dZ"][:, -1:] * np.exp(zc - other[:, None])
    np.testing.assert_allclose(dZ, full["dZ"], rtol=1e-11, atol=1e-14)
    # complement classes keep gradient p_v (zero occupancy)
    p = np.exp(Z - full["lambda"][:, None])
    np.testing.assert_allclose(full["dZ"][:, comp], p[:, comp], rtol=1e-12)


# ------------------------------------------------------------- invariants
def _random_batch(seed, V=11, D=4, N=5, blank=0):
    b = workloads.make_random(seed, N=N, T_lo=3, T_hi=12, V=V, D=D, blank=blank,
                              len_div=3.0, zipf_s=0.5)
    return b


def _run(bt, grad=1.0, **kw):
    return oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                      grad=grad, **kw)


def test_gradient_rows_sum_to_zero_and_unalignable_zero():
    bt = workloads.make_random(3, N=4, T_lo=4, T_hi=9, V=8, D=3, len_div=2.0,
                               frame_counts=[6, 5, 2, 9], target_lengths=[3, 2, 2, 4],
                               labels=[1, 2, 3, 4, 4, 5, 5, 1, 2, 3, 4])
    _, _, flags = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    assert flags.tolist() == [True, True, False, True]
    M = bt.M
    out = _run(bt, cols=list(range(bt.V)), want_gamma=True)
    p = np.exp(out["logp_cols"])
    dZ = p - out["gamma_cols"]
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    for n in range(bt.N):
        rows = slice(row_off[n], row_off[n + 1])
        if flags[n]:
            np.testing.assert_allclose(dZ[rows].sum(1), 0.0, atol=1e-14)
            np.testing.assert_allclose(out["gamma_cols"][rows].sum(1), 1.0, rtol=1e-14)
        else:
            assert np.all(out["gamma_cols"][rows] == 0.0)
            assert np.all(out["dX"][rows] == 0.0)
            assert out["utt_loss"][n] == 0.0 and out["status"][n] == 1
    np.testing.assert_allclose(out["db"].sum(), 0.0, atol=1e-12)
    np.testing.assert_allclose(out["dW"].sum(0), 0.0, atol=1e-12)
    assert M == row_off[-1]


def test_bias_shift_invariance():
    bt = _random_batch(4)
    a = _run(bt)
    bt.b = bt.b.astype(np.float64) + 3.25  # exact in FP64
    c = _run(bt)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    for k in ("dX", "dW", "db"):
        np.testing.assert_allclose(c[k], a[k], rtol=1e-10, atol=1e-13)


def test_class_permutation_invariance():
    bt = _random_batch(5, V=9, blank=0)
    a = _run(bt)
    rng = np.random.default_rng(0)
    perm = np.concatenate([[0], 1 + rng.permutation(bt.V - 1)])  # keep blank at 0
    W2 = np.zeros_like(bt.W); W2[perm] = bt.W
    b2 = np.zeros_like(bt.b); b2[perm] = bt.b
    c = oracle.pcx(bt.X, W2, b2, bt.frame_counts, bt.tgt_off, perm[bt.tgt], 0)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["dW"][perm], a["dW"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(c["db"][perm], a["db"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(c["dX"], a["dX"], rtol=1e-10, atol=1e-13)


def test_utterance_permutation_and_batch_additivity():
    bt = _random_batch(6, N=4)
    a = _run(bt)
    order = [2, 0, 3, 1]
    pb = workloads.sample_utterances(bt, order)
    c = _run(pb)
    assert c["loss"] == pytest.approx(a["loss"], rel=1e-13)
    np.testing.assert_allclose(c["utt_loss"], a["utt_loss"][order], rtol=1e-13)
    np.testing.assert_allclose(c["dW"], a["dW"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(c["db"], a["db"], rtol=1e-10, atol=1e-13)
    # additivity: each utterance alone gives the same per-utterance loss and
    # the head gradients add up
    dW = np.zeros_like(a["dW"])
    for n in range(bt.N):
        s = _run(workloads.sample_utterances(bt, [n]))
        assert s["loss"] == pytest.approx(a["utt_loss"][n], rel=1e-13)
        dW += s["dW"]
    np.testing.assert_allclose(dW, a["dW"], rtol=1e-10, atol=1e-13)


def test_grad_scale_is_linear():
    bt = _random_batch(7)
    a = _run(bt, grad=1.0)
    c = _run(bt, grad=-2.5)
    for k in ("dX", "dW", "db"):
        np.testing.assert_allclose(c[k], -2.5 * a[k], rtol=1e-13, atol=1e-15)


# --------------------------------------------------- selection and flags
@pytest.mark.parametrize("seed,V,blank", [(0, 50, 0), (1, 50, 49), (2, 31, 7), (3, 6, 0)])
def test_select_matches_set_arithmetic(seed, V, blank):
    rng = np.random.default_rng(seed)
    N = 7
    T = rng.integers(1, 15, size=N)
    L = rng.integers(0, 8, size=N)
    nonblank = np.array([v for v in range(V) if v != blank])
    tgt = rng.choice(nonblank[: max(2, V // 3)], size=int(L.sum()))
    off = np.concatenate([[0], np.cumsum(L)])
    U, rel, flags = oracle.select(V, blank, T, off, tgt)
    U_ref = [blank] + sorted(set(int(v) for v in tgt))
    assert U.tolist() == U_ref
    assert rel.tolist() == [U_ref.index(int(v)) for v in tgt]
    for n in range(N):
        y = tgt[off[n]:off[n + 1]].tolist()
        assert flags[n] == (len(y) + repeats(y) <= T[n])


def test_select_rejects_bad_targets():
    with pytest.raises(ValueError):
        oracle.select(5, 0, [3], [0, 1], [0])      # blank inside a target
    with pytest.raises(ValueError):
        oracle.select(5, 0, [3], [0, 1], [5])      # label out of range
    with pytest.raises(ValueError):
        oracle.select(5, 0, [0], [0, 1], [1])      # empty utterance
