"""Parity of the HIP path (through the C ABI) with the CPU FP64 oracle.

Bar: U, relabelled targets and alignability flags bit-exact; loss relative
error <= 1e-5 and dX / dW / db relative Frobenius error <= 1e-5 for fp32
inputs, <= 2e-2 for bf16 inputs; all-zero references (excluded utterances)
must come back as exact zeros.  Intermediates are checked too: the FP64
normalizer lambda, the FP32 scores S = Z[:, U] - lambda and the occupancies
gamma on the selected classes.
"""
import zlib

import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro, run_oracle, run_pcx, tolerance

pytestmark = pytest.mark.gpu


def _labels(rng, n, V, blank, k=None):
    ids = np.array([v for v in range(V) if v != blank])
    if k is not None:
        ids = ids[:k]
    return rng.choice(ids, size=n).astype(np.int32)


def case(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "readme":
        return workloads.make("tiny", seed=0)
    if name == "tiles":      # several M tiles, ragged D (K tail), ragged chunks
        return workloads.make_random(1, N=6, T_lo=40, T_hi=130, V=700, D=72, chunk=200)
    if name == "spans":      # several normalizer spans, ragged last span
        return workloads.make_random(2, N=4, T_lo=60, T_hi=160, V=5000, D=64, chunk=1024)
    if name == "blank_last":
        return workloads.make_random(3, N=5, T_lo=20, T_hi=90, V=300, D=64, blank=299, chunk=64)
    if name == "blank_mid":
        return workloads.make_random(4, N=5, T_lo=20, T_hi=90, V=257, D=40, blank=100, chunk=100)
    if name == "odd_D":      # D not a multiple of the vector width: scalar staging path
        return workloads.make_random(5, N=3, T_lo=10, T_hi=50, V=77, D=13, chunk=30)
    if name == "v_lt_c":
        return workloads.make_random(6, N=3, T_lo=30, T_hi=70, V=50, D=32, chunk=4096)
    if name == "all_classes":   # K = V
        T = [60, 50, 70]
        L = [13, 13, 13]
        labels = np.arange(1, 40, dtype=np.int32)
        return workloads.make_random(7, N=3, T_lo=0, T_hi=0, V=40, D=32, chunk=16,
                                     frame_counts=T, target_lengths=L, labels=labels)
    if name == "unalignable_mix":
        # targets: [1 1 2 2] needs 6 frames; [3 4 5] needs 3; [6 6 6] needs 5; [7] needs 1
        T = [5, 3, 4, 9, 40]
        ys = [[1, 1, 2, 2], [3, 4, 5], [6, 6, 6], [7], list(_labels(rng, 12, 60, 0))]
        L = [len(y) for y in ys]
        return workloads.make_random(8, N=5, T_lo=0, T_hi=0, V=60, D=24, chunk=32,
                                     frame_counts=T, target_lengths=L,
                                     labels=np.concatenate(ys).astype(np.int32))
    if name == "single_alignment":   # T = L + r for every utterance
        ys = []
        T = []
        for n in range(4):
            y = list(_labels(rng, 30 + 10 * n, 90, 0, k=6))  # few classes: many repeats
            r = sum(1 for i in range(len(y) - 1) if y[i] == y[i + 1])
            ys.append(y)
            T.append(len(y) + r)
        return workloads.make_random(9, N=4, T_lo=0, T_hi=0, V=90, D=48, chunk=64,
                                     frame_counts=T, target_lengths=[len(y) for y in ys],
                                     labels=np.concatenate(ys).astype(np.int32))
    if name == "empty_targets":
        T = [7, 20, 1, 33]
        ys = [[], list(_labels(rng, 5, 30, 0)), [], list(_labels(rng, 8, 30, 0))]
        return workloads.make_random(10, N=4, T_lo=0, T_hi=0, V=30, D=16, chunk=8,
                                     frame_counts=T, target_lengths=[len(y) for y in ys],
                                     labels=np.concatenate([np.asarray(y, np.int32) for y in ys]))
    if name == "long_targets":   # 2L + 1 > 1024 states: several states per thread
        T = [1300, 700]
        L = [600, 300]
        return workloads.make_random(11, N=2, T_lo=0, T_hi=0, V=500, D=32, chunk=256,
                                     frame_counts=T, target_lengths=L)
    if name == "max_target":   # the longest target accepted: 4095 states, 4 per thread
        T = [4200, 300]
        L = [2047, 50]
        return workloads.make_random(22, N=2, T_lo=0, T_hi=0, V=60, D=32, chunk=64,
                                     frame_counts=T, target_lengths=L)
    if name == "many_utts":    # several hundred short utterances: wide DP and occupancy grids
        return workloads.make_random(23, N=400, T_lo=5, T_hi=30, V=300, D=32, chunk=128,
                                     len_div=3.0)
    if name == "one_utt":
        return workloads.make_random(12, N=1, T_lo=200, T_hi=200, V=1000, D=64, chunk=512)
    if name == "bf16_llm":
        return workloads.make_random(13, N=4, T_lo=50, T_hi=120, V=3000, D=256, blank=2999,
                                     chunk=1024, dtype="bf16", llm_head=True, len_div=3.0,
                                     zipf_s=1.05)
    if name == "bf16_head":
        return workloads.make_random(14, N=3, T_lo=30, T_hi=90, V=900, D=136, chunk=256,
                                     dtype="bf16")
    # bf16 with D and the chunk width not multiples of 8: scalar staging and
    # the element-wise weight-chunk transpose
    if name == "bf16_odd_D":
        return workloads.make_random(24, N=3, T_lo=10, T_hi=50, V=77, D=13, chunk=30,
                                     dtype="bf16")
    # bf16 heads with D and the chunk width multiples of 64 run on the 256 x 256
    # core: one ragged frame tile and one ragged vocabulary tile, the chunk
    # narrower than a tile
    if name == "bf16_big_ragged":
        return workloads.make_random(15, N=2, T_lo=40, T_hi=60, V=200, D=64, chunk=128,
                                     dtype="bf16")
    # several frame tiles, chunks 320 / 320 / 60 (the last padded to 64), with
    # bias, dW and db
    if name == "bf16_big_grads":
        return workloads.make_random(16, N=5, T_lo=60, T_hi=130, V=700, D=128, chunk=320,
                                     dtype="bf16")
    # every class selected: many selected columns per wavefront
    if name == "bf16_big_dense":
        T = [200, 200, 200, 200]
        L = [75, 75, 75, 74]
        labels = np.arange(1, 300, dtype=np.int32)
        return workloads.make_random(17, N=4, T_lo=0, T_hi=0, V=300, D=64, chunk=64,
                                     dtype="bf16", frame_counts=T, target_lengths=L,
                                     labels=labels)
    # several normalizer spans of eight vocabulary tiles each, LLM-style head
    if name == "bf16_big_spans":
        return workloads.make_random(18, N=3, T_lo=100, T_hi=200, V=5000, D=128, blank=4999,
                                     chunk=1024, dtype="bf16", llm_head=True, len_div=3.0,
                                     zipf_s=1.05)
    # the 14B LLM head width (D = 5120)
    if name == "bf16_big_d5120":
        return workloads.make_random(19, N=3, T_lo=60, T_hi=120, V=2000, D=5120, blank=1999,
                                     chunk=1024, dtype="bf16", llm_head=True, len_div=3.0,
                                     zipf_s=1.05)
    # fp32 states with a bf16-stored head (fp32 projections on W widened one
    # chunk or 2048-class span at a time): several spans and chunks, ragged
    if name == "f32_bf16w_head":
        return workloads.make_random(20, N=4, T_lo=40, T_hi=110, V=5000, D=64, chunk=1024,
                                     dtype="f32_bf16w")
    # dX alone on the 256 x 256 core with at least two frame tiles: frames in
    # two parts, chunks in pairs (the last pair ragged: 7 x 128 + 4)
    if name == "bf16_big_parts":
        return workloads.make_random(25, N=6, T_lo=100, T_hi=140, V=900, D=64, chunk=128,
                                     dtype="bf16")
    # V a whole number of chunks (the last chunk full width; chunk pairs
    # exact for a dX-only backward)
    if name == "exact_chunks":
        return workloads.make_random(28, N=5, T_lo=60, T_hi=110, V=1024, D=64, chunk=256)
    if name == "bf16_big_exact":
        return workloads.make_random(29, N=6, T_lo=100, T_hi=140, V=1024, D=64, chunk=256,
                                     dtype="bf16")
    if name == "f32_bf16w_parts":
        return workloads.make_random(26, N=5, T_lo=60, T_hi=110, V=1500, D=64, chunk=256,
                                     dtype="f32_bf16w")
    if name == "f32_bf16w_llm":
        return workloads.make_random(21, N=3, T_lo=50, T_hi=100, V=3000, D=128, blank=2999,
                                     chunk=4096, dtype="f32_bf16w", llm_head=True,
                                     len_div=3.0, zipf_s=1.05)
    raise KeyError(name)


CASES = ["readme", "tiles", "spans", "blank_last", "blank_mid", "odd_D", "v_lt_c",
         "all_classes", "unalignable_mix", "single_alignment", "empty_targets", "long_targets",
         "max_target", "many_utts", "one_utt", "bf16_llm", "bf16_head", "bf16_odd_D",
         "exact_chunks", "bf16_big_exact", "bf16_big_ragged", "bf16_big_grads", "bf16_big_dense",
         "bf16_big_spans", "bf16_big_d5120", "f32_bf16w_head", "f32_bf16w_llm"]


@pytest.mark.parametrize("name", CASES)
def test_parity_with_oracle(name):
    bt = case(name)
    print("case", name, "N", bt.N, "M", bt.M, "D", bt.D, "V", bt.V, "C", bt.chunk, bt.dtype,
          flush=True)
    got = run_pcx(bt)
    U, rel, flags = __import__("oracle").select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off,
                                                bt.tgt)
    ref = run_oracle(bt, cols=U, want_gamma=True)
    tol = tolerance(bt)
    # integer outputs: bit-exact
    assert got["U"].tolist() == U.tolist()
    assert got["rel"].tolist() == rel.tolist()
    assert got["flags"].tolist() == flags.tolist()
    assert got["info"]["K"] == len(U)
    assert got["status"].tolist() == ref["status"].tolist()
    # loss and per-utterance losses
    assert abs(got["loss"] - ref["loss"]) <= tol * max(abs(ref["loss"]), 1e-30), \
        (got["loss"], ref["loss"])
    assert rel_fro(got["utt_loss"], ref["utt_loss"]) <= tol
    # intermediates
    if bt.dtype != "bf16":
        np.testing.assert_allclose(got["lam"], ref["lambda"], rtol=0, atol=2e-5)
        np.testing.assert_allclose(got["S"], ref["logp_cols"].T, rtol=0, atol=2e-5)
        np.testing.assert_allclose(got["Gam"], ref["gamma_cols"].T, rtol=0, atol=1e-5)
    else:
        # bf16 operands are exact in both; the difference is the fp32
        # accumulation of the D products
        np.testing.assert_allclose(got["lam"], ref["lambda"], rtol=0, atol=2e-4)
        np.testing.assert_allclose(got["S"], ref["logp_cols"].T, rtol=0, atol=2e-4)
    # gradients (dW and db of a bf16-stored head are bf16 outputs)
    for k in ("dX", "dW", "db"):
        if ref[k] is None or got[k] is None:
            continue
        e = rel_fro(got[k], ref[k])
        kt = 2e-2 if (bt.dtype == "f32_bf16w" and k != "dX") else tol
        assert e <= kt, (k, e)
    # excluded utterances: exact zeros in their dX rows
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    for n in range(bt.N):
        if ref["status"][n] != 0:
            assert np.all(got["dX"][row_off[n]:row_off[n + 1]] == 0.0)


@pytest.mark.parametrize("name", ["tiles", "bf16_big_grads"])
def test_nonfinite_input_utterance_is_excluded(name):
    """One utterance's encoder states are NaN (a precondition violation): its
    loss comes out nonfinite, so it is excluded like the pages' nonfinite
    utterances (zero loss, zero dX rows, counted), and every other
    utterance's loss and dX rows are unchanged.  dW and db mix all rows
    (0 * NaN) and are not checked."""
    import dataclasses
    bt = case(name)
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    X = bt.X.copy()
    X[row_off[2]:row_off[3]] = np.nan
    bt = dataclasses.replace(bt, X=X)
    got = run_pcx(bt, want_dW=False, want_db=False, getters="light")
    ref = run_oracle(bt, want_dW=False, want_db=False)
    tol = tolerance(bt)
    assert ref["status"][2] == 2 and got["status"].tolist() == ref["status"].tolist()
    assert got["info"]["n_nonfinite"] == 1
    assert got["utt_loss"][2] == 0.0
    assert abs(got["loss"] - ref["loss"]) <= tol * abs(ref["loss"])
    assert np.all(got["dX"][row_off[2]:row_off[3]] == 0.0)
    keep = np.ones(bt.M, bool)
    keep[row_off[2]:row_off[3]] = False
    assert rel_fro(got["dX"][keep], ref["dX"][keep]) <= tol


@pytest.mark.parametrize("name,grouped,where", [
    ("tiles", False, "unselected"), ("tiles", True, "unselected"), ("tiles", False, "selected"),
    ("tiles", True, "selected"), ("bf16_big_grads", False, "unselected"),
    ("bf16_big_grads", False, "bias")])
def test_nonfinite_head_row_poisons_every_frame(name, grouped, where):
    """A NaN row of the head (or a NaN bias entry) makes every logit of that
    class NaN, so every frame's normalizer, and with it every alignable
    utterance's loss, is nonfinite: the oracle marks them all nonfinite and
    excludes them.  The library must do the same rather than let the maximum
    and the clamped exponential drop the NaN and report a finite loss (the
    pages replace nonfinite per-utterance losses by zero, App. B.1)."""
    import dataclasses
    bt = case(name)
    U, _, _ = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    sel = set(int(u) for u in U)
    v = int(U[-1]) if where == "selected" else next(c for c in range(bt.V) if c not in sel)
    W = bt.W.copy()
    b = None if bt.b is None else bt.b.copy()
    if where == "bias":
        if b is None:
            b = np.zeros(bt.V, np.float32)
        b[v] = np.nan
    else:
        W[v] = np.nan
    bt = dataclasses.replace(bt, W=W, b=b)
    print("case", name, "grouped", grouped, "nan", where, v, flush=True)
    got = run_pcx(bt, want_dX=False, want_dW=False, want_db=False, getters="light",
                  grouped=grouped)
    ref = run_oracle(bt, want_dW=False, want_db=False)
    assert np.all(ref["status"] != 0)
    assert got["status"].tolist() == ref["status"].tolist()
    assert got["loss"] == 0.0 and ref["loss"] == 0.0
    assert got["info"]["n_nonfinite"] == int(np.sum(ref["status"] == 2))
    assert np.all(got["utt_loss"] == 0.0)


@pytest.mark.parametrize("name,grouped", [("tiles", False), ("tiles", True),
                                          ("bf16_big_parts", False), ("f32_bf16w_parts", False),
                                          ("exact_chunks", False), ("bf16_big_exact", False)])
def test_dx_only_frame_parts(name, grouped):
    """With dX alone requested the backward takes the frames in two parts and
    the chunks in pairs (a half-height block of two chunks in the same
    M x C elements): dX matches the oracle, and the all-gradients call (one
    part, single chunks) up to the summation grouping."""
    bt = case(name)
    assert bt.M >= 2 * (256 if name.startswith("bf16_big") else 128) and bt.V > 2 * bt.chunk
    print("case", name, "grouped", grouped, "M", bt.M, "V", bt.V, "C", bt.chunk, flush=True)
    got = run_pcx(bt, want_dW=False, want_db=False, getters="light", grouped=grouped)
    full = run_pcx(bt, getters="light", grouped=grouped)
    ref = run_oracle(bt, want_dW=False, want_db=False)
    tol = tolerance(bt)
    assert got["loss"] == full["loss"]
    assert rel_fro(got["dX"], ref["dX"]) <= tol
    assert rel_fro(got["dX"], full["dX"]) <= (1e-2 if bt.dtype == "bf16" else 1e-6)


def test_grad_scaling_and_skipped_outputs():
    bt = case("tiles")
    ref = run_oracle(bt, grad=-0.37)
    got = run_pcx(bt, grad=-0.37, want_dW=False, getters=False)
    assert got["dW"] is None
    assert rel_fro(got["dX"], ref["dX"]) <= 1e-5
    assert rel_fro(got["db"], ref["db"]) <= 1e-5


@pytest.mark.parametrize("name", ["spans", "bf16_big_spans", "bf16_head"])
def test_deterministic_bitwise(name):
    bt = case(name)
    a = run_pcx(bt, getters=False)
    b = run_pcx(bt, getters=False)
    assert a["loss"] == b["loss"]
    for k in ("dX", "dW", "db"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name,other,tol", [
    ("tiles", 700, 1e-6),
    # bf16: 1000 is not a multiple of 64, so the backward products leave the
    # 256 x 256 core while the forward stays on it
    ("bf16_big_spans", 1000, 2e-2),
])
def test_chunk_width_changes_only_rounding(name, other, tol):
    bt = case(name)
    a = run_pcx(bt, getters=False)
    import dataclasses
    b = run_pcx(dataclasses.replace(bt, chunk=other), getters=False)
    assert a["loss"] == b["loss"]  # forward does not depend on C
    for k in ("dX", "dW", "db"):
        assert rel_fro(b[k], a[k]) <= tol, k


@pytest.mark.parametrize("name", ["readme", "blank_mid", "unalignable_mix", "bf16_llm"])
def test_blank_offset_grad_matches_db_at_blank(name):
    """d(loss)/d(eta) for a blank-logit offset equals the oracle's db[blank]."""
    import oracle
    bt = case(name)
    ref = oracle.pcx(bt.X, bt.W, bt.b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank,
                     grad=0.75, want_dX=False, want_dW=False, want_db=True, want_lambda=False)
    want = ref["db"][bt.blank]
    import torch
    from pcx_harness import to_device
    from vocabulary_ctc_loss_amd import Context
    X, W, b, off, tgt, fc = to_device(bt)
    ctx = Context()
    try:
        ctx.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        # without a pcx_backward before it, then after one
        got = ctx.blank_offset_grad(0.75)
        ctx.backward(0.75, torch.empty_like(X))
        again = ctx.blank_offset_grad(0.75)
    finally:
        ctx.close()
    assert got == again
    assert abs(got - want) <= tolerance(bt) * max(abs(want), 1e-3), (got, want)


def test_context_reuse_and_repeated_backward():
    from vocabulary_ctc_loss_amd import Context
    ctx = Context()
    try:
        for name in ("tiles", "readme", "spans"):
            bt = case(name)
            ref = run_oracle(bt)
            got = run_pcx(bt, ctx=ctx, getters=False)
            assert abs(got["loss"] - ref["loss"]) <= 1e-5 * abs(ref["loss"])
            assert rel_fro(got["dW"], ref["dW"]) <= 1e-5
    finally:
        ctx.close()


def test_empty_batch():
    import torch
    from vocabulary_ctc_loss_amd import Context
    dev = "cuda:0"
    X = torch.zeros((0, 16), device=dev)
    W = torch.randn((10, 16), device=dev)
    b = torch.randn((10,), device=dev)
    off = torch.zeros(1, dtype=torch.int32, device=dev)
    tgt = torch.zeros(0, dtype=torch.int32, device=dev)
    fc = torch.zeros(0, dtype=torch.int32, device=dev)
    c = Context()
    loss, info = c.forward(X, W, b, off, tgt, fc, 0, 4)
    assert loss == 0.0 and info["K"] == 1
    dW = torch.full_like(W, 7.0)
    db = torch.full_like(b, 7.0)
    c.backward(1.0, None, dW, db)
    torch.cuda.synchronize()
    assert torch.all(dW == 0) and torch.all(db == 0)
    c.close()


def test_device_side_validation_errors():
    import torch
    from vocabulary_ctc_loss_amd import Context, PcxError
    bt = case("readme")
    from pcx_harness import to_device
    X, W, b, off, tgt, fc = to_device(bt)
    c = Context()
    with pytest.raises(PcxError) as e:
        bad = tgt.clone()
        bad[1] = 0  # blank inside a target
        c.forward(X, W, b, off, bad, fc, 0, 4)
    assert e.value.status == 3
    with pytest.raises(PcxError) as e:
        bad = tgt.clone()
        bad[0] = 6  # label == V
        c.forward(X, W, b, off, bad, fc, 0, 4)
    assert e.value.status == 3
    with pytest.raises(PcxError) as e:
        badfc = fc.clone()
        badfc[0] = 11  # frame counts no longer sum to M
        c.forward(X, W, b, off, tgt, badfc, 0, 4)
    assert e.value.status == 4
    with pytest.raises(PcxError) as e:
        badfc = fc.clone()
        badfc[0] = 0
        badfc[1] = 21
        c.forward(X, W, b, off, tgt, badfc, 0, 4)
    assert e.value.status == 4
    with pytest.raises(ValueError, match="dtypes"):   # fp16: the binding refuses it
        c.forward(X.half(), W.half(), b.half(), off, tgt, fc, 0, 4)
    with pytest.raises(PcxError) as e:   # failed forward leaves no state for backward
        c.backward(1.0, torch.empty_like(X))
    assert e.value.status == 5
    # and the context still works afterwards
    loss, _ = c.forward(X, W, b, off, tgt, fc, 0, 4)
    assert np.isfinite(loss)
    c.close()


def test_target_limit_and_offset_errors():
    """A target one label over PCX_MAX_TARGET_LEN (2047) is refused with
    PCX_ERR_LIMIT (the longest accepted one is the max_target parity case);
    target offsets that do not start at 0, or decrease, with PCX_ERR_TARGET.
    The context stays usable."""
    import torch
    from vocabulary_ctc_loss_amd import Context, PcxError
    from pcx_harness import to_device
    bt = workloads.make_random(27, N=1, T_lo=0, T_hi=0, V=60, D=8, chunk=64,
                               frame_counts=[2100], target_lengths=[2048])
    X, W, b, off, tgt, fc = to_device(bt)
    c = Context()
    with pytest.raises(PcxError) as e:
        c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
    assert e.value.status == 7
    bt = case("readme")
    X, W, b, off, tgt, fc = to_device(bt)
    for bad_off in ([1, 3, 5], [0, 4, 3]):   # the valid offsets are [0, 3, 5]
        bad = torch.tensor(bad_off, dtype=torch.int32, device=X.device)
        with pytest.raises(PcxError) as e:
            c.forward(X, W, b, bad, tgt, fc, 0, 4)
        assert e.value.status == 3, bad_off
    loss, _ = c.forward(X, W, b, off, tgt, fc, 0, 4)
    assert np.isfinite(loss)
    c.close()


def test_profile_counts_and_mask():
    """Per-family event timing: launch counts per step follow the chunking
    (V = 700 in chunks of 200: four recompute, dX and dW launches per
    backward, one forward product, and one reduction launch: the reductions
    of the first three chunks run inside the next chunk's recompute launch),
    they accumulate over steps that read nothing, and a mask times only the
    families it names."""
    import torch
    from vocabulary_ctc_loss_amd import Context
    from pcx_harness import to_device
    bt = case("tiles")
    X, W, b, off, tgt, fc = to_device(bt)
    dX, dW, db = torch.empty_like(X), torch.empty_like(W), torch.empty_like(b)
    c = Context()
    c.profile_enable(True)
    c.profile_reset()
    steps = 5
    for _ in range(steps):
        c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        c.backward(1.0, dX, dW, db)
    prof = c.profile_read()
    for fam, per_step in (("fwd_gemm_lse", 1), ("ctc_alpha_beta", 1), ("bwd_recompute_dz", 4),
                          ("dx_gemm", 4), ("dw_gemm", 4), ("grad_reduce", 1)):
        ms, n = prof[fam]
        assert n == steps * per_step, (fam, n)
        assert ms > 0.0, fam
    c.profile_mask(["dx_gemm"])
    c.profile_reset()
    for _ in range(2):
        c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        c.backward(1.0, dX, dW, db)
    prof = c.profile_read()
    assert prof["dx_gemm"][1] == 8
    assert all(n == 0 for fam, (_, n) in prof.items() if fam != "dx_gemm")
    c.profile_enable(False)
    c.close()


def test_autograd_steps_reuse_pooled_contexts():
    """The autograd function leases a context per graph and gets it back
    when the graph is freed, so a training loop reuses sized workspaces.
    Steps alternate two batches of different shapes; one step holds two live
    graphs at once (a summed loss); one backward runs twice (retain_graph).
    Every gradient matches the oracle, and the pool stays small."""
    import gc
    import torch
    import vocabulary_ctc_loss_amd as pcx
    from pcx_harness import to_device
    batches = [case("blank_mid"), case("tiles")]
    devs = [to_device(bt) for bt in batches]
    refs = [run_oracle(bt, grad=1.0) for bt in batches]

    def loss_of(i):
        bt, (X, W, b, off, tgt, fc) = batches[i], devs[i]
        X, W, b = (t.detach().clone().requires_grad_(True) for t in (X, W, b))
        return pcx.pruned_ctc_loss(X, W, b, (off, tgt), fc, blank_id=bt.blank,
                                   chunk_size=bt.chunk), (X, W, b)

    def check(i, leaves, scale=1.0):
        for t, k in zip(leaves, ("dX", "dW", "db")):
            assert rel_fro(t.grad.double().cpu().numpy(), scale * refs[i][k]) <= 1e-5, (i, k)

    used = set()
    for step in range(4):
        i = step % 2
        loss, leaves = loss_of(i)
        used.add(id(loss.grad_fn.lease.ctx))
        loss.backward()
        check(i, leaves)
        del loss
        gc.collect()
    assert len(used) == 1  # one graph at a time: one context, reused
    la, va = loss_of(0)
    lb, vb = loss_of(1)
    (la + lb).backward()
    check(0, va)
    check(1, vb)
    loss, leaves = loss_of(1)
    loss.backward(retain_graph=True)
    loss.backward()
    check(1, leaves, scale=2.0)
    del la, lb, loss
    gc.collect()
    idle = pcx._POOL.get(torch.device("cuda:0").index, [])
    assert 1 <= len(idle) <= pcx._POOL_KEEP


def test_autograd_function():
    import torch
    from vocabulary_ctc_loss_amd import pruned_ctc_loss
    bt = case("blank_mid")
    from pcx_harness import to_device
    X, W, b, off, tgt, fc = to_device(bt)
    X.requires_grad_(True)
    W.requires_grad_(True)
    b.requires_grad_(True)
    loss = pruned_ctc_loss(X, W, b, (off, tgt), fc, blank_id=bt.blank, chunk_size=bt.chunk)
    (2.0 * loss).backward()
    ref = run_oracle(bt, grad=2.0)
    assert loss.dtype == torch.float32
    assert abs(loss.item() - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    assert rel_fro(X.grad.double().cpu().numpy(), ref["dX"]) <= 1e-5
    assert rel_fro(W.grad.double().cpu().numpy(), ref["dW"]) <= 1e-5
    assert rel_fro(b.grad.double().cpu().numpy(), ref["db"]) <= 1e-5
