"""The recompute's unselected-first column order (small vocabularies).

"Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", App. B.2:
the backward reuses S, so a selected class's logit gradient needs only S,
the occupancy and g, never the recomputed logit.  When a chunk can be
expected to hold a tile's worth of selected classes (K * min(C, V) >= V *
tile width) and at least a quarter of the classes are selected, the library
walks the chunk's columns unselected-first: the selected classes then fill
whole tiles, which skip the product and go to a pass of their own.  The same batch run with a narrow chunk (C = 64, below
one tile width) takes the in-order recompute.  Both are held to the oracle's
bar, to rounding-level agreement with each other, and the profiler's launch
counts show which path ran.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro, run_oracle, run_pcx, to_device, tolerance

pytestmark = pytest.mark.gpu

V = 300


def _batch(dtype):
    # uniform labels (zipf_s = 0) over a small vocabulary: nearly every class
    # is selected
    return workloads.make_random(21 if dtype == "f32" else 22, N=10, T_lo=300, T_hi=400, V=V,
                                 D=64 if dtype == "f32" else 96, chunk=512, dtype=dtype,
                                 zipf_s=0.0)


def _recompute_launches(bt, grouped):
    import torch
    from vocabulary_ctc_loss_amd import Context
    X, W, b, off, tgt, fc = to_device(bt)
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    db = torch.empty_like(b) if b is not None else None
    c = Context()
    try:
        c.set_formulation(grouped)
        c.profile_enable(True)
        c.profile_reset()
        c.forward(X, W, b, off, tgt, fc, bt.blank, bt.chunk)
        c.backward(1.0, dX, dW, db)
        torch.cuda.synchronize()
        return c.profile_read()["bwd_recompute_dz"][1]
    finally:
        c.close()


@pytest.mark.parametrize("dtype,grouped", [("f32", False), ("f32", True), ("bf16", False)])
def test_selected_first_order_matches_oracle_and_in_order(dtype, grouped):
    bt = _batch(dtype)
    U, _, _ = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    K = len(U)
    tile = 128 if dtype == "f32" else 256  # column tile of the recompute core
    print("dtype", dtype, "grouped", grouped, "K", K, "M", bt.M, flush=True)
    assert K * min(bt.chunk, V) >= V * tile and 4 * K >= V  # the ordered path
    narrow = dataclasses.replace(bt, chunk=64)
    assert K * 64 < V * tile                     # the in-order path
    # one chunk group: the order pass and the recompute; five groups in order
    assert _recompute_launches(bt, grouped) == 2
    assert _recompute_launches(narrow, grouped) == (V + 63) // 64

    ordered = run_pcx(bt, grouped=grouped, getters="light")
    in_order = run_pcx(narrow, grouped=grouped, getters="light")
    ref = run_oracle(bt, cols=U)
    tol = tolerance(bt)
    assert ordered["loss"] == in_order["loss"]  # the forward does not depend on C
    assert abs(ordered["loss"] - ref["loss"]) <= tol * abs(ref["loss"])
    for k in ("dX", "dW", "db"):
        assert rel_fro(ordered[k], ref[k]) <= tol, k
        assert rel_fro(in_order[k], ref[k]) <= tol, k
        # the same per-element formulas; only the summation grouping differs
        assert rel_fro(ordered[k], in_order[k]) <= (1e-6 if dtype == "f32" else 1e-2), k
    assert np.all(np.isfinite(ordered["dX"]))
