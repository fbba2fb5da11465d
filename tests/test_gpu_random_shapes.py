"""Parity with the oracle on seeded random shapes.

Each case draws its own sizes: vocabulary size (tens to thousands), head
width (multiples of 64, which the bf16 256 x 256 core takes, or not), chunk
width (a multiple of 64 or ragged), blank position, utterance count and
lengths, dtype (fp32, bf16, fp32 states with a bf16-stored head), the
formulation (direct or grouped) and, for every fourth seed, a backward that
wants dX alone (frames in parts, chunks in groups where the batch allows).
The bar is the one of test_gpu_parity.py.
The draws are fixed by the case seed, so a failure names a reproducible
shape.
"""
import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro, run_oracle, run_pcx, tolerance

pytestmark = pytest.mark.gpu

SEEDS = list(range(100, 356))


def draw(seed):
    rng = np.random.default_rng(seed)
    dtype = ["f32", "bf16", "f32_bf16w"][seed % 3]
    V = int(rng.choice([30, 97, 256, 700, 1500, 2600, 5000, 9000]))
    D = int(rng.choice([40, 64, 128, 136, 192, 256, 512]))
    chunk = int(rng.choice([64, 100, 128, 320, 512, 1024, 4096]))
    blank = int(rng.choice([0, V - 1, V // 2]))
    N = int(rng.integers(1, 7))
    T_lo = int(rng.integers(8, 60))
    T_hi = T_lo + int(rng.integers(0, 150))
    grouped = bool(seed % 2)
    bt = workloads.make_random(seed, N=N, T_lo=T_lo, T_hi=T_hi, V=V, D=D, blank=blank,
                               chunk=chunk, dtype=dtype, len_div=float(rng.choice([2.5, 3.0, 4.0])),
                               zipf_s=float(rng.choice([0.8, 1.1])))
    return bt, grouped


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_parity(seed):
    bt, grouped = draw(seed)
    full = seed % 4 != 3  # else dX alone
    print("seed", seed, bt.dtype, "grouped" if grouped else "direct", "N", bt.N, "M", bt.M,
          "D", bt.D, "V", bt.V, "C", bt.chunk, "blank", bt.blank,
          "all gradients" if full else "dX only", flush=True)
    got = run_pcx(bt, grouped=grouped, want_dW=full, want_db=full)
    U, rel, flags = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    ref = run_oracle(bt, cols=U, want_gamma=True, want_dW=full, want_db=full)
    tol = tolerance(bt)
    assert got["U"].tolist() == U.tolist()
    assert got["rel"].tolist() == rel.tolist()
    assert got["flags"].tolist() == flags.tolist()
    assert got["status"].tolist() == ref["status"].tolist()
    assert abs(got["loss"] - ref["loss"]) <= tol * max(abs(ref["loss"]), 1e-30)
    atol = 2e-4 if bt.dtype == "bf16" else 2e-5
    np.testing.assert_allclose(got["lam"], ref["lambda"], rtol=0, atol=atol)
    np.testing.assert_allclose(got["S"], ref["logp_cols"].T, rtol=0, atol=atol)
    for k in ("dX", "dW", "db"):
        if ref[k] is None or got[k] is None:
            continue
        kt = 2e-2 if (bt.dtype == "f32_bf16w" and k != "dX") else tol
        assert rel_fro(got[k], ref[k]) <= kt, (k, rel_fro(got[k], ref[k]))
