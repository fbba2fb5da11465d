"""The CTC recursions alone, against the oracle's FP64 CTC on the library's
own scores.

"Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", Sec. 3.1
Eq. 2 and Sec. 3.2 Eq. 3 (the loss over the selected classes from S) and
App. B.1 / App. C.2 (FP32 scores, FP64 accumulation).  The parity tests hold
the loss to 1e-5, a bar set by the fp32 projection.  Here the projection is
taken out: the oracle's CTC runs in FP64 on exactly the fp32 scores S the
library's recursions read (S of utterance n with one extra column holding
the mass of the unselected classes, log(1 - sum_k exp S_k), so that the
oracle's log-softmax leaves S unchanged).  What remains is the recursions'
own arithmetic: FP64 sums and products of scaled probabilities, the
emission exp(S) formed to fp32 precision (about 2^-22 relative, at most
~2.4e-7 in log-probability per frame), and alpha and beta stored with fp32
mantissas for the occupancies.  So the per-utterance loss is held to 5e-7 per
frame and the occupancies to 2e-6 absolute (measured: at most 1.3e-7 per
frame and 3.4e-7).
"""
import numpy as np
import pytest

import oracle
from pcx_harness import run_pcx
from test_gpu_parity import case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiles", "spans", "long_targets", "many_utts", "blank_mid",
                                  "single_alignment", "unalignable_mix"])
def test_recursions_on_library_scores(name):
    bt = case(name)
    assert bt.dtype == "f32"
    got = run_pcx(bt)
    S, Gam, rel, st = got["S"], got["Gam"], got["rel"], got["status"]
    K = S.shape[0]
    row_off = np.concatenate([[0], np.cumsum(bt.frame_counts)])
    checked = 0
    for n in range(bt.N):
        if st[n] != 0:
            continue
        r0, r1 = int(row_off[n]), int(row_off[n + 1])
        Sn = S[:, r0:r1].astype(np.float64).T  # T x K
        mass = np.exp(Sn).sum(1)
        # the unselected classes must carry some mass for the extra column
        # (it holds in these cases, which draw V well above K)
        assert np.all(1.0 - mass > 1e-6), (name, n)
        Z = np.concatenate([Sn, np.log1p(-mass)[:, None]], 1)
        ref = oracle.ctc_logits(Z, rel[bt.tgt_off[n]:bt.tgt_off[n + 1]], 0)
        assert ref["status"] == 0
        T = r1 - r0
        assert abs(got["utt_loss"][n] - ref["loss"]) <= 5e-7 * T, (n, got["utt_loss"][n],
                                                                    ref["loss"])
        np.testing.assert_allclose(Gam[:, r0:r1].T, ref["gamma"][:, :K], rtol=0, atol=2e-6)
        checked += 1
    assert checked > 0
