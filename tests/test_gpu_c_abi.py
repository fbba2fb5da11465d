"""The C ABI on its own: a plain-C program (tests/c_abi/pcx_c_run.c, built by
__graft_entry__.build) takes device memory from the HIP runtime API, calls
pcx_create / pcx_forward / pcx_backward / pcx_destroy with plain pointers and
sizes as include/pcx.h declares them, and writes the loss and gradients to a
file; no Python or PyTorch is in that process.  Its outputs are held to the
fp32 bar against the oracle, once with the library's own hipMalloc workspace
(NULL callbacks) and once with the workspace taken from allocation callbacks
of the program (which fails unless pcx_destroy released all of it)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from pcx_harness import rel_fro

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "pcx_c_run")


def _batch(name):
    if name == "readme":
        return workloads.make("tiny", seed=0)
    # several frame tiles, ragged D and chunks
    return workloads.make_random(1, N=6, T_lo=40, T_hi=130, V=700, D=72, chunk=200)


@pytest.mark.parametrize("name,callbacks", [("readme", False), ("tiles", False),
                                            ("tiles", True)])
def test_c_program_matches_oracle(name, callbacks, tmp_path):
    assert os.path.exists(EXE), "C ABI test program not built (run __graft_entry__.build())"
    bt = _batch(name)
    assert bt.dtype == "f32"
    b = bt.b if bt.b is not None else np.zeros(bt.V)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([bt.N, bt.M, bt.D, bt.V, len(bt.tgt), bt.blank, bt.chunk],
                         np.int32).tobytes())
        for a in (bt.X, bt.W, b):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
        for a in (bt.tgt_off, bt.tgt, bt.frame_counts):
            f.write(np.ascontiguousarray(a, np.int32).tobytes())
    print("case", name, "M", bt.M, "V", bt.V, "D", bt.D, "callbacks", callbacks, flush=True)
    r = subprocess.run([EXE, str(src), str(dst)] + (["callbacks"] if callbacks else []),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = dst.read_bytes()
    loss = np.frombuffer(raw[:8], np.float64)[0]
    K, n_unal, n_nonf = np.frombuffer(raw[8:20], np.int32)
    vals = np.frombuffer(raw[20:], np.float32)
    nX, nW = bt.M * bt.D, bt.V * bt.D
    dX = vals[:nX].reshape(bt.M, bt.D)
    dW = vals[nX:nX + nW].reshape(bt.V, bt.D)
    db = vals[nX + nW:]
    ref = oracle.pcx(bt.X, bt.W, b, bt.frame_counts, bt.tgt_off, bt.tgt, bt.blank)
    U, _, flags = oracle.select(bt.V, bt.blank, bt.frame_counts, bt.tgt_off, bt.tgt)
    assert K == len(U)
    assert n_unal == int(np.sum(flags == 0)) and n_nonf == 0
    assert abs(loss - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    for k, got in (("dX", dX), ("dW", dW), ("db", db)):
        assert rel_fro(got, ref[k]) <= 1e-5, k
