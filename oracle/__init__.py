"""CPU FP64 oracle for the vocabulary-head + CTC loss path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  It shares
no code with the HIP implementation under ``vocabulary_ctc_loss_amd/``.

The arithmetic lives in ``ctc_oracle.c`` (plain C, IEEE FP64, natural-order
loops); this module only builds it with gcc and marshals numpy arrays.  What
it computes is the full-vocabulary definition of CTC through an affine head
("Pruned CTC for Memory-Efficient Large-Vocabulary ASR Training", Sec. 3.1
Eq. 1-2 and Sec. 3.2 Eq. 5): every logit is formed, log-softmax is taken over
the whole vocabulary, the standard forward/backward recursions give the loss
and the occupancies, and the analytic gradient p - gamma is pushed through the
head.  Pins: tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ctc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STATUS_OK = 0
STATUS_UNALIGNABLE = 1
STATUS_NONFINITE = 2


def build(force: bool = False) -> str:
    """Compile ctc_oracle.c into liboracle.so with gcc (IEEE FP64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_select.argtypes = [I, I, I, P, P, P, P, P, P]
    lib.oracle_select.restype = I
    lib.oracle_ctc_logits.argtypes = [I, I, I, P, P, I, ctypes.c_double, P, P, P, P, P]
    lib.oracle_ctc_logits.restype = I
    lib.oracle_pcx.argtypes = [I, I, I, I, I, P, P, P, P, P, P, ctypes.c_double, P, P, P, P,
                               I, P, P, P, P, P, P]
    lib.oracle_pcx.restype = I
    lib.oracle_ctc_beam.argtypes = [I, I, I, P, P, I, ctypes.c_double, ctypes.c_double, P, P,
                                    P, P, P, P, P]
    lib.oracle_ctc_beam.restype = I
    lib.oracle_pcx_beam.argtypes = [I, I, I, I, I, P, P, P, P, P, P, ctypes.c_double,
                                    ctypes.c_double, P, P, P, P, P, P, I, P, P, P, P, P, P]
    lib.oracle_pcx_beam.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class Oracle:
    """The oracle's functions bound to one compiled copy of ctc_oracle.c."""

    def __init__(self, path):
        self.lib = _bind(path)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def select(self, V, blank, frame_counts, tgt_off, tgt):
        """Selected classes U (blank first, then ascending distinct labels),
        relabelled targets and structural-alignability flags."""
        fc, off, y = _i32(frame_counts), _i32(tgt_off), _i32(tgt)
        N = fc.shape[0]
        U = np.zeros(max(1, min(V, y.shape[0] + 1)), dtype=np.int32)
        rel = np.zeros(max(1, y.shape[0]), dtype=np.int32)
        flags = np.zeros(max(1, N), dtype=np.uint8)
        K = self.lib.oracle_select(N, V, blank, _ptr(fc), _ptr(off), _ptr(y), _ptr(U),
                                   _ptr(rel), _ptr(flags))
        if K < 0:
            raise ValueError("oracle_select rejected the batch (code %d)" % -K)
        return U[:K].copy(), rel[: y.shape[0]].copy(), flags[:N].astype(bool)

    def ctc_logits(self, Z, y, blank, grad=1.0, want_grad=True):
        """CTC of one utterance from its raw logits Z (T x V)."""
        Z = _f64(Z)
        T, V = Z.shape
        y = _i32(y)
        loss = ctypes.c_double(0.0)
        st = ctypes.c_int(0)
        lam = np.zeros(T)
        dZ = np.zeros((T, V)) if want_grad else None
        gam = np.zeros((T, V)) if want_grad else None
        rc = self.lib.oracle_ctc_logits(T, V, blank, _ptr(Z), _ptr(y) if y.size else None,
                                        int(y.shape[0]), float(grad), ctypes.byref(loss),
                                        ctypes.byref(st), _ptr(lam), _ptr(dZ), _ptr(gam))
        if rc != 0:
            raise ValueError("oracle_ctc_logits failed (code %d)" % rc)
        return {"loss": loss.value, "status": st.value, "lambda": lam, "dZ": dZ, "gamma": gam}

    def ctc_beam(self, Z, y, blank, beam, grad=1.0, want_grad=True):
        """Finite-beam CTC of one utterance from its raw logits Z (T x V): loss
        over the retained alignments, the unpruned loss, the pruning margin,
        occupancies and logit gradient (see oracle_ctc_beam)."""
        Z = _f64(Z)
        T, V = Z.shape
        y = _i32(y)
        loss = ctypes.c_double(0.0)
        full = ctypes.c_double(0.0)
        margin = ctypes.c_double(0.0)
        st = ctypes.c_int(0)
        lam = np.zeros(T)
        dZ = np.zeros((T, V)) if want_grad else None
        gam = np.zeros((T, V)) if want_grad else None
        rc = self.lib.oracle_ctc_beam(T, V, blank, _ptr(Z), _ptr(y) if y.size else None,
                                      int(y.shape[0]), float(beam), float(grad),
                                      ctypes.byref(loss), ctypes.byref(st), ctypes.byref(full),
                                      _ptr(lam), _ptr(dZ), _ptr(gam), ctypes.byref(margin))
        if rc != 0:
            raise ValueError("oracle_ctc_beam failed (code %d)" % rc)
        return {"loss": loss.value, "status": st.value, "full_loss": full.value,
                "margin": margin.value, "lambda": lam, "dZ": dZ, "gamma": gam}

    def pcx(self, X, W, b, frame_counts, tgt_off, tgt, blank, grad=1.0, cols=None,
            want_dX=True, want_dW=True, want_db=True, want_gamma=False, want_lambda=True,
            beam=None):
        """Full path: head projection, summed CTC loss and gradients in FP64.

        X (M x D), W (V x D), b (V or None) are upcast exactly to FP64.  Returns
        a dict with loss, utt_loss, status, lambda, logp_cols/gamma_cols (at the
        columns ``cols``), dX, dW and db.  With ``beam`` (a number, inf
        included) the finite-beam objective is used and the dict also holds
        delta (discarded posterior mass per utterance) and margin.
        """
        X, W = _f64(X), _f64(W)
        bb = None if b is None else _f64(b)
        M, D = X.shape
        V = W.shape[0]
        fc, off, y = _i32(frame_counts), _i32(tgt_off), _i32(tgt)
        N = fc.shape[0]
        cols = _i32(cols if cols is not None else [])
        nc = int(cols.shape[0])
        loss = ctypes.c_double(0.0)
        utt = np.zeros(max(1, N))
        st = np.zeros(max(1, N), dtype=np.int32)
        lam = np.zeros(max(1, M)) if want_lambda else None
        lpc = np.zeros((max(1, M), max(1, nc))) if nc else None
        gmc = np.zeros((max(1, M), max(1, nc))) if (nc and want_gamma) else None
        dX = np.zeros((M, D)) if want_dX else None
        dW = np.zeros((V, D)) if want_dW else None
        db = np.zeros(V) if want_db else None
        yy = _ptr(y) if y.size else _ptr(np.zeros(1, np.int32))
        if beam is None:
            rc = self.lib.oracle_pcx(N, M, D, V, blank, _ptr(X), _ptr(W), _ptr(bb), _ptr(fc),
                                     _ptr(off), yy, float(grad), ctypes.byref(loss), _ptr(utt),
                                     _ptr(st), _ptr(lam), nc, _ptr(cols) if nc else None,
                                     _ptr(lpc), _ptr(gmc), _ptr(dX), _ptr(dW), _ptr(db))
        else:
            delta = np.zeros(max(1, N))
            margin = np.zeros(max(1, N))
            rc = self.lib.oracle_pcx_beam(N, M, D, V, blank, _ptr(X), _ptr(W), _ptr(bb), _ptr(fc),
                                          _ptr(off), yy, float(beam), float(grad),
                                          ctypes.byref(loss), _ptr(utt), _ptr(st), _ptr(delta),
                                          _ptr(margin), _ptr(lam), nc,
                                          _ptr(cols) if nc else None, _ptr(lpc), _ptr(gmc),
                                          _ptr(dX), _ptr(dW), _ptr(db))
        if rc != 0:
            raise ValueError("oracle_pcx failed (code %d)" % rc)
        out = {"loss": loss.value, "utt_loss": utt[:N].copy(), "status": st[:N].copy(),
               "dX": dX, "dW": dW, "db": db}
        if beam is not None:
            out["delta"] = delta[:N].copy()
            out["margin"] = margin[:N].copy()
        out["lambda"] = lam[:M].copy() if want_lambda else None
        out["logp_cols"] = lpc[:M, :nc].copy() if nc else None
        out["gamma_cols"] = gmc[:M, :nc].copy() if gmc is not None else None
        return out


_default = None


def _oracle() -> Oracle:
    global _default
    if _default is None:
        # PCX_ORACLE_LIB: a separately compiled copy of ctc_oracle.c (the
        # sanitizer build of the tests) in place of liboracle.so
        alt = os.environ.get("PCX_ORACLE_LIB")
        _default = Oracle(alt if alt else build())
    return _default


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build_sanitized(out_path: str, src_text: str = None) -> str:
    """Compile ctc_oracle.c (or a test-modified copy of its text) with
    AddressSanitizer and UndefinedBehaviorSanitizer (gcc; any finding aborts)
    for the tests that run the pins under them."""
    src = _SRC
    if src_text is not None:
        src = out_path + ".c"
        with open(src, "w") as f:
            f.write(src_text)
    subprocess.run(["gcc", "-O1", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-Wall", "-Wextra"] + SANITIZE_FLAGS +
                   ["-o", out_path, src, "-lm"], check=True)
    return out_path


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile a (test-modified) copy of the oracle source; used by the tests
    that check the pins reject planted mistakes."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", out_path, src, "-lm"], check=True)
    return out_path


def source_text() -> str:
    return open(_SRC).read()


def num_threads() -> int:
    return _oracle().num_threads()


def select(V, blank, frame_counts, tgt_off, tgt):
    return _oracle().select(V, blank, frame_counts, tgt_off, tgt)


def ctc_logits(Z, y, blank, grad=1.0, want_grad=True):
    return _oracle().ctc_logits(Z, y, blank, grad=grad, want_grad=want_grad)


def ctc_beam(Z, y, blank, beam, grad=1.0, want_grad=True):
    return _oracle().ctc_beam(Z, y, blank, beam, grad=grad, want_grad=want_grad)


def pcx(X, W, b, frame_counts, tgt_off, tgt, blank, grad=1.0, cols=None, want_dX=True,
        want_dW=True, want_db=True, want_gamma=False, want_lambda=True, beam=None):
    return _oracle().pcx(X, W, b, frame_counts, tgt_off, tgt, blank, grad=grad, cols=cols,
                         want_dX=want_dX, want_dW=want_dW, want_db=want_db,
                         want_gamma=want_gamma, want_lambda=want_lambda, beam=beam)
