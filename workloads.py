"""Seeded synthetic inputs for the head + CTC loss path.

This module draws random numbers and nothing else: it holds none of the loss
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it.  Shapes follow the workloads measured in "Pruned CTC for Memory-Efficient
Large-Vocabulary ASR Training" (App. C.2 head-and-loss benchmark: M = 16,000
frames at V = 180,000 with a 512-wide head input; App. B.2 batches with about
480 selected classes at V = 500; App. C.3 LLM head with V = 151,936 and
D = 4096).  The pages' GigaSpeech batches are not available; seeded stand-ins
of the same shape are used instead:

* frame counts T_n ~ U[lo, hi]; where the total M is fixed, counts are nudged
  by +-1 round-robin (staying in [lo, hi]) until they sum to M;
* target length L_n = floor(T_n / len_div);
* labels are i.i.d. from a finite-support Zipf law P(r) ~ r^-s over ranks
  r = 1..V-1, sampled by inverse CDF; rank r maps to the r-th non-blank class
  id in ascending order;
* X ~ N(0, 1); W, b ~ U(-1/sqrt(D), 1/sqrt(D)) in fp32 mode; in bf16 mode the
  LLM-head stand-in uses W ~ N(0, 0.02^2) and b = 0; bf16 values are the
  round-to-nearest-even bf16 of the fp32 draws.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass
class Batch:
    name: str
    N: int
    M: int
    D: int
    V: int
    blank: int
    chunk: int
    dtype: str                 # "f32" or "bf16"
    X: np.ndarray              # M x D float32 (exact values; bf16-representable in bf16 mode)
    W: np.ndarray              # V x D float32
    b: Optional[np.ndarray]    # V float32 or None
    frame_counts: np.ndarray   # N int32
    tgt_off: np.ndarray        # N+1 int32
    tgt: np.ndarray            # L_tot int32
    want_dW: bool = True
    want_db: bool = True

    def bf16_bits(self, a: np.ndarray) -> np.ndarray:
        """uint16 bf16 bit patterns of an array whose values are bf16-exact."""
        u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        if np.any(u & 0xFFFF):
            raise ValueError("array is not bf16-representable")
        return (u >> 16).astype(np.uint16)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16, returned as fp32 values."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def zipf_labels(rng, n, V, blank, s):
    """n i.i.d. non-blank labels with P(rank r) ~ r^-s, r = 1..V-1."""
    if n == 0:
        return np.zeros(0, dtype=np.int32)
    ranks = np.arange(1, V, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    u = rng.random(n) * cdf[-1]
    r = np.searchsorted(cdf, u, side="right") + 1
    r = np.minimum(r, V - 1)
    ids = np.where(r - 1 < blank, r - 1, r)
    return ids.astype(np.int32)


def frame_counts_uniform(rng, N, lo, hi, total=None):
    T = rng.integers(lo, hi + 1, size=N).astype(np.int64)
    if total is not None:
        if not (N * lo <= total <= N * hi):
            raise ValueError("total frame count outside [N*lo, N*hi]")
        i = 0
        while T.sum() != total:
            if T.sum() < total and T[i % N] < hi:
                T[i % N] += 1
            elif T.sum() > total and T[i % N] > lo:
                T[i % N] -= 1
            i += 1
    return T.astype(np.int32)


def _head(rng, V, D, dtype, llm_head):
    if llm_head:
        W = (rng.standard_normal((V, D), dtype=np.float32) * np.float32(0.02))
        b = np.zeros(V, dtype=np.float32)
    else:
        a = np.float32(1.0 / np.sqrt(D))
        W = rng.uniform(-a, a, size=(V, D)).astype(np.float32)
        b = rng.uniform(-a, a, size=V).astype(np.float32)
    if dtype in ("bf16", "f32_bf16w"):
        W = round_bf16(W)
        b = round_bf16(b)
    return W, b


def _assemble(name, rng, T, L, V, D, blank, chunk, dtype, zipf_s, llm_head,
              want_dW=True, want_db=True, labels=None):
    N = len(T)
    off = np.zeros(N + 1, dtype=np.int32)
    off[1:] = np.cumsum(L)
    if labels is None:
        labels = zipf_labels(rng, int(off[-1]), V, blank, zipf_s)
    M = int(np.sum(T))
    X = rng.standard_normal((M, D), dtype=np.float32)
    if dtype == "bf16":
        X = round_bf16(X)
    W, b = _head(rng, V, D, dtype, llm_head)
    return Batch(name=name, N=N, M=M, D=D, V=V, blank=blank, chunk=chunk,
                 dtype=dtype, X=X, W=W, b=b, frame_counts=np.asarray(T, np.int32),
                 tgt_off=off, tgt=np.asarray(labels, np.int32),
                 want_dW=want_dW, want_db=want_db)


# Workloads: (name, description) -> builder.  The first is the two-utterance
# example of the PrunedCTC README usage section; the next three follow the
# head-and-loss benchmark grid of App. C.2 / App. B.2; the last the frozen
# LLM head of App. C.3.
CONFIGS = {
    "tiny": "N=2, T={12,9}, D=8, V=6, blank 0, targets {1,2,3},{2,2}, C=4, fp32",
    "v500": "V=500, D=512, N=80, T~U[300,900], L=T/4, Zipf 1.1, C=4096, fp32",
    "v5k": "V=5000, D=512, N=50, M=32000, T~U[400,880], L=T/4, Zipf 1.1, C=4096, fp32",
    "v180k": "V=180000, D=512, N=25, M=16000, T~U[400,880], L=T/4, Zipf 1.1, C=4096, fp32",
    "llm152k": "V=151936, D=4096, N=40, M=32000, T~U[500,1100], L=T/3, Zipf 1.05, "
               "blank=V-1, bf16, frozen head (dX only), C=4096",
}


def make(name: str, seed: int = 0) -> Batch:
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        T = np.array([12, 9], np.int32)
        labels = np.array([1, 2, 3, 2, 2], np.int32)
        return _assemble("tiny", rng, T, np.array([3, 2]), 6, 8, 0, 4, "f32",
                         1.1, False, labels=labels)
    if name == "v500":
        T = frame_counts_uniform(rng, 80, 300, 900)
        return _assemble("v500", rng, T, T // 4, 500, 512, 0, 4096, "f32", 1.1, False)
    if name == "v5k":
        T = frame_counts_uniform(rng, 50, 400, 880, total=32000)
        return _assemble("v5k", rng, T, T // 4, 5000, 512, 0, 4096, "f32", 1.1, False)
    if name == "v180k":
        T = frame_counts_uniform(rng, 25, 400, 880, total=16000)
        return _assemble("v180k", rng, T, T // 4, 180000, 512, 0, 4096, "f32", 1.1, False)
    if name == "llm152k":
        V = 151936
        T = frame_counts_uniform(rng, 40, 500, 1100, total=32000)
        return _assemble("llm152k", rng, T, T // 3, V, 4096, V - 1, 4096, "bf16",
                         1.05, True, want_dW=False, want_db=False)
    raise KeyError(name)


def make_random(seed: int, N: int, T_lo: int, T_hi: int, V: int, D: int,
                blank: int = 0, chunk: int = 64, dtype: str = "f32",
                len_div: float = 4.0, zipf_s: float = 1.1,
                frame_counts=None, target_lengths=None, labels=None,
                llm_head: bool = False, name: str = "random") -> Batch:
    """A general seeded batch for parity and edge-case tests.

    frame_counts / target_lengths / labels override the random draws, which
    is how edge cases (unalignable utterances, T = L + r, empty targets,
    every class selected) are built.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if frame_counts is None:
        T = frame_counts_uniform(rng, N, T_lo, T_hi)
    else:
        T = np.asarray(frame_counts, np.int32)
    if target_lengths is None:
        L = (T / len_div).astype(np.int64)
    else:
        L = np.asarray(target_lengths, np.int64)
    return _assemble(name, rng, T, L, V, D, blank, chunk, dtype, zipf_s,
                     llm_head, labels=labels)


def sample_utterances(batch: Batch, idx) -> Batch:
    """The sub-batch made of utterances ``idx`` (rows and targets sliced)."""
    idx = list(idx)
    row_off = np.concatenate([[0], np.cumsum(batch.frame_counts)])
    rows = np.concatenate([np.arange(row_off[i], row_off[i + 1]) for i in idx])
    labs = [batch.tgt[batch.tgt_off[i]:batch.tgt_off[i + 1]] for i in idx]
    L = np.array([len(x) for x in labs], np.int64)
    off = np.zeros(len(idx) + 1, np.int32)
    off[1:] = np.cumsum(L)
    return dataclasses.replace(
        batch, name=batch.name + "-sample", N=len(idx), M=int(rows.shape[0]),
        X=batch.X[rows], frame_counts=batch.frame_counts[idx].copy(), tgt_off=off,
        tgt=np.concatenate(labs).astype(np.int32) if labs else np.zeros(0, np.int32))
