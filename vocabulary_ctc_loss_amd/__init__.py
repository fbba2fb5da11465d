"""pcx: vocabulary-head projection fused with the exact reduced-class CTC loss
on AMD MI355X (gfx950).

Python face of the C ABI in include/pcx.h ("Pruned CTC for Memory-Efficient
Large-Vocabulary ASR Training", unpruned reduced CTC; interface after the
PrunedCTC README's pruned_ctc_loss).  PyTorch supplies device memory and
streams; the computation runs in the library's HIP kernels.  Importing works
without a GPU; any call that reaches the library needs it built and a GPU.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from ._lib import (ALLOC_FN, FREE_FN, FwdInfo, LIB_PATH, PCX_BF16, PCX_F32,  # noqa: F401
                   PCX_F32_BF16W, PCX_FORM_DIRECT, PCX_FORM_GROUPED, PcxError, check, load)

__all__ = ["Context", "PcxError", "pruned_ctc_loss", "pack_targets", "load", "LIB_PATH"]


def _torch():
    import torch
    return torch


def _dtype_code(X, W) -> int:
    """pcx_dtype of an (X, W) pair: both fp32, both bf16, or fp32 X with a
    bf16-stored head (float16 is not supported, PrunedCTC README
    constraints)."""
    torch = _torch()
    if X.dtype == torch.float32 and W.dtype == torch.float32:
        return PCX_F32
    if X.dtype == torch.bfloat16 and W.dtype == torch.bfloat16:
        return PCX_BF16
    if X.dtype == torch.float32 and W.dtype == torch.bfloat16:
        return PCX_F32_BF16W
    raise ValueError("X / W dtypes %s / %s are not supported (fp32 / fp32, bf16 / bf16, or "
                     "fp32 / bf16 for a bf16-stored head)" % (X.dtype, W.dtype))


def _check_forward_args(X, W, b, tgt_off, tgt, frame_counts):
    """Reject, before anything reaches the library, what it would otherwise
    read out of bounds or in the wrong element type: shapes, dtypes,
    contiguity, and (last) that every tensor is on one GPU.  The targets,
    offsets and lengths themselves are checked by the library on the device.
    Returns the pcx_dtype code."""
    torch = _torch()
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D (M x D and V x D); got %s and %s"
                         % (tuple(X.shape), tuple(W.shape)))
    if W.shape[1] != X.shape[1]:
        raise ValueError("W must be V x D with D = X.shape[1] = %d; got %s"
                         % (X.shape[1], tuple(W.shape)))
    code = _dtype_code(X, W)
    if b is not None:
        if b.dim() != 1 or b.shape[0] != W.shape[0]:
            raise ValueError("b must have V = %d entries; got shape %s"
                             % (W.shape[0], tuple(b.shape)))
        if b.dtype != W.dtype:
            raise ValueError("b must have the dtype of W (%s); got %s" % (W.dtype, b.dtype))
    for name, t in (("tgt_off", tgt_off), ("tgt", tgt), ("frame_counts", frame_counts)):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError("%s must be a 1-D int32 tensor; got %s %s"
                             % (name, t.dtype, tuple(t.shape)))
    if tgt_off.shape[0] != frame_counts.shape[0] + 1:
        raise ValueError("tgt_off must have N + 1 = %d entries; got %d"
                         % (frame_counts.shape[0] + 1, tgt_off.shape[0]))
    for name, t in (("X", X), ("W", W), ("b", b), ("tgt_off", tgt_off), ("tgt", tgt),
                    ("frame_counts", frame_counts)):
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    dev = X.device
    for name, t in (("X", X), ("W", W), ("b", b), ("tgt_off", tgt_off), ("tgt", tgt),
                    ("frame_counts", frame_counts)):
        if t is not None and (t.device.type != "cuda" or t.device != dev):
            raise ValueError("%s must be on the GPU of X (%s); got %s" % (name, dev, t.device))
    return code


def _check_grad_out(name, out, like_shape, like_dtype, dev):
    """A gradient output must match its input's shape and dtype, on its GPU."""
    if out is None:
        return
    if tuple(out.shape) != tuple(like_shape) or out.dtype != like_dtype:
        raise ValueError("%s must be %s %s; got %s %s" % (name, like_dtype, tuple(like_shape),
                                                          out.dtype, tuple(out.shape)))
    if not out.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if out.device != dev:
        raise ValueError("%s must be on %s; got %s" % (name, dev, out.device))


# Workspace through torch's caching allocator (pcx_create's callbacks): the
# library's device memory then shows in torch.cuda.memory_allocated and is
# reused like any tensor's.  A block is allocated on the stream of the call
# and released on that same stream, the contract of torch's raw allocator.
def _torch_alloc(nbytes, user, stream):
    try:
        torch = _torch()
        return torch.cuda.caching_allocator_alloc(int(nbytes), torch.cuda.current_device(),
                                                  int(stream or 0))
    except Exception:
        return None  # the library reports PCX_ERR_WORKSPACE


def _torch_free(ptr, nbytes, user, stream):
    try:
        _torch().cuda.caching_allocator_delete(int(ptr))
    except Exception:
        pass


_TORCH_ALLOC = ALLOC_FN(_torch_alloc)
_TORCH_FREE = FREE_FN(_torch_free)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def pack_targets(targets: Sequence[Sequence[int]], device=None):
    """Ragged targets -> (offsets int32 [N+1], labels int32 [L_tot]) tensors."""
    torch = _torch()
    lens = [len(y) for y in targets]
    off = np.zeros(len(targets) + 1, dtype=np.int32)
    off[1:] = np.cumsum(lens)
    vals = np.concatenate([np.asarray(y, np.int32) for y in targets]) if targets \
        else np.zeros(0, np.int32)
    return (torch.from_numpy(off).to(device), torch.from_numpy(vals.astype(np.int32)).to(device))


class Context:
    """One pcx_ctx: workspace plus the forward state a backward pass needs.

    allocator="torch" (default) takes the workspace from torch's caching
    allocator on the call's stream; None lets the library use hipMalloc.
    """

    def __init__(self, allocator: Optional[str] = "torch"):
        self._lib = load()
        h = ctypes.c_void_p()
        if allocator == "torch":
            check(self._lib.pcx_create(ctypes.byref(h), ctypes.cast(_TORCH_ALLOC, ctypes.c_void_p),
                                       ctypes.cast(_TORCH_FREE, ctypes.c_void_p), None))
        elif allocator is None:
            check(self._lib.pcx_create(ctypes.byref(h), None, None, None))
        else:
            raise ValueError("allocator must be 'torch' or None")
        self._h = h
        self.info = None
        self._shape = None
        self._dev = None

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            if self._dev is not None:
                with _torch().cuda.device(self._dev):
                    self._lib.pcx_destroy(self._h)
            else:
                self._lib.pcx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------- calls
    def set_beam(self, beam: float = float("inf")):
        """Alignment beam of the following forward calls (inf: every
        alignment, the exact loss; a finite beam: the pruned objective
        L_beta, see pcx_set_beam)."""
        check(self._lib.pcx_set_beam(self._h, float(beam)))

    def discarded_mass(self):
        """delta_n = 1 - exp(-(L_beta,n - L_n)) of the last forward, per
        utterance (NaN for excluded ones)."""
        return self._get(self._lib.pcx_get_discarded_mass, self._shape["N"], np.float64)

    def set_formulation(self, grouped: bool):
        """Direct (default) or grouped ("other"-column) normalizer and
        complement gradient for the following forward calls."""
        check(self._lib.pcx_set_formulation(self._h, PCX_FORM_GROUPED if grouped
                                            else PCX_FORM_DIRECT))

    def forward(self, X, W, b, tgt_off, tgt, frame_counts, blank: int = 0,
                chunk: int = 4096, stream=None):
        """Run pcx_forward; returns (summed loss as float, info dict)."""
        code = _check_forward_args(X, W, b, tgt_off, tgt, frame_counts)
        if self._dev is not None and X.device != self._dev:
            raise ValueError("this context runs on %s; X is on %s" % (self._dev, X.device))
        M, D = X.shape
        V = W.shape[0]
        N = frame_counts.shape[0]
        L_tot = tgt.shape[0]
        loss = ctypes.c_double(0.0)
        info = FwdInfo()
        with _torch().cuda.device(X.device):
            check(self._lib.pcx_forward(
                self._h, _ptr(X), _ptr(W), _ptr(b), code, M, D, V, N, _ptr(tgt_off),
                _ptr(tgt) if L_tot else None, L_tot, _ptr(frame_counts), int(blank), int(chunk),
                _stream_handle(stream), ctypes.byref(loss), ctypes.byref(info)))
        self._dev = X.device
        self.info = {f: getattr(info, f) for f, _ in FwdInfo._fields_}
        self._shape = dict(M=M, D=D, V=V, N=N, L_tot=L_tot, K=info.K, X=(X.shape, X.dtype),
                           W=(W.shape, W.dtype))
        return loss.value, self.info

    def backward(self, grad_loss: float = 1.0, dX=None, dW=None, db=None, stream=None):
        """Run pcx_backward for the last forward: dX / dW / db (any may be None)
        are overwritten; each must match its input's shape and dtype (db: V
        entries in W's dtype)."""
        if self._shape is not None:
            sh = self._shape
            _check_grad_out("dX", dX, *sh["X"], self._dev)
            _check_grad_out("dW", dW, *sh["W"], self._dev)
            _check_grad_out("db", db, (sh["V"],), sh["W"][1], self._dev)
        dev = self._dev if self._dev is not None else _torch().cuda.current_device()
        with _torch().cuda.device(dev):
            check(self._lib.pcx_backward(self._h, float(grad_loss), _ptr(dX), _ptr(dW), _ptr(db),
                                         _stream_handle(stream)))

    def blank_offset_grad(self, grad_loss: float = 1.0, stream=None) -> float:
        """d(loss)/d(eta) for an offset eta added to the blank logit of every
        frame (db[blank] without computing db); see pcx_blank_offset_grad."""
        out = ctypes.c_double(0.0)
        dev = self._dev if self._dev is not None else _torch().cuda.current_device()
        with _torch().cuda.device(dev):
            check(self._lib.pcx_blank_offset_grad(self._h, float(grad_loss), ctypes.byref(out),
                                                  _stream_handle(stream)))
        return out.value

    # -------------------------------------------------------------- getters
    def _get(self, fn, n, dtype):
        out = np.zeros(max(1, n), dtype=dtype)
        check(fn(self._h, out.ctypes.data_as(ctypes.c_void_p), n))
        return out[:n]

    def selected(self):
        return self._get(self._lib.pcx_get_selected, self._shape["K"], np.int32)

    def relabeled(self):
        return self._get(self._lib.pcx_get_relabeled, self._shape["L_tot"], np.int32)

    def alignable(self):
        return self._get(self._lib.pcx_get_alignable, self._shape["N"], np.uint8).astype(bool)

    def utt_losses(self):
        return self._get(self._lib.pcx_get_utt_losses, self._shape["N"], np.float64)

    def utt_status(self):
        return self._get(self._lib.pcx_get_utt_status, self._shape["N"], np.int32)

    def normalizer(self):
        return self._get(self._lib.pcx_get_normalizer, self._shape["M"], np.float64)

    def other(self):
        """The other column o_m of the last (grouped) forward pass."""
        return self._get(self._lib.pcx_get_other, self._shape["M"], np.float64)

    def scores(self):
        K, M = self._shape["K"], self._shape["M"]
        return self._get(self._lib.pcx_get_scores, K * M, np.float32).reshape(K, M)

    def occupancy(self):
        K, M = self._shape["K"], self._shape["M"]
        return self._get(self._lib.pcx_get_occupancy, K * M, np.float32).reshape(K, M)

    # -------------------------------------------------------------- timing
    def profile_enable(self, on: bool = True):
        check(self._lib.pcx_profile_enable(self._h, 1 if on else 0))

    def profile_mask(self, names=None):
        """Time only the kernel families named (all of them for None)."""
        mask = 0xFFFFFFFF
        if names is not None:
            mask = 0
            all_names = list(self.profile_read())
            for n in names:
                mask |= 1 << all_names.index(n)
        check(self._lib.pcx_profile_mask(self._h, mask))

    def profile_reset(self):
        check(self._lib.pcx_profile_reset(self._h))

    def profile_read(self):
        out = {}
        for i in range(self._lib.pcx_profile_count()):
            name = ctypes.c_char_p()
            ms = ctypes.c_double()
            n = ctypes.c_int64()
            check(self._lib.pcx_profile_read(self._h, i, ctypes.byref(name), ctypes.byref(ms),
                                             ctypes.byref(n)))
            out[name.value.decode()] = (ms.value, n.value)
        return out


# Idle contexts per device, kept for the autograd function: a context goes
# back here when the autograd graph that used it is freed (nothing can call
# its backward any more), so later steps reuse a workspace that is already
# sized instead of allocating and freeing it every step.
_POOL = {}
_POOL_KEEP = 4


class _Lease:
    """A context held by one autograd graph, returned to the pool when the
    graph (and with it this object) is freed."""

    def __init__(self, device):
        self.device = device
        idle = _POOL.setdefault(device, [])
        self.ctx = idle.pop() if idle else Context()

    def __del__(self):
        try:
            idle = _POOL.setdefault(self.device, [])
            if len(idle) < _POOL_KEEP:
                idle.append(self.ctx)
            else:
                self.ctx.close()
        except Exception:
            pass


def _make_function():
    torch = _torch()

    class PcxLossFunction(torch.autograd.Function):
        @staticmethod
        def forward(fctx, X, W, b, tgt_off, tgt, frame_counts, blank, chunk, beam):
            lease = _Lease(X.device.index)
            lease.ctx.set_beam(beam)
            loss, _ = lease.ctx.forward(X, W, b, tgt_off, tgt, frame_counts, blank, chunk)
            fctx.lease = lease
            fctx.shapes = (X, W, b)
            return torch.tensor(loss, dtype=torch.float32, device=X.device)

        @staticmethod
        def backward(fctx, grad):
            X, W, b = fctx.shapes
            need = fctx.needs_input_grad
            dX = torch.empty_like(X) if need[0] else None
            dW = torch.empty_like(W) if need[1] else None
            db = torch.empty_like(b) if (b is not None and need[2]) else None
            fctx.lease.ctx.backward(float(grad.item()), dX, dW, db)
            return dX, dW, db, None, None, None, None, None, None

    return PcxLossFunction


_FN = None


def pruned_ctc_loss(X, weight, bias, targets, frame_counts, blank_id: int = 0,
                    chunk_size: int = 4096, output_beam: float = float("inf")):
    """Summed CTC loss of the affine head (X weight^T + bias) over ragged targets.

    X: (M, D) stacked head inputs (fp32 or bf16) on the GPU; weight (V, D); bias
    (V,) or None; targets: list of label lists or an (offsets, labels) pair of
    int32 device tensors; frame_counts: (N,) frame counts; output_beam: the
    alignment beam (inf: exact; finite: the pruned objective).  Returns a
    float32 scalar; gradients flow to X, weight and bias in their own dtypes.
    """
    global _FN
    torch = _torch()
    if _FN is None:
        _FN = _make_function()
    if isinstance(targets, (tuple, list)) and len(targets) == 2 and torch.is_tensor(targets[0]):
        tgt_off, tgt = targets
    else:
        tgt_off, tgt = pack_targets(targets, device=X.device)
    tgt_off = tgt_off.to(device=X.device, dtype=torch.int32).contiguous()
    tgt = tgt.to(device=X.device, dtype=torch.int32).contiguous()
    fc = frame_counts.to(device=X.device, dtype=torch.int32).contiguous()
    return _FN.apply(X.contiguous(), weight.contiguous(),
                     None if bias is None else bias.contiguous(), tgt_off, tgt, fc,
                     int(blank_id), int(chunk_size), float(output_beam))
