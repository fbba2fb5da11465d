"""ctypes binding of libpcx.so (the C ABI declared in include/pcx.h).

Argument marshalling only: every step of the loss runs in the HIP kernels of
the library.  If the library has not been built the import of this module
fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpcx.so")

PCX_F32 = 0
PCX_BF16 = 1
PCX_F32_BF16W = 2

PCX_FORM_DIRECT = 0
PCX_FORM_GROUPED = 1

STATUS_NAMES = {
    0: "PCX_OK", 1: "PCX_ERR_ARG", 2: "PCX_ERR_DTYPE", 3: "PCX_ERR_TARGET",
    4: "PCX_ERR_LENGTHS", 5: "PCX_ERR_STATE", 6: "PCX_ERR_HIP", 7: "PCX_ERR_LIMIT",
    8: "PCX_ERR_WORKSPACE",
}

# The allocation callbacks of pcx_create (pcx_alloc_fn / pcx_free_fn).
ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p)
FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                           ctypes.c_void_p)

# Every function include/pcx.h declares, with its ctypes signature.
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double
SIGNATURES = {
    "pcx_create": (_I32, [ctypes.POINTER(_P), _P, _P, _P]),
    "pcx_destroy": (None, [_P]),
    "pcx_forward": (_I32, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _I64, _P,
                           _I32, _I32, _P, ctypes.POINTER(_D), _P]),
    "pcx_backward": (_I32, [_P, _D, _P, _P, _P, _P]),
    "pcx_blank_offset_grad": (_I32, [_P, _D, ctypes.POINTER(_D), _P]),
    "pcx_set_formulation": (_I32, [_P, _I32]),
    "pcx_set_beam": (_I32, [_P, _D]),
    "pcx_loss_grad_static": (_I32, [_P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _I64, _P,
                                    _I32, _I32, _D, _P, _P, _P, _P, ctypes.POINTER(_D), _P]),
    "pcx_get_discarded_mass": (_I32, [_P, _P, _I64]),
    "pcx_last_error": (ctypes.c_char_p, []),
    "pcx_get_selected": (_I32, [_P, _P, _I64]),
    "pcx_get_relabeled": (_I32, [_P, _P, _I64]),
    "pcx_get_alignable": (_I32, [_P, _P, _I64]),
    "pcx_get_utt_losses": (_I32, [_P, _P, _I64]),
    "pcx_get_utt_status": (_I32, [_P, _P, _I64]),
    "pcx_get_normalizer": (_I32, [_P, _P, _I64]),
    "pcx_get_scores": (_I32, [_P, _P, _I64]),
    "pcx_get_occupancy": (_I32, [_P, _P, _I64]),
    "pcx_get_other": (_I32, [_P, _P, _I64]),
    "pcx_profile_enable": (_I32, [_P, _I32]),
    "pcx_profile_mask": (_I32, [_P, ctypes.c_uint32]),
    "pcx_profile_reset": (_I32, [_P]),
    "pcx_profile_count": (_I32, []),
    "pcx_profile_read": (_I32, [_P, _I32, ctypes.POINTER(ctypes.c_char_p),
                                ctypes.POINTER(_D), ctypes.POINTER(_I64)]),
}


class FwdInfo(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("n_unalignable", ctypes.c_int32),
                ("n_nonfinite", ctypes.c_int32), ("max_target_len", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("lse_spans", ctypes.c_int32)]


class PcxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libpcx.so; raises if it was not built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libpcx.so is not built (expected at %s); run "
                "`python -m vocabulary_ctc_loss_amd.build` or __graft_entry__.build()" % LIB_PATH)
        # torch first: it carries its own HIP runtime (same soname as the
        # system one), and the library must bind to the runtime that owns
        # the tensors' device memory and streams.  Loaded before torch it
        # bound to the system runtime, and its first allocation on the
        # device then failed ("no ROCm-capable device").
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = load().pcx_last_error()
        raise PcxError(status, msg.decode() if msg else "")
