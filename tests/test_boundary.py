"""Host-side tests of the C ABI (no GPU needed).

* libpcx.so loads and exports every function include/pcx.h declares, and the
  Python binding's signature table covers exactly those functions;
* argument validation that happens before any device work: NULL context,
  unsupported dtype (fp16), bad sizes, bad blank / chunk, backward or getters
  before a forward pass (PCX_ERR_* codes, message via pcx_last_error);
* the Python binding's checks of shapes, dtypes, contiguity and devices,
  which reject a call before any pointer reaches the library.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pcx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pcx_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from vocabulary_ctc_loss_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from vocabulary_ctc_loss_amd import build
        build.build()
    return _lib.load()


def test_header_declares_the_expected_api():
    fns = declared_functions()
    for f in ("pcx_create", "pcx_destroy", "pcx_forward", "pcx_backward", "pcx_last_error"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    from vocabulary_ctc_loss_amd import _lib
    fns = declared_functions()
    for f in fns:
        assert hasattr(lib, f), f
    assert sorted(_lib.SIGNATURES) == fns


def _ctx(lib):
    h = ctypes.c_void_p()
    assert lib.pcx_create(ctypes.byref(h), None, None, None) == 0
    return h


def _fwd(lib, h, **kw):
    a = dict(X=1, W=1, b=None, dtype=0, M=4, D=8, V=6, N=1, off=1, tgt=1, L=2, fc=1,
             blank=0, chunk=4)
    a.update(kw)
    loss = ctypes.c_double()
    return lib.pcx_forward(h, a["X"], a["W"], a["b"], a["dtype"], a["M"], a["D"], a["V"], a["N"],
                           a["off"], a["tgt"], a["L"], a["fc"], a["blank"], a["chunk"], None,
                           ctypes.byref(loss), None)


def test_null_context_is_rejected(lib):
    assert _fwd(lib, None) == 1
    assert b"ctx" in lib.pcx_last_error()
    assert lib.pcx_backward(None, 1.0, None, None, None, None) == 1


def test_argument_validation_before_device_work(lib):
    h = _ctx(lib)
    try:
        assert _fwd(lib, h, dtype=3) == 2          # no such dtype (fp16 has no code)
        assert b"dtype" in lib.pcx_last_error()
        assert _fwd(lib, h, dtype=7) == 2
        assert _fwd(lib, h, M=-1) == 1
        assert _fwd(lib, h, D=0) == 1
        assert _fwd(lib, h, V=0) == 1
        assert _fwd(lib, h, N=-2) == 1
        assert _fwd(lib, h, blank=6) == 1          # blank outside [0, V)
        assert _fwd(lib, h, blank=-1) == 1
        assert _fwd(lib, h, chunk=0) == 1
        assert _fwd(lib, h, off=None) == 1
        assert _fwd(lib, h, tgt=None) == 1          # L_tot > 0 needs labels
        assert _fwd(lib, h, X=None) == 1
        assert _fwd(lib, h, M=2**31) == 1           # beyond the 32-bit index range
        # no forward has succeeded: backward and getters refuse
        assert lib.pcx_backward(h, 1.0, None, None, None, None) == 5
        buf = (ctypes.c_int32 * 8)()
        assert lib.pcx_get_selected(h, buf, 8) == 5
        assert lib.pcx_get_occupancy(h, buf, 8) == 5
    finally:
        lib.pcx_destroy(h)


def test_profile_api_without_device(lib):
    h = _ctx(lib)
    try:
        assert lib.pcx_profile_count() >= 10
        assert lib.pcx_profile_enable(h, 1) == 0
        assert lib.pcx_profile_reset(h) == 0
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        assert lib.pcx_profile_read(h, 1, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)) == 0
        assert name.value == b"fwd_gemm_lse" and n.value == 0
        assert lib.pcx_profile_read(h, 999, None, None, None) == 1
        assert lib.pcx_profile_mask(h, 1 << 1) == 0
        assert lib.pcx_profile_mask(None, 0) == 1
    finally:
        lib.pcx_destroy(h)


def test_formulation_switch_without_device(lib):
    h = _ctx(lib)
    try:
        assert lib.pcx_set_formulation(None, 1) == 1
        assert lib.pcx_set_formulation(h, 2) == 1      # neither direct nor grouped
        assert b"formulation" in lib.pcx_last_error()
        assert lib.pcx_set_formulation(h, -1) == 1
        assert lib.pcx_set_formulation(h, 1) == 0
        assert lib.pcx_set_formulation(h, 0) == 0
        buf = (ctypes.c_double * 8)()
        assert lib.pcx_get_other(h, buf, 8) == 5       # no forward yet
    finally:
        lib.pcx_destroy(h)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """Without the built HIP library every entry point raises: there is no
    CPU or oracle fallback anywhere in the product."""
    from vocabulary_ctc_loss_amd import _lib
    import vocabulary_ctc_loss_amd as pcx
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libpcx.so"))
    with pytest.raises(ImportError, match="not built"):
        _lib.load()
    with pytest.raises(ImportError, match="not built"):
        pcx.Context()


def test_create_rejects_half_an_allocator(lib):
    h = ctypes.c_void_p()
    from vocabulary_ctc_loss_amd import _lib
    cb = _lib.ALLOC_FN(lambda n, u, st: None)
    assert lib.pcx_create(ctypes.byref(h), ctypes.cast(cb, ctypes.c_void_p), None, None) == 1
    assert b"callbacks" in lib.pcx_last_error()
    assert lib.pcx_create(None, None, None, None) == 1


def _cpu_batch():
    import torch
    M, D, V, N = 7, 4, 6, 2
    return dict(X=torch.zeros(M, D), W=torch.zeros(V, D), b=torch.zeros(V),
                tgt_off=torch.tensor([0, 1, 2], dtype=torch.int32),
                tgt=torch.tensor([1, 2], dtype=torch.int32),
                frame_counts=torch.tensor([3, 4], dtype=torch.int32))


@pytest.mark.parametrize("change,match", [
    (dict(X="half"), "dtypes"),
    (dict(W="bf16"), "dtype of W"),               # fp32 b with a bf16 head
    (dict(W="wide"), "V x D"),
    (dict(X="1d"), "2-D"),
    (dict(b="short"), "V = 6"),
    (dict(tgt="i64"), "tgt must be a 1-D int32"),
    (dict(frame_counts="i64"), "frame_counts must be a 1-D int32"),
    (dict(tgt_off="short"), "N \\+ 1"),
    (dict(X="strided"), "X must be contiguous"),
    ({}, "must be on the GPU"),                    # every check passes but the device
])
def test_binding_rejects_bad_arguments(lib, change, match):
    import torch
    import vocabulary_ctc_loss_amd as pcx
    a = _cpu_batch()
    for k, how in change.items():
        if how == "half":
            a[k] = a[k].half()
        elif how == "bf16":
            a[k] = a[k].bfloat16()
        elif how == "wide":
            a[k] = torch.zeros(6, 5)
        elif how == "1d":
            a[k] = torch.zeros(28)
        elif how == "short":
            a[k] = a[k][:-1]
        elif how == "i64":
            a[k] = a[k].long()
        elif how == "strided":
            a[k] = torch.zeros(4, 7).t()
    ctx = pcx.Context()
    try:
        with pytest.raises(ValueError, match=match):
            ctx.forward(a["X"], a["W"], a["b"], a["tgt_off"], a["tgt"], a["frame_counts"], 0, 4)
    finally:
        ctx.close()


def test_binding_rejects_bad_gradient_outputs():
    import torch
    from vocabulary_ctc_loss_amd import _check_grad_out
    dev = torch.device("cpu")
    _check_grad_out("dX", None, (3, 4), torch.float32, dev)
    _check_grad_out("dX", torch.zeros(3, 4), (3, 4), torch.float32, dev)
    with pytest.raises(ValueError, match="dX must be"):
        _check_grad_out("dX", torch.zeros(3, 4, dtype=torch.bfloat16), (3, 4), torch.float32, dev)
    with pytest.raises(ValueError, match="db must be"):
        _check_grad_out("db", torch.zeros(5), (6,), torch.float32, dev)
    with pytest.raises(ValueError, match="contiguous"):
        _check_grad_out("dW", torch.zeros(4, 3).t(), (3, 4), torch.float32, dev)
    with pytest.raises(ValueError, match="allocator"):
        import vocabulary_ctc_loss_amd as pcx
        pcx.Context(allocator="numpy")
