"""The C-ABI library loads and exports every entry point include/snack.h declares
(CPU only: no compute call is made)."""
import ctypes
import os
import re

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "snack.h")
LIB = os.path.join(ROOT, "coo_spmm_amd", "libsnack.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(snack_[a-z_0-9]+)\s*\(", text)))


def _ensure_built():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._builder().build()


def test_header_declares_the_core_entry_points():
    names = _declared()
    for core in ("snack_layer_create", "snack_forward", "snack_backward", "snack_prune_regrow",
                 "snack_layer_destroy"):
        assert core in names


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_python_binding_covers_the_abi():
    _ensure_built()
    import coo_spmm_amd
    assert set(_declared()) == set(coo_spmm_amd.EXPORTED)
    for n in _declared():
        assert callable(getattr(coo_spmm_amd, n))


def test_status_strings_and_host_side_argument_checks():
    """Calls that fail on host-side validation never touch the device."""
    _ensure_built()
    import coo_spmm_amd as L
    assert L.snack_status_string(0) == "ok"
    assert L.snack_status_string(3) == "duplicate position"
    lib = L._lib
    h = ctypes.c_void_p()
    assert lib.snack_layer_create(0, 4, 0, None, None, None, 0, None, ctypes.byref(h)) == L.ERR_INVALID_ARG
    assert lib.snack_layer_create(4, 4, 17, None, None, None, 0, None, ctypes.byref(h)) == L.ERR_INVALID_ARG
    assert lib.snack_layer_create(4, 4, 3, None, None, None, 0, None, None) == L.ERR_INVALID_ARG
    assert lib.snack_forward(None, None, None, 1, None) == L.ERR_INVALID_ARG
    assert lib.snack_backward(None, None, None, None, None, 1, None) == L.ERR_INVALID_ARG
    assert lib.snack_prune_regrow(None, 0, None) == L.ERR_INVALID_ARG
    assert lib.snack_layer_destroy(None) == L.OK
    assert lib.snack_mse_grad(None, None, None, -1, 1.0, None) == L.ERR_INVALID_ARG
    assert L.snack_profile_name(0) == "spmm_forward"
