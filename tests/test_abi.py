"""CPU tests of the C-ABI library: it loads, exports every symbol that
include/*.h declares, and rejects bad arguments before touching the GPU
(validation runs first; no GPU compute call is made here)."""
import ctypes
import os
import re

import pytest

import rank_linear_layer_amd as lrl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(lr_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lrl.LIB_PATH):
        pytest.fail("liblr_linear.so is not built; run `python -m rank_linear_layer_amd.build`")
    return lrl.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("lr_linear_create", "lr_linear_run", "lr_mlp_packed_run", "lr_group_run", "lr_linear_destroy",
              "lr_status_str", "lr_last_error"):
        assert n in names
    assert set(names) == set(lrl.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.lr_status_str(0) == b"LR_OK"
    assert lib.lr_status_str(1) == b"LR_ERR_INVALID_ARG"
    assert lib.lr_status_str(4) == b"LR_ERR_HIP"
    assert lib.lr_status_str(99) == b"LR_ERR_UNKNOWN"


def test_create_rejects_bad_arguments_before_any_hip_call(lib):
    h = ctypes.c_void_p(1)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # null factor
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, None, fake, 4, 0) == lrl.LR_ERR_INVALID_ARG
    assert h.value is None
    assert b"non-null" in lib.lr_last_error()
    # bad sizes
    assert lib.lr_linear_create(ctypes.byref(h), 0, 4, 8, fake, fake, 4, 0) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, fake, fake, -1, 0) == lrl.LR_ERR_INVALID_ARG
    # misaligned factor
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, ctypes.c_void_p(0x1002), fake, 4, 0) == lrl.LR_ERR_INVALID_ARG
    # unknown flags / contradictory flags / forced decode above 16 rows
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, fake, fake, 4, 0x400) == lrl.LR_ERR_UNSUPPORTED
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, fake, fake, 4, 3) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_linear_create(ctypes.byref(h), 8, 4, 8, fake, fake, 17, 1) == lrl.LR_ERR_UNSUPPORTED
    # null out pointer
    assert lib.lr_linear_create(None, 8, 4, 8, fake, fake, 4, 0) == lrl.LR_ERR_INVALID_ARG


def test_run_and_packed_reject_null_handles(lib):
    assert lib.lr_linear_run(None, None, None, 1, None) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_mlp_packed_run(None, None, None, None, None, 1, None) == lrl.LR_ERR_INVALID_ARG
    # group: null arrays, null handle, n out of range, a repeated handle --
    # all rejected before the handles are read or any HIP call is made
    assert lib.lr_group_run(None, 1, None, None, 1, None) == lrl.LR_ERR_INVALID_ARG
    vp = ctypes.c_void_p
    ys = (vp * 4)(0x1000, 0x2000, 0x3000, 0x4000)
    assert lib.lr_group_run((vp * 1)(None), 1, vp(0x1000), ys, 1, None) == lrl.LR_ERR_INVALID_ARG
    assert b"handle 0 is null" in lib.lr_last_error()
    fake_h = (vp * 5)(0x10, 0x20, 0x30, 0x40, 0x50)
    assert lib.lr_group_run(fake_h, 0, vp(0x1000), ys, 1, None) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_group_run(fake_h, 5, vp(0x1000), ys, 1, None) == lrl.LR_ERR_INVALID_ARG
    assert b"1 to 4" in lib.lr_last_error()
    lib.lr_linear_destroy(None)  # no-op
    buf = ctypes.create_string_buffer(16)
    assert lib.lr_linear_describe(None, buf, 16) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_linear_workspace_bytes(None) == 0


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    A = torch.zeros(8, 4, dtype=torch.bfloat16)
    B = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lrl.LowRankLinear(A, B, max_M=4)
    with pytest.raises(TypeError):
        lrl.LowRankLinear(A.float(), B, max_M=4)


def test_noalloc_entry_point_validates_before_any_hip_call(lib):
    fake = ctypes.c_void_p(0x1000)
    y = ctypes.c_void_p(0x100000)
    # M above the decode range, null input, zero-sized shape, misaligned factor
    assert lib.lr_decode_noalloc(fake, fake, fake, y, 17, 8, 4, 8, None, None) == lrl.LR_ERR_INVALID_ARG
    assert b"M <= 16" in lib.lr_last_error()
    assert lib.lr_decode_noalloc(None, fake, fake, y, 1, 8, 4, 8, None, None) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_decode_noalloc(fake, fake, fake, y, 1, 0, 4, 8, None, None) == lrl.LR_ERR_INVALID_ARG
    assert lib.lr_decode_noalloc(fake, ctypes.c_void_p(0x1002), fake, y, 1, 8, 4, 8, None, None) == lrl.LR_ERR_INVALID_ARG
    # M = 0 is a no-op that touches nothing
    assert lib.lr_decode_noalloc(fake, fake, fake, y, 0, 8, 4, 8, None, None) == lrl.LR_OK
