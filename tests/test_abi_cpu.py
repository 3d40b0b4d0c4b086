"""The C-ABI library loads and exports every function include/ep_layout.h
declares; host-side argument checks reject bad configurations before any HIP
call (CPU only: nothing here launches GPU work)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_layout.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+(ep_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("ep_handle_create", "ep_handle_destroy", "ep_layout", "ep_dispatch",
                     "ep_combine", "ep_handle_get_view", "ep_counts_to_host",
                     "ep_handle_sync_status", "ep_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import combine_ep_layout_amd as ep
    lib = ep.library()
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ep.EXPORTS) == names


def test_probe_library_rejects_bad_arguments_without_gpu():
    """libep_ceiling.so (the benchmark's bandwidth probes) loads and rejects
    invalid arguments before it launches anything."""
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_ep_layout_amd", "libep_ceiling.so"))
    f = lib.ep_ceiling_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    rows = ctypes.c_void_p(16)
    buf = ctypes.c_void_p(1 << 20)
    assert f(7, 1, buf, buf, 4, 64, rows, 1, buf, None) == -1        # unknown probe
    assert f(5, 1, buf, None, 4, 64, rows, 5, None, None) == -1      # flat beyond dst
    assert f(0, 3, buf, None, 4, 64, rows, 1, None, None) == -1      # 3 waves per row
    assert f(0, 1, buf, None, 4, 24, rows, 1, None, None) == -1      # row not a multiple of 16
    assert f(0, 1, ctypes.c_void_p((1 << 20) + 8), None, 4, 64, rows, 1, None, None) == -1
    assert f(2, 1, None, buf, 4, 64, rows, 1, None, None) == -1      # read without a sink
    assert f(3, 1, buf, None, 4, 64, rows, 1, None, None) == -1      # copy without a source
    assert f(0, 1, buf, None, 4, 64, None, 1, None, None) == -1      # no row list
    assert f(0, 5, buf, None, 4, 64, rows, 1, None, None) == -1     # 5 waves per row
    assert f(0, 4, buf, None, 4, 64, rows, 0, None, None) == 0       # nothing to do
    assert f(0, 0, buf, None, 4, 64, rows, 0, None, None) == 0       # (one wave per piece)


def test_status_strings():
    import combine_ep_layout_amd as ep
    lib = ep.library()
    for s in range(8):
        assert lib.ep_status_string(s)
    assert lib.ep_status_string(0) == b"ok"


@pytest.mark.parametrize("cfg", [
    (-1, 2, 8, 16),        # negative max_tokens
    (16, 0, 8, 16),        # top_k 0
    (16, 33, 8, 16),       # top_k above 32
    (16, 2, 0, 16),        # no experts
    (16, 2, 1025, 16),     # too many experts
    (16, 2, 8, 0),         # block_m 0
    (16, 2, 8, 4097),      # block_m above 4096
    (1 << 30, 8, 8, 16),   # capacity beyond int32 rows
    ((1 << 19) + 1, 1, 1, 1),  # more tokens than one launch's grid allows
])
def test_create_rejects_bad_config_without_gpu(cfg):
    import combine_ep_layout_amd as ep
    with pytest.raises(ep.EpError) as ei:
        ep.ep_handle_create(*cfg)
    assert ei.value.status == ep.EP_ERR_INVALID_ARGUMENT


def test_null_handle_calls_are_rejected():
    import combine_ep_layout_amd as ep
    lib = ep.library()
    assert lib.ep_layout(None, None, None, 0, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_dispatch(None, None, 128, None, None, 0, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_combine(None, 1, None, 128, None, None) == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_layout_dispatch(None, None, None, 0, None, 128, None, None, 0, None, None, None) \
        == ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_handle_destroy(None) == ep.EP_OK
    assert lib.ep_pool_capacity_rows(None) == -1 and lib.ep_max_tiles(None) == -1
    assert lib.ep_handle_create(None, None) == ep.EP_ERR_INVALID_ARGUMENT


def test_new_entry_points_reject_before_any_hip_call():
    import combine_ep_layout_amd as ep
    lib = ep.library()
    INV = ep.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_combine_gated(None, 1, None, 128, None, 1, 1000, None) == INV
    assert lib.ep_combine_backward(None, 1, None, None, 128, None, None, None) == INV
    assert lib.ep_dispatch_backward(None, 1, None, 128, None, None) == INV
    assert lib.ep_tile_consume(None, 1, None, None, 128, 0, None, 1, 1000, None) == INV
    assert lib.ep_borrow_release(None, None) == INV
    assert lib.ep_set_density_hint(None, 0) == INV
    assert lib.ep_layout_density(None, None) == ep.EP_DENSITY_AUTO
    assert lib.ep_set_density_hint(None, 0) == INV
    assert lib.ep_layout_density(None, None) == ep.EP_DENSITY_AUTO
    assert lib.ep_scale_ld(None) == -1
    # the cast back needs no handle: every check happens on the host first
    assert lib.ep_fp8_cast_back(None, None, 0, 0, 0, 256, None, None) == ep.EP_OK      # no rows
    assert lib.ep_fp8_cast_back(None, None, ep.EP_DISPATCH_TILE_READY, 0, 0, 256, None, None) == INV
    assert lib.ep_fp8_cast_back(None, None, 0, 4, 0, 192, None, None) == INV            # hidden % 128
    assert lib.ep_fp8_cast_back(None, None, 0, -1, 0, 256, None, None) == INV
    assert lib.ep_fp8_cast_back(None, None, ep.EP_SCALE_MN_MAJOR, 8, 7, 256, None, None) == INV
    assert lib.ep_fp8_cast_back(None, None, 0, 4, 0, 256, None, None) == INV             # null buffers
    assert lib.ep_fp8_cast_back(0x1000, 0x2002, ep.EP_SCALE_F32, 4, 0, 256, 0x3000,
                                None) == INV                                              # float scales misaligned
    assert lib.ep_fp8_cast_back(0x1008, 0x2000, 0, 4, 0, 256, 0x3000, None) == INV       # codes not 16-byte aligned
    assert lib.ep_fp8_cast_back(None, None, 0, 0, 0, 1 << 17, None, None) == ep.EP_ERR_UNSUPPORTED
    # the allocation-free layout checks sizes, capacity and output pointers first
    nul = [None] * 7
    assert lib.ep_layout_noalloc(None, -1, 2, 4, 8, 100, *nul, None, None) == INV
    assert lib.ep_layout_noalloc(None, (1 << 19) + 1, 1, 4, 8, 1 << 22, *nul, None, None) == INV
    assert lib.ep_layout_noalloc(None, 10, 33, 4, 8, 1000, *nul, None, None) == INV
    assert lib.ep_layout_noalloc(None, 10, 2, 1025, 8, 10000, *nul, None, None) == INV
    assert lib.ep_layout_noalloc(None, 10, 2, 4, 8, 47, *nul, None, None) == INV     # < 20 + 28
    assert lib.ep_layout_noalloc(None, 10, 2, 4, 8, 48, *nul, None, None) == INV     # no outputs
    big = (1 << 19) * 32 + 1024 * 127                                                # workspace too big
    assert lib.ep_layout_noalloc(None, 1 << 19, 32, 1024, 128, big, *nul, None, None) == ep.EP_ERR_UNSUPPORTED


@pytest.mark.parametrize("kind,mn,shape,dtype", [
    ("ue8m0", False, (100, 5), "uint8"),
    ("f32", False, (100, 5), "float32"),
    ("pow2_f32", False, (100, 5), "float32"),
    ("ue8m0", True, (2, 104), "int32"),          # 5 groups packed into 2 words per row
    ("f32", True, (5, 104), "float32"),
    ("pow2_f32", True, (5, 104), "float32"),
])
def test_scale_shapes_and_flags(kind, mn, shape, dtype):
    import torch
    import combine_ep_layout_amd as ep
    got, dt = ep.scale_shape(100, 640, kind, mn, 104)
    assert got == shape and dt == getattr(torch, dtype)
    f = ep.scale_flags(kind, mn)
    assert bool(f & ep.EP_SCALE_MN_MAJOR) == mn
    assert bool(f & ep.EP_SCALE_F32) == (kind != "ue8m0")
    assert bool(f & ep.EP_SCALE_ROUND) == (kind == "pow2_f32")
