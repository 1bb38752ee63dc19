"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call.

No compute call is made here: every call has an invalid argument, so it
returns before reaching the device (fake pointers are never dereferenced).
"""
import ctypes
import os
import re

import pytest

import sample_gradient_clipping_layer_amd as dpc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dpclip.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced
FAKE_MIS = FAKE + 4


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(dp_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dpc.LIB_PATH):
        pytest.fail("libdpclip.so is not built (run __graft_entry__.build())")
    return dpc.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(dpc.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dp_abi_version() == 1


def test_status_strings(lib):
    for s in range(0, 9):
        assert lib.dp_status_string(s).decode()
    assert lib.dp_status_string(99).decode() == "unknown status"


def _ghost(lib, A=FAKE, G=FAKE, dt=0, B=4, T=3, d=5, p=6, hb=0, mode=0, kappa=1, ws=FAKE, wsb=1 << 20,
           sq=FAKE, acc=0):
    path = ctypes.c_int32(-7)
    st = lib.dp_ghost_norm(None, A, G, dt, B, T, d, p, hb, mode, kappa, ws, wsb, sq, acc, ctypes.byref(path))
    return st, path.value


def test_ghost_norm_validation(lib):
    assert _ghost(lib, A=None)[0] == dpc.DP_ERR_NULL
    assert _ghost(lib, sq=None)[0] == dpc.DP_ERR_NULL
    assert _ghost(lib, B=0)[0] == dpc.DP_ERR_SHAPE
    assert _ghost(lib, T=-1)[0] == dpc.DP_ERR_SHAPE
    assert _ghost(lib, p=0)[0] == dpc.DP_ERR_SHAPE
    assert _ghost(lib, B=1 << 31)[0] == dpc.DP_ERR_SHAPE
    assert _ghost(lib, B=1 << 30, T=1 << 12, d=1 << 12)[0] == dpc.DP_ERR_SHAPE   # element count overflow
    assert _ghost(lib, dt=2)[0] == dpc.DP_ERR_DTYPE
    assert _ghost(lib, A=FAKE_MIS)[0] == dpc.DP_ERR_ALIGN
    assert _ghost(lib, mode=3)[0] == dpc.DP_ERR_VALUE
    assert _ghost(lib, kappa=0)[0] == dpc.DP_ERR_VALUE
    # T = 100 spans 3 Gram tiles per sample: partials + arrival counters in the workspace
    assert _ghost(lib, ws=None, T=100, mode=dpc.MODE_GHOST)[0] == dpc.DP_ERR_NULL
    assert _ghost(lib, wsb=4, T=100, mode=dpc.MODE_GHOST)[0] == dpc.DP_ERR_WORKSPACE
    st, path = _ghost(lib, wsb=4, T=100, mode=dpc.MODE_GHOST)
    assert path == -7                                    # nothing written on failure
    # a sample that is a single tile needs no workspace
    assert lib.dp_workspace_bytes(0, 4, 3, 5, 6, 0, 1) == 0
    # more than 65535 explicit tiles per sample is refused
    assert _ghost(lib, T=1 << 16, d=1 << 15, p=1 << 15, B=1, mode=dpc.MODE_EXPLICIT, wsb=1 << 40)[0] == dpc.DP_ERR_SHAPE


def test_clip_and_threshold_validation(lib):
    f = ctypes.c_float
    assert lib.dp_clip_factors(None, None, 4, f(1.0), FAKE, None) == dpc.DP_ERR_NULL
    assert lib.dp_clip_factors(None, FAKE, 0, f(1.0), FAKE, None) == dpc.DP_ERR_SHAPE
    for C in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.dp_clip_factors(None, FAKE, 4, f(C), FAKE, None) == dpc.DP_ERR_VALUE
    assert lib.dp_clip_factors(None, FAKE + 2, 4, f(1.0), FAKE, None) == dpc.DP_ERR_ALIGN
    thr = lib.dp_adaptive_threshold
    assert thr(None, None, 4, 1.0, 1.1, 2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_NULL
    assert thr(None, FAKE, 0, 1.0, 1.1, 2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_SHAPE
    assert thr(None, FAKE, 4, 1.0, 0.0, 2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_VALUE
    assert thr(None, FAKE, 4, 1.0, 1.1, -2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_VALUE
    assert thr(None, FAKE, 4, 1.0, 1.1, 2.0, -1.0, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_VALUE
    assert thr(None, FAKE, 4, 0.0, 1.1, 2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_VALUE  # C_prev
    assert thr(None, FAKE, 4, float("nan"), 1.1, 2.0, 2.5, 0, 0, 0, 0, FAKE, None) == dpc.DP_ERR_VALUE


def test_clipped_sum_validation(lib):
    def call(A=FAKE, dt=0, B=4, T=3, d=5, p=6, c=FAKE, C=1.0, sigma=1.0, denom=4.0, ws=FAKE, wsb=1 << 30,
             out=FAKE, bout=None):
        return lib.dp_clipped_sum_noise(None, A, FAKE, dt, B, T, d, p, c, C, sigma, denom, 0, 0, 0, ws, wsb, out,
                                        bout)
    assert call(A=None) == dpc.DP_ERR_NULL
    assert call(c=None) == dpc.DP_ERR_NULL
    assert call(out=None) == dpc.DP_ERR_NULL
    assert call(d=0) == dpc.DP_ERR_SHAPE
    assert call(d=1 << 20, p=1 << 15) == dpc.DP_ERR_SHAPE      # d*p beyond the noise counter range
    assert call(dt=-1) == dpc.DP_ERR_DTYPE
    assert call(C=0.0) == dpc.DP_ERR_VALUE
    assert call(sigma=-0.1) == dpc.DP_ERR_VALUE
    assert call(denom=0.0) == dpc.DP_ERR_VALUE
    assert call(denom=float("inf")) == dpc.DP_ERR_VALUE
    # a long K with a single small output tile is split over K: it needs a workspace
    big = dict(B=4096, T=64, d=8, p=8)
    assert lib.dp_workspace_bytes(0, 4096, 64, 8, 8, 0, 1) > 0
    assert call(ws=None, **big) == dpc.DP_ERR_NULL
    assert call(wsb=8, **big) == dpc.DP_ERR_WORKSPACE
    assert call(ws=FAKE + 8, **big) == dpc.DP_ERR_ALIGN
    assert call(out=FAKE + 1) == dpc.DP_ERR_ALIGN


def test_workspace_and_path_helpers(lib):
    assert lib.dp_workspace_bytes(0, 0, 1, 1, 1, 0, 1) == 0
    assert lib.dp_workspace_bytes(5, 4, 1, 1, 1, 0, 1) == 0
    w = lib.dp_workspace_bytes(1, 64, 128, 768, 2304, 0, 1)
    assert w > 0 and w % 256 == 0
    assert lib.dp_choose_path(1, 64, 32, 0, 1) == dpc.PATH_T1
    assert lib.dp_choose_path(1024, 27, 64, 0, 1) == dpc.PATH_EXPLICIT
    assert lib.dp_choose_path(256, 576, 128, 0, 1) == dpc.PATH_GHOST
    assert lib.dp_choose_path(256, 576, 128, 0, 2) == dpc.PATH_EXPLICIT
    assert lib.dp_choose_path(4, 2, 8, 0, 1) == dpc.PATH_GHOST
    assert lib.dp_choose_path(1, 2, 8, 2, 1) == dpc.PATH_EXPLICIT
    assert lib.dp_choose_path(0, 2, 8, 0, 1) == -1


def test_path_rule_agrees_with_oracle(lib):
    """The library's integer path decision equals the oracle's on every layer
    shape of the five workloads, both kappas and all modes (bit-exact)."""
    from oracle import definitions as D
    import workloads as W
    for name in W.WORKLOAD_ORDER:
        wl = W.WORKLOADS[name]
        for (T, d, p) in wl.layers:
            for mode in (0, 1, 2):
                for kappa in (1, 2):
                    assert lib.dp_choose_path(T, d, p, mode, kappa) == D.choose_path(T, d, p, mode, kappa)


def test_valid_call_without_device_reports_no_device(lib):
    """A fully valid call reaches the device check; with no GPU present it
    returns DP_ERR_NO_DEVICE and launches nothing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, _ = _ghost(lib)
    assert st == dpc.DP_ERR_NO_DEVICE


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    A = torch.zeros(2, 1, 3)
    with pytest.raises(ValueError):
        dpc.dp_ghost_norm(A, A, torch.zeros(2))
