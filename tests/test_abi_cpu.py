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
    assert lib.dp_abi_version() == 3


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
    assert _ghost(lib, mode=4)[0] == dpc.DP_ERR_VALUE
    assert _ghost(lib, kappa=0)[0] == dpc.DP_ERR_VALUE
    # T = 100 spans 3 Gram tiles per sample: tile partials in the workspace
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
    assert lib.dp_choose_path(4, 2, 8, 4, 1) == -1
    # the time rule: explicit on the conv layers whose per-sample product is the smaller work
    conv = [(1024, 27, 64), (1024, 576, 64), (256, 576, 128), (256, 1152, 128), (64, 1152, 256),
            (64, 2304, 256), (16, 2304, 512), (16, 4608, 512)]
    assert [lib.dp_choose_path(T, d, p, dpc.MODE_TIME, 1) for (T, d, p) in conv] == \
        [dpc.PATH_EXPLICIT] * 4 + [dpc.PATH_GHOST] * 4
    for (T, d, p) in [(128, 768, 2304), (128, 768, 768), (1024, 1280, 1280), (1024, 5120, 1280)]:
        assert lib.dp_choose_path(T, d, p, dpc.MODE_TIME, 1) == dpc.PATH_GHOST
    assert lib.dp_choose_path(1, 64, 32, dpc.MODE_TIME, 1) == dpc.PATH_T1


def test_path_rule_agrees_with_oracle(lib):
    """The library's integer path decision equals the oracle's on every layer
    shape of the five workloads, both kappas and all modes (bit-exact)."""
    from oracle import definitions as D
    import workloads as W
    for name in W.WORKLOAD_ORDER:
        wl = W.WORKLOADS[name]
        for (T, d, p) in wl.layers:
            for mode in (0, 1, 2, 3):
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


def _layers(specs, A=FAKE, G=FAKE, reserved=0):
    arr = (dpc.DpLayer * max(1, len(specs)))()
    for k, (T, d, p, hb) in enumerate(specs):
        arr[k] = dpc.DpLayer(A, G, T, d, p, hb, reserved)
    return arr


GPT_BLOCK = [(128, 768, 2304, 0), (128, 768, 768, 0), (128, 768, 3072, 0), (128, 3072, 768, 0)]


def test_ghost_norm_layers_validation(lib):
    """The multi-layer norm call validates every layer before any HIP call
    and writes nothing on failure."""
    fn = lib.dp_ghost_norm_layers

    def call(arr, n=None, dt=1, B=64, mode=0, kappa=1, ws=FAKE, wsb=1 << 30, sq=FAKE):
        paths = (ctypes.c_int32 * 16)(*([-7] * 16))
        st = fn(None, arr, len(GPT_BLOCK) if n is None else n, dt, B, mode, kappa, ws, wsb, sq, 0, paths)
        return st, list(paths)

    ok = _layers(GPT_BLOCK)
    assert call(None)[0] == dpc.DP_ERR_NULL
    assert call(ok, n=0)[0] == dpc.DP_ERR_SHAPE
    assert call(ok, n=4097)[0] == dpc.DP_ERR_SHAPE
    assert call(ok, sq=None)[0] == dpc.DP_ERR_NULL
    assert call(ok, B=0)[0] == dpc.DP_ERR_SHAPE
    assert call(ok, dt=3)[0] == dpc.DP_ERR_DTYPE
    assert call(ok, mode=5)[0] == dpc.DP_ERR_VALUE
    assert call(ok, kappa=0)[0] == dpc.DP_ERR_VALUE
    assert call(_layers(GPT_BLOCK, reserved=1))[0] == dpc.DP_ERR_VALUE
    assert call(_layers(GPT_BLOCK, A=FAKE_MIS))[0] == dpc.DP_ERR_ALIGN
    assert call(_layers(GPT_BLOCK, G=None))[0] == dpc.DP_ERR_NULL
    bad = _layers(GPT_BLOCK[:3] + [(128, 0, 768, 0)])  # the last layer's d
    assert call(bad)[0] == dpc.DP_ERR_SHAPE
    assert call(ok, ws=None)[0] == dpc.DP_ERR_NULL
    st, paths = call(ok, wsb=16)
    assert st == dpc.DP_ERR_WORKSPACE and paths[:4] == [-7] * 4
    # an explicit layer beyond the per-sample tile limit fails the whole call
    huge = _layers(GPT_BLOCK[:1] + [(1 << 16, 1 << 15, 1 << 15, 0)])
    assert call(huge, n=2, B=1, mode=dpc.MODE_EXPLICIT)[0] == dpc.DP_ERR_SHAPE
    import torch
    if not torch.cuda.is_available():
        assert call(ok)[0] == dpc.DP_ERR_NO_DEVICE


def _r256(x):
    return (x + 255) // 256 * 256


def _norm_need_ok(lib, arr, n, dt, B, mode, need):
    """dp_ghost_norm_layers accepts a workspace of `need` bytes and refuses one
    byte less (validation only: with no GPU the valid call reports no device)."""
    paths = (ctypes.c_int32 * n)()
    fn = lib.dp_ghost_norm_layers
    if need > 0:
        assert fn(None, arr, n, dt, B, mode, 1, FAKE, need - 1, FAKE, 0, paths) == dpc.DP_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():  # fake pointers: only where nothing can launch
        st = fn(None, arr, n, dt, B, mode, 1, FAKE if need else None, need, FAKE, 0, paths)
        assert st == dpc.DP_ERR_NO_DEVICE, st
    assert lib.dp_layers_workspace_bytes(arr, n, dt, B, mode, 1) >= need


def test_layers_workspace_follows_the_runs(lib):
    """Consecutive ghost layers of one tile size share a launch (at most 8)
    whose tile partials ([B][tiles of the run] fp32) span all their tiles;
    other layers need their own."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("checks the no-device validation path")
    B = 64
    # four T = 128 layers on the long-sequence engine: one launch, one 128 x 128
    # Gram tile per layer and sample
    _norm_need_ok(lib, _layers(GPT_BLOCK), 4, 1, B, 0, _r256(B * 4 * 4))
    # T = 128 layers on the 64-row tiled kernel (d not a multiple of 64): 3 tiles
    # per layer and sample; nine layers: runs of 8 and 1
    tiled = (128, 136, 256, 0)
    _norm_need_ok(lib, _layers([tiled] * 9), 9, 1, B, 0, _r256(B * 24 * 4))
    # a T = 1 layer in between splits the run; it needs no workspace
    mixed = _layers([tiled, (1, 64, 32, 0), (128, 136, 128, 0)])
    _norm_need_ok(lib, mixed, 3, 1, B, 0, _r256(B * 3 * 4))
    # runs of one single-tile layer each: nothing
    _norm_need_ok(lib, _layers([GPT_BLOCK[0], (1, 64, 32, 0), GPT_BLOCK[1]]), 3, 1, B, 0, 0)
    # one single-tile ghost layer: nothing
    _norm_need_ok(lib, _layers([(64, 32, 48, 0)]), 1, 0, 5, dpc.MODE_GHOST, 0)
    # two single-tile ghost layers share a launch: two tiles per sample
    two = _layers([(64, 32, 48, 0), (40, 16, 16, 1)])
    _norm_need_ok(lib, two, 2, 0, 5, dpc.MODE_GHOST, _r256(5 * 2 * 4))
    # the long-sequence bf16 engine runs alone, with its own tile count
    assert lib.dp_layers_workspace_bytes(_layers([(1024, 1280, 3840, 0)]), 1, 1, 32, 0, 1) > 0
    assert lib.dp_layers_workspace_bytes(None, 1, 1, B, 0, 1) == 0
    assert lib.dp_layers_workspace_bytes(_layers(GPT_BLOCK), 0, 1, B, 0, 1) == 0


def test_unfold2d_validation(lib):
    """dp_unfold2d checks its arguments before any HIP call: NULL pointers,
    the dtype, geometry limits and U's 16-byte alignment."""
    import torch
    geo = dpc.conv_geometry(3, 8, 8, 3, 1, 1)
    fn = lib.dp_unfold2d
    assert fn(None, None, ctypes.byref(geo), 0, 2, FAKE) == dpc.DP_ERR_NULL
    assert fn(None, FAKE, ctypes.byref(geo), 0, 2, None) == dpc.DP_ERR_NULL
    assert fn(None, FAKE, None, 0, 2, FAKE) == dpc.DP_ERR_NULL
    assert fn(None, FAKE, ctypes.byref(geo), 7, 2, FAKE) == dpc.DP_ERR_DTYPE
    assert fn(None, FAKE, ctypes.byref(geo), 0, 2, FAKE + 4) == dpc.DP_ERR_ALIGN
    assert fn(None, FAKE, ctypes.byref(geo), 0, 0, FAKE) == dpc.DP_ERR_SHAPE
    bad = dpc.conv_geometry(3, 2, 2, 5, 1, 0)  # a kernel larger than the input
    assert fn(None, FAKE, ctypes.byref(bad), 0, 2, FAKE) == dpc.DP_ERR_SHAPE
    if not torch.cuda.is_available():
        assert fn(None, FAKE, ctypes.byref(geo), 0, 2, FAKE) == dpc.DP_ERR_NO_DEVICE


GPT2L_BLOCK = [(1024, 1280, 3840, 0), (1024, 1280, 1280, 0), (1024, 1280, 5120, 0), (1024, 5120, 1280, 0)]


def test_sum_layers_workspace_two_regions(lib):
    """A call with several shared contraction launches keeps each launch's
    split partials intact while the next launch reduces them: two regions,
    each as large as one launch's, used in turn; one launch needs one."""
    import torch
    B = 32
    one = lib.dp_layers_workspace_bytes(_layers(GPT2L_BLOCK * 2), 8, 1, B, 0, 1)
    two = lib.dp_layers_workspace_bytes(_layers(GPT2L_BLOCK * 4), 16, 1, B, 0, 1)
    three = lib.dp_layers_workspace_bytes(_layers(GPT2L_BLOCK * 6), 24, 1, B, 0, 1)
    assert one > 0 and one % 256 == 0
    assert two == 2 * one
    assert three == two
    fn = lib.dp_clipped_sum_noise_layers
    outs = (ctypes.c_void_p * 16)(*([FAKE] * 16))
    call = lambda wsb: fn(None, _layers(GPT2L_BLOCK * 4), 16, 1, B, FAKE, 1.0, 1.0, float(B), 0, None, 0, FAKE, wsb,
                          outs, None)
    assert call(two - 256) == dpc.DP_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert call(two) == dpc.DP_ERR_NO_DEVICE


def test_clipped_sum_layers_validation(lib):
    """The multi-layer clipped-sum call validates everything before any HIP
    call; its workspace need is covered by dp_layers_workspace_bytes."""
    fn = lib.dp_clipped_sum_noise_layers
    n = len(GPT_BLOCK)
    outs = (ctypes.c_void_p * n)(*([FAKE] * n))

    def call(arr=None, n_=n, dt=1, B=64, c=FAKE, C=1.0, sigma=1.0, denom=64.0, ws=FAKE, wsb=1 << 34, o=outs,
             b=None):
        arr = _layers(GPT_BLOCK) if arr is None else arr
        return fn(None, arr, n_, dt, B, c, C, sigma, denom, 0, None, 0, ws, wsb, o, b)

    assert fn(None, None, n, 1, 64, FAKE, 1.0, 1.0, 64.0, 0, None, 0, FAKE, 1 << 34, outs, None) == dpc.DP_ERR_NULL
    assert call(n_=0) == dpc.DP_ERR_SHAPE
    assert call(c=None) == dpc.DP_ERR_NULL
    assert call(o=None) == dpc.DP_ERR_NULL
    assert call(o=(ctypes.c_void_p * n)(FAKE, None, FAKE, FAKE)) == dpc.DP_ERR_NULL
    assert call(o=(ctypes.c_void_p * n)(FAKE, FAKE + 2, FAKE, FAKE)) == dpc.DP_ERR_ALIGN
    assert call(C=0.0) == dpc.DP_ERR_VALUE
    assert call(sigma=-1.0) == dpc.DP_ERR_VALUE
    assert call(denom=float("nan")) == dpc.DP_ERR_VALUE
    assert call(dt=4) == dpc.DP_ERR_DTYPE
    assert call(arr=_layers(GPT_BLOCK, reserved=2)) == dpc.DP_ERR_VALUE
    # a layer with a bias needs its bias output
    biased = _layers(GPT_BLOCK[:3] + [(128, 3072, 768, 1)])
    assert call(arr=biased) == dpc.DP_ERR_NULL
    assert call(arr=biased, b=(ctypes.c_void_p * n)(None, None, None, None)) == dpc.DP_ERR_NULL
    need = lib.dp_layers_workspace_bytes(_layers(GPT_BLOCK), n, 1, 64, 0, 1)
    assert need > 0
    assert call(ws=None) == dpc.DP_ERR_NULL
    assert call(wsb=need // 2) == dpc.DP_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert call(wsb=need) == dpc.DP_ERR_NO_DEVICE


def test_virtual_step_validation(lib):
    """dp_clipped_sum_accumulate and dp_noise_mean validate before any HIP
    call; accumulating needs room for the batch's sum in the workspace."""
    acc_fn = lib.dp_clipped_sum_accumulate

    def acc_call(A=FAKE, dt=1, B=4, T=64, d=128, p=64, c=FAKE, ws=FAKE, wsb=1 << 30, acc=FAKE, bacc=None, accum=1):
        return acc_fn(None, A, FAKE, dt, B, T, d, p, c, ws, wsb, acc, bacc, accum)

    assert acc_call(A=None) == dpc.DP_ERR_NULL
    assert acc_call(c=None) == dpc.DP_ERR_NULL
    assert acc_call(acc=None) == dpc.DP_ERR_NULL
    assert acc_call(acc=FAKE + 2) == dpc.DP_ERR_ALIGN
    assert acc_call(d=0) == dpc.DP_ERR_SHAPE
    assert acc_call(dt=7) == dpc.DP_ERR_DTYPE
    need = lib.dp_accumulate_workspace_bytes(1, 4, 64, 128, 64, 0)
    plain = lib.dp_workspace_bytes(1, 4, 64, 128, 64, 0, 1)
    assert need >= plain + 128 * 64 * 4
    assert acc_call(wsb=need - 1) == dpc.DP_ERR_WORKSPACE
    assert acc_call(ws=None) == dpc.DP_ERR_NULL
    assert lib.dp_accumulate_workspace_bytes(1, 0, 64, 128, 64, 0) == 0
    nm = lib.dp_noise_mean
    f = ctypes.c_float

    def nm_call(acc=FAKE, bacc=None, d=8, p=4, C=1.0, sigma=1.0, denom=4.0, out=FAKE, bout=None):
        return nm(None, acc, bacc, d, p, f(C), f(sigma), f(denom), 0, 0, 0, out, bout)

    assert nm_call(acc=None) == dpc.DP_ERR_NULL
    assert nm_call(out=None) == dpc.DP_ERR_NULL
    assert nm_call(bacc=FAKE) == dpc.DP_ERR_NULL          # bias in without bias out
    assert nm_call(bout=FAKE) == dpc.DP_ERR_NULL
    assert nm_call(d=0) == dpc.DP_ERR_SHAPE
    assert nm_call(d=1 << 20, p=1 << 15) == dpc.DP_ERR_SHAPE  # noise counters beyond 32 bits
    assert nm_call(C=0.0) == dpc.DP_ERR_VALUE
    assert nm_call(sigma=-1.0) == dpc.DP_ERR_VALUE
    assert nm_call(denom=0.0) == dpc.DP_ERR_VALUE
    assert nm_call(out=FAKE + 1) == dpc.DP_ERR_ALIGN
    import torch
    if not torch.cuda.is_available():
        assert nm_call() == dpc.DP_ERR_NO_DEVICE
        assert acc_call(wsb=need) == dpc.DP_ERR_NO_DEVICE


def test_engine_refuses_unclipped_parameters():
    """The privacy engine front end covers Linear and Conv2d layers only; any
    other trainable parameter (its per-sample gradient would go unclipped),
    a frozen weight beside a trainable bias, or grouped convolutions are
    refused when it is built (no GPU needed)."""
    import torch
    from sample_gradient_clipping_layer_amd.engine import PrivacyEngine
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Sequential(torch.nn.Linear(4, 4), torch.nn.LayerNorm(4)), C=1.0, sigma=1.0)
    frozen_w = torch.nn.Linear(4, 4)
    frozen_w.weight.requires_grad_(False)
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Sequential(frozen_w), C=1.0, sigma=1.0)
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Conv2d(4, 4, 3, groups=2), C=1.0, sigma=1.0)
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Linear(4, 4), C=1.0, sigma=1.0, mode="fast")
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Conv2d(3, 4, 3, padding="same"), C=1.0, sigma=1.0)
    with pytest.raises(ValueError):
        PrivacyEngine(torch.nn.Linear(4, 4), C=1.0, sigma=1.0, conv_input="im2col")
    assert PrivacyEngine(torch.nn.Conv2d(3, 4, 3, padding="valid"), C=1.0, sigma=1.0, conv_input="folded").folded
    e = PrivacyEngine(torch.nn.Sequential(torch.nn.Conv2d(3, 4, 3), torch.nn.Flatten(), torch.nn.Linear(4, 2)),
                      C=1.0, sigma=1.0)
    assert len(e.layers) == 2
    e.detach()


def test_accumulate_layers_validation(lib):
    fn = lib.dp_clipped_sum_accumulate_layers
    n = len(GPT_BLOCK)
    accs = (ctypes.c_void_p * n)(*([FAKE] * n))
    need = lib.dp_layers_accumulate_workspace_bytes(_layers(GPT_BLOCK), n, 1, 64)
    assert need >= sum(d * p * 4 for (_, d, p, _) in GPT_BLOCK)
    assert fn(None, None, n, 1, 64, FAKE, FAKE, need, accs, None, 1) == dpc.DP_ERR_NULL
    assert fn(None, _layers(GPT_BLOCK), n, 1, 64, None, FAKE, need, accs, None, 1) == dpc.DP_ERR_NULL
    assert fn(None, _layers(GPT_BLOCK), n, 1, 64, FAKE, FAKE, need, None, None, 1) == dpc.DP_ERR_NULL
    assert fn(None, _layers(GPT_BLOCK), n, 1, 64, FAKE, FAKE, need - 1, accs, None, 1) == dpc.DP_ERR_WORKSPACE
    assert fn(None, _layers(GPT_BLOCK), n, 1, 64, FAKE, None, need, accs, None, 1) == dpc.DP_ERR_NULL
    bad = (ctypes.c_void_p * n)(FAKE, FAKE, None, FAKE)
    assert fn(None, _layers(GPT_BLOCK), n, 1, 64, FAKE, FAKE, need, bad, None, 1) == dpc.DP_ERR_NULL
    assert lib.dp_layers_accumulate_workspace_bytes(None, n, 1, 64) == 0
    import torch
    if not torch.cuda.is_available():
        assert fn(None, _layers(GPT_BLOCK), n, 1, 64, FAKE, FAKE, need, accs, None, 1) == dpc.DP_ERR_NO_DEVICE


def test_norm_clip_layers_validation(lib):
    fn = lib.dp_ghost_norm_clip_layers
    f = ctypes.c_float
    n = len(GPT_BLOCK)
    paths = (ctypes.c_int32 * n)()

    def call(C=1.0, c=FAKE, norm=None, sq=FAKE, wsb=1 << 30):
        return fn(None, _layers(GPT_BLOCK), n, 1, 64, 0, 1, FAKE, wsb, sq, 0, f(C), c, norm, paths)

    assert call(c=None) == dpc.DP_ERR_NULL
    assert call(c=FAKE + 2) == dpc.DP_ERR_ALIGN
    assert call(norm=FAKE + 1) == dpc.DP_ERR_ALIGN
    for C in (0.0, -1.0, float("inf"), float("nan")):
        assert call(C=C) == dpc.DP_ERR_VALUE
    assert call(sq=None) == dpc.DP_ERR_NULL
    assert call(wsb=16) == dpc.DP_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert call() == dpc.DP_ERR_NO_DEVICE


def _conv(lib, a=FAKE, G=FAKE, geo=None, dt=0, B=4, p=6, hb=0, mode=0, kappa=1, ws=FAKE, wsb=1 << 20, sq=FAKE):
    geo = dpc.conv_geometry(3, 8, 8, 3, 1, 1) if geo is None else geo
    path = ctypes.c_int32(-7)
    st = lib.dp_conv_norm(None, a, G, ctypes.byref(geo) if geo is not False else None, dt, B, p, hb, mode, kappa,
                          ws, wsb, sq, 0, ctypes.byref(path))
    return st, path.value


def _conv_sum(lib, a=FAKE, G=FAKE, geo=None, dt=0, B=4, p=6, c=FAKE, C=1.0, sigma=1.0, denom=4.0, ws=FAKE,
              wsb=1 << 20, out=FAKE, bout=None):
    geo = dpc.conv_geometry(3, 8, 8, 3, 1, 1) if geo is None else geo
    return lib.dp_conv_clipped_sum_noise(None, a, G, ctypes.byref(geo), dt, B, p, c, C, sigma, denom, 0, 0, 0, ws,
                                         wsb, out, bout)


def test_conv_validation(lib):
    """Folded-input conv calls: geometry, pointers, alignment and scalars are
    checked before any device work; a failed call writes nothing."""
    g = dpc.conv_geometry
    assert _conv(lib, geo=False)[0] == dpc.DP_ERR_NULL
    assert _conv(lib, a=None)[0] == dpc.DP_ERR_NULL
    assert _conv(lib, sq=None)[0] == dpc.DP_ERR_NULL
    assert _conv(lib, geo=g(3, 8, 8, 3, 0, 1))[0] == dpc.DP_ERR_SHAPE          # stride 0
    assert _conv(lib, geo=g(3, 8, 8, 3, 1, -1))[0] == dpc.DP_ERR_SHAPE         # negative padding
    assert _conv(lib, geo=g(3, 8, 8, 3, 1, 1, 0))[0] == dpc.DP_ERR_SHAPE       # dilation 0
    assert _conv(lib, geo=g(3, 4, 4, 7, 1, 1))[0] == dpc.DP_ERR_SHAPE          # kernel beyond the padded input
    assert _conv(lib, geo=g(3, 4, 4, (3, 3), 1, 0, (2, 1)))[0] == dpc.DP_ERR_SHAPE  # dilated span 5 > 4
    assert _conv(lib, geo=g(1 << 12, 1 << 10, 1 << 10, 1))[0] == dpc.DP_ERR_SHAPE  # C_in*H*W >= 2^31
    assert _conv(lib, geo=g(0, 8, 8, 3, 1, 1))[0] == dpc.DP_ERR_SHAPE
    assert _conv(lib, B=0)[0] == dpc.DP_ERR_SHAPE
    assert _conv(lib, dt=2)[0] == dpc.DP_ERR_DTYPE
    assert _conv(lib, a=FAKE + 2)[0] == dpc.DP_ERR_ALIGN                        # fp32 input needs 4 bytes
    assert _conv(lib, G=FAKE_MIS)[0] == dpc.DP_ERR_ALIGN
    assert _conv(lib, mode=4)[0] == dpc.DP_ERR_VALUE
    import torch
    no_gpu = not torch.cuda.is_available()  # calls that pass validation use fake pointers: only where nothing launches
    if no_gpu:
        st, path = _conv(lib, ws=None, mode=dpc.MODE_GHOST)                     # T = 64: 1 tile, no workspace
        assert st == dpc.DP_ERR_NO_DEVICE
    big = g(3, 32, 32, 3, 1, 1)                                                 # T = 1024: tile partials
    assert _conv(lib, geo=big, ws=None, mode=dpc.MODE_GHOST)[0] == dpc.DP_ERR_NULL
    st, path = _conv(lib, geo=big, wsb=4, mode=dpc.MODE_GHOST)
    assert st == dpc.DP_ERR_WORKSPACE and path == -7
    assert _conv_sum(lib, c=None) == dpc.DP_ERR_NULL
    assert _conv_sum(lib, out=None) == dpc.DP_ERR_NULL
    assert _conv_sum(lib, C=0.0) == dpc.DP_ERR_VALUE
    assert _conv_sum(lib, sigma=-1.0) == dpc.DP_ERR_VALUE
    assert _conv_sum(lib, denom=float("nan")) == dpc.DP_ERR_VALUE
    assert _conv_sum(lib, bout=FAKE + 2) == dpc.DP_ERR_ALIGN
    if no_gpu:
        assert _conv_sum(lib, a=FAKE + 2, dt=1) == dpc.DP_ERR_NO_DEVICE         # bf16 input: 2-byte alignment


def test_conv_workspace_and_geometry(lib):
    """dp_conv_workspace_bytes covers the path the norm call takes (tiles of the
    tiled ghost kernel or the explicit tiles) and the contraction's splits; the
    binding's output shape is the oracle unfolding's."""
    import numpy as np
    from oracle.definitions import unfold2d
    for args in [(3, 32, 32, 3, 1, 1), (64, 16, 16, 3, 2, 1), (16, 9, 11, (5, 3), (2, 1), (2, 0), (1, 2)),
                 (5, 6, 6, 6, 1, 0)]:
        geo = dpc.conv_geometry(*args)
        x = np.zeros((1, geo.C_in, geo.H, geo.W))
        U = unfold2d(x, (geo.kh, geo.kw), (geo.stride_h, geo.stride_w), (geo.pad_h, geo.pad_w),
                     (geo.dil_h, geo.dil_w))
        assert dpc.conv_out_shape(geo) == U.shape[1:]
    big = dpc.conv_geometry(3, 32, 32, 3, 1, 1)
    w = dpc.dp_conv_workspace_bytes(big, dpc.DP_F32, 256, 64, False, dpc.MODE_GHOST)
    assert w >= 256 * 36 * 4                  # T = 1024: 8 x 8 blocks of 128 rows, 36 Gram tiles per sample
    assert dpc.dp_conv_workspace_bytes(dpc.conv_geometry(3, 4, 4, 7), dpc.DP_F32, 4, 6) == 0   # invalid
    assert dpc.dp_conv_workspace_bytes(big, dpc.DP_F32, 4, 6, mode=7) == 0


def test_conv_offset_limit_boundary(lib):
    """The folded-input kernels index one sample with 32-bit offsets: a
    geometry with (C_in + 2) * (H + 2 pad_h) * (W + 2 pad_w) just below 2^31
    passes validation (with no GPU present the call then reports
    DP_ERR_NO_DEVICE), one channel more is refused with DP_ERR_SHAPE before
    any device work."""
    ok = dpc.conv_geometry(2045, 1024, 1024, 1)      # 2047 * 2^20 < 2^31
    over = dpc.conv_geometry(2046, 1024, 1024, 1)    # 2048 * 2^20 = 2^31
    assert _conv(lib, geo=over, B=2, p=8, mode=dpc.MODE_EXPLICIT, wsb=1 << 40)[0] == dpc.DP_ERR_SHAPE
    assert dpc.dp_conv_workspace_bytes(over, dpc.DP_F32, 2, 8) == 0
    assert dpc.dp_conv_workspace_bytes(ok, dpc.DP_F32, 2, 8, mode=dpc.MODE_EXPLICIT) > 0
    import torch
    if not torch.cuda.is_available():  # fake pointers: only where nothing can launch
        assert _conv(lib, geo=ok, B=2, p=8, mode=dpc.MODE_EXPLICIT, wsb=1 << 40)[0] == dpc.DP_ERR_NO_DEVICE


class _FakeGpuTensor:
    """Stands in for a contiguous GPU tensor in binding-level checks that
    raise before any library call (its pointer is never used)."""

    def __init__(self, shape, dtype=None):
        import torch
        self.shape = tuple(shape)
        self.dtype = torch.float32 if dtype is None else dtype
        self.is_cuda = True
        self.device = "cuda:0"

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return FAKE

    def element_size(self):
        return 4


def test_binding_checks_bias_vectors_and_layer_ids(lib, monkeypatch):
    """The multi-layer binding validates every bias vector (float32, p
    elements, present for each layer with a bias) and layer_ids (one distinct
    uint32 per layer) before calling the library: a short or bf16 bias vector
    would take p fp32 writes past its end, and repeated ids would draw two
    layers' noise from one stream."""
    import torch

    def no_call(*a, **k):
        raise AssertionError("the library must not be called")

    # the stream is fetched as the library call's first argument: reaching it means every check passed
    monkeypatch.setattr(dpc, "_stream", no_call)
    monkeypatch.setattr(dpc, "_check", no_call)
    ws = _FakeGpuTensor((1 << 20,))
    layers = [(_FakeGpuTensor((4, 2, 8)), _FakeGpuTensor((4, 2, 16))),
              (_FakeGpuTensor((4, 2, 8)), _FakeGpuTensor((4, 2, 24)))]
    c = _FakeGpuTensor((4,))
    outs = [_FakeGpuTensor((8, 16)), _FakeGpuTensor((8, 24))]
    good_b = [_FakeGpuTensor((16,)), _FakeGpuTensor((24,))]
    call = lambda **kw: dpc.dp_clipped_sum_noise_layers(layers, c, 1.0, 1.0, 4.0, 0, 0, outs, workspace=ws, **kw)
    with pytest.raises(ValueError, match="required"):
        call(has_bias=True)                                            # no bias outputs at all
    with pytest.raises(ValueError, match="required"):
        call(has_bias=True, bias_outs=[good_b[0], None])               # one missing
    with pytest.raises(ValueError, match="p = 24"):
        call(has_bias=True, bias_outs=[good_b[0], _FakeGpuTensor((16,))])   # short
    with pytest.raises(ValueError, match="float32"):
        call(has_bias=True, bias_outs=[good_b[0], _FakeGpuTensor((24,), torch.bfloat16)])
    with pytest.raises(ValueError, match="one bias_outs entry"):
        call(has_bias=True, bias_outs=[good_b[0]])
    with pytest.raises(ValueError, match="one id per layer"):
        call(layer_ids=[3])
    with pytest.raises(ValueError, match="distinct"):
        call(layer_ids=[5, 5])
    with pytest.raises(ValueError, match="distinct"):
        call(layer_ids=[1, 1 << 32])
    accs = [_FakeGpuTensor((8, 16)), _FakeGpuTensor((8, 24))]
    with pytest.raises(ValueError, match="p = 16"):
        dpc.dp_clipped_sum_accumulate_layers(layers, c, accs, bias_accs=[_FakeGpuTensor((8,)), good_b[1]],
                                             has_bias=[True, False], workspace=ws)
    # entries of layers without a bias are ignored; the checks then pass and the call goes ahead
    with pytest.raises(AssertionError, match="must not be called"):
        call(has_bias=[False, True], bias_outs=[None, good_b[1]], layer_ids=[7, 2])


def test_noalloc_norm_call_validation(lib):
    """dp_ghost_norm_clip_layers_noalloc validates like the workspace call and
    refuses, before any HIP call, layer sets whose scratch would exceed its
    fixed 4 MiB array: four T = 1024 ghost layers (80 tiles per sample) need
    B * 80 * 4 bytes of tile partials, over 4 MiB from B = 13108 on."""
    def call(layers, n, B=14000, sq=FAKE, c=FAKE, C=1.0):
        return lib.dp_ghost_norm_clip_layers_noalloc(None, layers, n, dpc.DP_BF16, B, dpc.MODE_MIXED, 1, sq, 0,
                                                     C, c, None, None)
    wide = (dpc.DpLayer * 4)(*[dpc.DpLayer(FAKE, FAKE, 1024, 1024, 1024, 0, 0)] * 4)
    assert call(wide, 4, B=13108) == dpc.DP_ERR_WORKSPACE
    import torch
    if not torch.cuda.is_available():      # placeholder pointers: only where nothing can be launched
        assert call(wide, 4, B=13107) == dpc.DP_ERR_NO_DEVICE  # fits: goes on to the device check
    assert call(wide, 0) == dpc.DP_ERR_SHAPE
    assert call(wide, 1025) == dpc.DP_ERR_SHAPE
    assert call(None, 4) == dpc.DP_ERR_NULL
    assert call(wide, 4, sq=None) == dpc.DP_ERR_NULL
    assert call(wide, 4, c=None) == dpc.DP_ERR_NULL
    assert call(wide, 4, C=0.0) == dpc.DP_ERR_VALUE
    mis = (dpc.DpLayer * 1)(dpc.DpLayer(FAKE_MIS, FAKE, 1024, 1024, 1024, 0, 0))
    assert call(mis, 1) == dpc.DP_ERR_ALIGN
