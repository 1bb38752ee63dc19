"""Python binding of libdpclip.so, the MI355X per-sample gradient clipping path.

Argument marshalling only: torch tensors are turned into device pointers and
sizes, the current HIP stream is passed along, and a status code other than
DP_OK raises ``DpError``. Every step of the path runs in the library's HIP
kernels; there is no CPU fallback, and a missing library raises on first use.

The functions mirror the C ABI in ``include/dpclip.h``:

    dp_ghost_norm(A, G, sqnorm, has_bias=False, mode=MODE_MIXED, kappa=1,
                  accumulate=False, workspace=None) -> path
    dp_ghost_norm_layers(layers, sqnorm, has_bias=False, mode=MODE_MIXED, kappa=1,
                         accumulate=False, workspace=None) -> [path, ...]
    dp_ghost_norm_clip_layers(layers, sqnorm, C, c, norm=None, has_bias=False, mode=MODE_MIXED, kappa=1,
                              accumulate=False, workspace=None) -> [path, ...]
    dp_ghost_norm_clip_layers_noalloc(layers, sqnorm, C, c, norm=None, has_bias=False, mode=MODE_MIXED,
                                      kappa=1, accumulate=False) -> [path, ...]   (allocates nothing)
    dp_layers_workspace_bytes(layers, has_bias=False, mode=MODE_MIXED, kappa=1) -> int
    dp_clipped_sum_noise_layers(layers, c, C, sigma, denom, seed, step, outs,
                                bias_outs=None, has_bias=False, layer_ids=None, workspace=None)
    dp_clipped_sum_accumulate(A, G, c, acc, bias_acc=None, accumulate=False, workspace=None)
    dp_clipped_sum_accumulate_layers(layers, c, accs, bias_accs=None, has_bias=False, accumulate=False,
                                     workspace=None)
    dp_noise_mean(acc, C, sigma, denom, seed, layer_id, step, out, bias_acc=None, bias_out=None)
    dp_clip_factors(sqnorm, C, c, norm=None)
    dp_clipped_sum_noise(A, G, c, C, sigma, denom, seed, layer_id, step, out,
                         bias_out=None, workspace=None)
    dp_adaptive_threshold(norm, C_prev, alpha, beta, sigma_l2, init, seed,
                          layer_id, step, C_next, C_l2_out=None)
    dp_workspace_bytes(dtype, B, T, d, p, mode=MODE_MIXED, kappa=1) -> int
    dp_choose_path(T, d, p, mode=MODE_MIXED, kappa=1) -> int
    dp_conv_norm(a, G, conv, sqnorm, has_bias=False, mode=MODE_MIXED, kappa=1,
                 accumulate=False, workspace=None) -> path
    dp_conv_clipped_sum_noise(a, G, conv, c, C, sigma, denom, seed, layer_id, step, out,
                              bias_out=None, workspace=None)
    dp_conv_workspace_bytes(conv, dtype, B, p, has_bias=False, mode=MODE_MIXED, kappa=1) -> int
    dp_unfold2d(a, conv, out=None) -> U [B, T, d]

The dp_conv_* calls take a convolution layer's folded input a [B, C_in, H, W]
and its geometry (``conv_geometry(C_in, H, W, kernel_size, stride, padding,
dilation)``); the unfolded rows are formed inside the kernels. dp_unfold2d
writes the unfolding U(a) itself, for the unfolded (multi-layer) calls.

A and G are contiguous [B, T, d] / [B, T, p] tensors (float32 or bfloat16) on
the current GPU; norm, factor and output vectors are float32. Every call also
takes ``stream=`` (a torch stream; default: torch's current stream).
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdpclip.so")

DP_OK = 0
DP_ERR_NULL, DP_ERR_SHAPE, DP_ERR_DTYPE, DP_ERR_VALUE = 1, 2, 3, 4
DP_ERR_WORKSPACE, DP_ERR_HIP, DP_ERR_NO_DEVICE, DP_ERR_ALIGN = 5, 6, 7, 8
DP_F32, DP_BF16 = 0, 1
MODE_MIXED, MODE_GHOST, MODE_EXPLICIT, MODE_TIME = 0, 1, 2, 3
PATH_GHOST, PATH_EXPLICIT, PATH_T1 = 1, 2, 3

EXPORTS = ("dp_ghost_norm", "dp_ghost_norm_layers", "dp_ghost_norm_clip_layers", "dp_ghost_norm_clip_layers_noalloc",
           "dp_layers_workspace_bytes", "dp_clipped_sum_noise_layers",
           "dp_clip_factors", "dp_clipped_sum_accumulate", "dp_noise_mean", "dp_accumulate_workspace_bytes",
           "dp_clipped_sum_accumulate_layers", "dp_layers_accumulate_workspace_bytes", "dp_clipped_sum_noise", "dp_adaptive_threshold",
           "dp_workspace_bytes", "dp_choose_path", "dp_status_string", "dp_abi_version",
           "dp_conv_norm", "dp_conv_clipped_sum_noise", "dp_conv_workspace_bytes", "dp_unfold2d")

_lib = None


class DpLayer(ctypes.Structure):
    """struct dp_layer of the C ABI."""
    _fields_ = [("A", ctypes.c_void_p), ("G", ctypes.c_void_p), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
                ("p", ctypes.c_int64), ("has_bias", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class DpConv2d(ctypes.Structure):
    """struct dp_conv2d of the C ABI."""
    _fields_ = [(n, ctypes.c_int64) for n in ("C_in", "H", "W", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w",
                                              "dil_h", "dil_w")]


def conv_geometry(C_in, H, W, kernel_size, stride=1, padding=0, dilation=1) -> DpConv2d:
    """DpConv2d from torch-style Conv2d arguments (ints or pairs)."""
    pair = lambda v: (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = pair(kernel_size), pair(stride), pair(padding), pair(dilation)
    return DpConv2d(int(C_in), int(H), int(W), kh, kw, sh, sw, ph, pw, dh, dw)


def conv_out_shape(g: DpConv2d):
    """(T, d) of the unfolded input U(a): T = H_out*W_out rows, d = C_in*kh*kw columns."""
    Ho = (g.H + 2 * g.pad_h - g.dil_h * (g.kh - 1) - 1) // g.stride_h + 1
    Wo = (g.W + 2 * g.pad_w - g.dil_w * (g.kw - 1) - 1) // g.stride_w + 1
    return Ho * Wo, g.C_in * g.kh * g.kw


class DpError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def _declare(lib):
    c_i64, c_i32, c_u32, c_u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
    vp, fp, f = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float
    lib.dp_ghost_norm.argtypes = [vp, vp, vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32,
                                  vp, ctypes.c_size_t, fp, c_i32, ctypes.POINTER(c_i32)]
    lib.dp_ghost_norm.restype = c_i32
    lp = ctypes.POINTER(DpLayer)
    lib.dp_ghost_norm_layers.argtypes = [vp, lp, c_i32, c_i32, c_i64, c_i32, c_i32, vp, ctypes.c_size_t, fp, c_i32,
                                         ctypes.POINTER(c_i32)]
    lib.dp_ghost_norm_layers.restype = c_i32
    lib.dp_ghost_norm_clip_layers.argtypes = [vp, lp, c_i32, c_i32, c_i64, c_i32, c_i32, vp, ctypes.c_size_t, fp,
                                              c_i32, f, fp, fp, ctypes.POINTER(c_i32)]
    lib.dp_ghost_norm_clip_layers.restype = c_i32
    lib.dp_ghost_norm_clip_layers_noalloc.argtypes = [vp, lp, c_i32, c_i32, c_i64, c_i32, c_i32, fp, c_i32, f, fp,
                                                      fp, ctypes.POINTER(c_i32)]
    lib.dp_ghost_norm_clip_layers_noalloc.restype = c_i32
    lib.dp_clipped_sum_noise_layers.argtypes = [vp, lp, c_i32, c_i32, c_i64, fp, f, f, f, c_u64,
                                                ctypes.POINTER(c_u32), c_u32, vp, ctypes.c_size_t,
                                                ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.dp_clipped_sum_noise_layers.restype = c_i32
    lib.dp_clipped_sum_accumulate.argtypes = [vp, vp, vp, c_i32, c_i64, c_i64, c_i64, c_i64, fp, vp, ctypes.c_size_t,
                                              fp, fp, c_i32]
    lib.dp_clipped_sum_accumulate.restype = c_i32
    lib.dp_clipped_sum_accumulate_layers.argtypes = [vp, lp, c_i32, c_i32, c_i64, fp, vp, ctypes.c_size_t,
                                                     ctypes.POINTER(vp), ctypes.POINTER(vp), c_i32]
    lib.dp_clipped_sum_accumulate_layers.restype = c_i32
    lib.dp_layers_accumulate_workspace_bytes.argtypes = [lp, c_i32, c_i32, c_i64]
    lib.dp_layers_accumulate_workspace_bytes.restype = ctypes.c_size_t
    lib.dp_noise_mean.argtypes = [vp, fp, fp, c_i64, c_i64, f, f, f, c_u64, c_u32, c_u32, fp, fp]
    lib.dp_noise_mean.restype = c_i32
    lib.dp_accumulate_workspace_bytes.argtypes = [c_i32, c_i64, c_i64, c_i64, c_i64, c_i32]
    lib.dp_accumulate_workspace_bytes.restype = ctypes.c_size_t
    lib.dp_layers_workspace_bytes.argtypes = [lp, c_i32, c_i32, c_i64, c_i32, c_i32]
    lib.dp_layers_workspace_bytes.restype = ctypes.c_size_t
    lib.dp_clip_factors.argtypes = [vp, fp, c_i64, f, fp, fp]
    lib.dp_clip_factors.restype = c_i32
    lib.dp_clipped_sum_noise.argtypes = [vp, vp, vp, c_i32, c_i64, c_i64, c_i64, c_i64, fp, f, f, f,
                                         c_u64, c_u32, c_u32, vp, ctypes.c_size_t, fp, fp]
    lib.dp_clipped_sum_noise.restype = c_i32
    lib.dp_adaptive_threshold.argtypes = [vp, fp, c_i64, f, f, f, f, c_i32, c_u64, c_u32, c_u32, fp, fp]
    lib.dp_adaptive_threshold.restype = c_i32
    lib.dp_workspace_bytes.argtypes = [c_i32, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32]
    lib.dp_workspace_bytes.restype = ctypes.c_size_t
    lib.dp_choose_path.argtypes = [c_i64, c_i64, c_i64, c_i32, c_i32]
    lib.dp_choose_path.restype = c_i32
    lib.dp_status_string.argtypes = [c_i32]
    lib.dp_status_string.restype = ctypes.c_char_p
    cp = ctypes.POINTER(DpConv2d)
    lib.dp_conv_norm.argtypes = [vp, vp, vp, cp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32, vp, ctypes.c_size_t, fp,
                                 c_i32, ctypes.POINTER(c_i32)]
    lib.dp_conv_norm.restype = c_i32
    lib.dp_conv_clipped_sum_noise.argtypes = [vp, vp, vp, cp, c_i32, c_i64, c_i64, fp, f, f, f, c_u64, c_u32, c_u32,
                                              vp, ctypes.c_size_t, fp, fp]
    lib.dp_conv_clipped_sum_noise.restype = c_i32
    lib.dp_conv_workspace_bytes.argtypes = [cp, c_i32, c_i64, c_i64, c_i32, c_i32, c_i32]
    lib.dp_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.dp_unfold2d.argtypes = [vp, vp, cp, c_i32, c_i64, vp]
    lib.dp_unfold2d.restype = c_i32
    lib.dp_abi_version.argtypes = []
    lib.dp_abi_version.restype = c_i32
    return lib


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sample_gradient_clipping_layer_amd._build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(fn: str, status: int):
    if status != DP_OK:
        raise DpError(fn, status, lib().dp_status_string(status).decode())


def _stream(stream=None):
    """HIP stream handle: the given torch stream, else torch's current one."""
    import torch
    st = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(st.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DP_F32
    if t.dtype == torch.bfloat16:
        return DP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; float32 or bfloat16")


def _layer(A, G):
    if A.dim() != 3 or G.dim() != 3 or A.shape[:2] != G.shape[:2]:
        raise ValueError(f"A [B,T,d] and G [B,T,p] expected, got {tuple(A.shape)} and {tuple(G.shape)}")
    if A.dtype != G.dtype:
        raise TypeError("A and G must share one dtype")
    if not (A.is_contiguous() and G.is_contiguous()):
        raise ValueError("A and G must be contiguous")
    if not (A.is_cuda and G.is_cuda):
        raise ValueError("A and G must be GPU tensors")
    B, T, d = A.shape
    return _dtype_code(A), int(B), int(T), int(d), int(G.shape[2])


def _f32_vec(t, name):
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor")


def dp_workspace_bytes(dtype: int, B: int, T: int, d: int, p: int, mode: int = MODE_MIXED, kappa: int = 1) -> int:
    return int(lib().dp_workspace_bytes(dtype, B, T, d, p, mode, kappa))


def dp_choose_path(T: int, d: int, p: int, mode: int = MODE_MIXED, kappa: int = 1) -> int:
    return int(lib().dp_choose_path(T, d, p, mode, kappa))


def dp_abi_version() -> int:
    return int(lib().dp_abi_version())


def dp_status_string(status: int) -> str:
    return lib().dp_status_string(status).decode()


def _scratch(nbytes: int, device, stream=None):
    """A workspace of at least nbytes (>= 256) that the binding allocates for
    one call. torch's caching allocator ties a block to the stream current at
    allocation; when the call runs on another stream, record_stream keeps the
    block from being handed out again before that stream has passed the call
    (the library keeps every buffer in use until then)."""
    import torch
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def _ws_bytes(workspace) -> int:
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.numel() * workspace.element_size()


def _workspace(workspace, dt, B, T, d, p, mode, kappa, device, stream=None):
    if workspace is None:
        workspace = _scratch(dp_workspace_bytes(dt, B, T, d, p, mode, kappa), device, stream)
    return workspace, _ws_bytes(workspace)


def _bias_ptrs(vecs, arr, n, name):
    """ctypes array of the per-layer bias vectors (None where a layer has no
    bias). Entry l must be a contiguous float32 GPU vector of p_l elements
    when layer l has a bias; entries of layers without one are ignored."""
    if vecs is None:
        if any(arr[k].has_bias for k in range(n)):
            raise ValueError(f"{name} is required when a layer has a bias")
        return None
    if len(vecs) != n:
        raise ValueError(f"one {name} entry (or None) per layer")
    ptrs = []
    for k, b in enumerate(vecs):
        if not arr[k].has_bias:
            ptrs.append(None)
            continue
        if b is None:
            raise ValueError(f"{name}[{k}] is required: layer {k} has a bias")
        _f32_vec(b, f"{name}[{k}]")
        if b.numel() != arr[k].p:
            raise ValueError(f"{name}[{k}] must have p = {arr[k].p} elements")
        ptrs.append(b.data_ptr())
    return (ctypes.c_void_p * n)(*ptrs)


def dp_ghost_norm(A, G, sqnorm, has_bias: bool = False, mode: int = MODE_MIXED, kappa: int = 1,
                  accumulate: bool = False, workspace=None, stream=None) -> int:
    dt, B, T, d, p = _layer(A, G)
    _f32_vec(sqnorm, "sqnorm")
    if sqnorm.numel() != B:
        raise ValueError("sqnorm must have B elements")
    ws, nbytes = _workspace(workspace, dt, B, T, d, p, mode, kappa, A.device, stream)
    path = ctypes.c_int32(0)
    _check("dp_ghost_norm", lib().dp_ghost_norm(_stream(stream), _ptr(A), _ptr(G), dt, B, T, d, p, int(bool(has_bias)),
                                                int(mode), int(kappa), _ptr(ws), nbytes, _ptr(sqnorm),
                                                int(bool(accumulate)), ctypes.byref(path)))
    return path.value


def _layer_table(layers, has_bias):
    """(dtype, B, ctypes array of DpLayer) for a list of (A, G) pairs;
    has_bias is one flag for all layers or one per layer."""
    if len(layers) < 1:
        raise ValueError("at least one layer")
    flags = list(has_bias) if isinstance(has_bias, (list, tuple)) else [has_bias] * len(layers)
    if len(flags) != len(layers):
        raise ValueError("one has_bias flag per layer")
    arr = (DpLayer * len(layers))()
    dt0 = B0 = None
    for k, ((A, G), hb) in enumerate(zip(layers, flags)):
        dt, B, T, d, p = _layer(A, G)
        if dt0 is None:
            dt0, B0 = dt, B
        elif dt != dt0 or B != B0:
            raise ValueError("all layers must share one dtype and batch size")
        arr[k] = DpLayer(A.data_ptr(), G.data_ptr(), T, d, p, int(bool(hb)), 0)
    return dt0, B0, arr


def dp_layers_workspace_bytes(layers, has_bias=False, mode: int = MODE_MIXED, kappa: int = 1) -> int:
    dt, B, arr = _layer_table(layers, has_bias)
    return int(lib().dp_layers_workspace_bytes(arr, len(layers), dt, B, int(mode), int(kappa)))


def dp_ghost_norm_layers(layers, sqnorm, has_bias=False, mode: int = MODE_MIXED, kappa: int = 1,
                         accumulate: bool = False, workspace=None, stream=None):
    """Squared norms summed over `layers` (a list of (A, G) pairs) into sqnorm."""
    dt, B, arr = _layer_table(layers, has_bias)
    _f32_vec(sqnorm, "sqnorm")
    if sqnorm.numel() != B:
        raise ValueError("sqnorm must have B elements")
    if workspace is None:
        workspace = _scratch(lib().dp_layers_workspace_bytes(arr, len(layers), dt, B, int(mode), int(kappa)),
                             sqnorm.device, stream)
    paths = (ctypes.c_int32 * len(layers))()
    _check("dp_ghost_norm_layers", lib().dp_ghost_norm_layers(
        _stream(stream), arr, len(layers), dt, B, int(mode), int(kappa), _ptr(workspace),
        _ws_bytes(workspace), _ptr(sqnorm), int(bool(accumulate)), paths))
    return list(paths)


def dp_ghost_norm_clip_layers(layers, sqnorm, C: float, c, norm=None, has_bias=False, mode: int = MODE_MIXED,
                              kappa: int = 1, accumulate: bool = False, workspace=None, stream=None):
    """dp_ghost_norm_layers plus the clip factors (and norms) of the result, in the same pass."""
    dt, B, arr = _layer_table(layers, has_bias)
    for t, nm in ((sqnorm, "sqnorm"), (c, "c")) + (((norm, "norm"),) if norm is not None else ()):
        _f32_vec(t, nm)
        if t.numel() != B:
            raise ValueError(f"{nm} must have B elements")
    if workspace is None:
        workspace = _scratch(lib().dp_layers_workspace_bytes(arr, len(layers), dt, B, int(mode), int(kappa)),
                             sqnorm.device, stream)
    paths = (ctypes.c_int32 * len(layers))()
    _check("dp_ghost_norm_clip_layers", lib().dp_ghost_norm_clip_layers(
        _stream(stream), arr, len(layers), dt, B, int(mode), int(kappa), _ptr(workspace),
        _ws_bytes(workspace), _ptr(sqnorm), int(bool(accumulate)), float(C), _ptr(c),
        _ptr(norm), paths))
    return list(paths)


def dp_ghost_norm_clip_layers_noalloc(layers, sqnorm, C: float, c, norm=None, has_bias=False,
                                      mode: int = MODE_MIXED, kappa: int = 1, accumulate: bool = False, stream=None):
    """dp_ghost_norm_clip_layers with the library's fixed scratch array instead
    of a workspace: allocates nothing. Calls that overlap on one GPU race."""
    dt, B, arr = _layer_table(layers, has_bias)
    for t, nm in ((sqnorm, "sqnorm"), (c, "c")) + (((norm, "norm"),) if norm is not None else ()):
        _f32_vec(t, nm)
        if t.numel() != B:
            raise ValueError(f"{nm} must have B elements")
    paths = (ctypes.c_int32 * len(layers))()
    _check("dp_ghost_norm_clip_layers_noalloc", lib().dp_ghost_norm_clip_layers_noalloc(
        _stream(stream), arr, len(layers), dt, B, int(mode), int(kappa), _ptr(sqnorm), int(bool(accumulate)),
        float(C), _ptr(c), _ptr(norm), paths))
    return list(paths)


def dp_clipped_sum_noise_layers(layers, c, C: float, sigma: float, denom: float, seed: int, step: int, outs,
                                bias_outs=None, has_bias=False, layer_ids=None, workspace=None, stream=None):
    """Clipped noised means of `layers` (a list of (A, G) pairs) under one c
    into outs[l] ([d_l, p_l]); bias_outs[l] for the layers with a bias."""
    dt, B, arr = _layer_table(layers, has_bias)
    n = len(layers)
    _f32_vec(c, "c")
    if c.numel() != B or len(outs) != n:
        raise ValueError("c must have B elements and outs one tensor per layer")
    for k, o in enumerate(outs):
        _f32_vec(o, "outs[k]")
        if o.numel() != arr[k].d * arr[k].p:
            raise ValueError(f"outs[{k}] must have d*p elements")
    bptr = _bias_ptrs(bias_outs, arr, n, "bias_outs")
    ids = None
    if layer_ids is not None:
        ids_list = [int(v) for v in layer_ids]
        if len(ids_list) != n:
            raise ValueError("layer_ids must hold one id per layer")
        if any(v < 0 or v > 0xFFFFFFFF for v in ids_list) or len(set(ids_list)) != n:
            raise ValueError("layer_ids must be distinct uint32 values (each layer its own noise stream)")
        ids = (ctypes.c_uint32 * n)(*ids_list)
    if workspace is None:
        workspace = _scratch(lib().dp_layers_workspace_bytes(arr, n, dt, B, MODE_MIXED, 1), c.device, stream)
    optr = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    _check("dp_clipped_sum_noise_layers", lib().dp_clipped_sum_noise_layers(
        _stream(stream), arr, n, dt, B, _ptr(c), float(C), float(sigma), float(denom),
        int(seed) & 0xFFFFFFFFFFFFFFFF, ids, int(step) & 0xFFFFFFFF, _ptr(workspace),
        _ws_bytes(workspace), optr, bptr))


def dp_clipped_sum_accumulate(A, G, c, acc, bias_acc=None, accumulate: bool = False, workspace=None, stream=None):
    """acc (+)= the clipped sum of one physical batch (no noise, no mean)."""
    dt, B, T, d, p = _layer(A, G)
    _f32_vec(c, "c")
    _f32_vec(acc, "acc")
    if c.numel() != B or acc.numel() != d * p:
        raise ValueError("c must have B elements and acc d*p")
    if bias_acc is not None:
        _f32_vec(bias_acc, "bias_acc")
        if bias_acc.numel() != p:
            raise ValueError("bias_acc must have p elements")
    if workspace is None:
        workspace = _scratch(lib().dp_accumulate_workspace_bytes(dt, B, T, d, p, int(bias_acc is not None)),
                             A.device, stream)
    _check("dp_clipped_sum_accumulate", lib().dp_clipped_sum_accumulate(
        _stream(stream), _ptr(A), _ptr(G), dt, B, T, d, p, _ptr(c), _ptr(workspace),
        _ws_bytes(workspace), _ptr(acc), _ptr(bias_acc), int(bool(accumulate))))


def dp_clipped_sum_accumulate_layers(layers, c, accs, bias_accs=None, has_bias=False, accumulate: bool = False,
                                     workspace=None, stream=None):
    """accs[l] (+)= the clipped sum of layer l over one physical batch (no noise, no mean)."""
    dt, B, arr = _layer_table(layers, has_bias)
    n = len(layers)
    _f32_vec(c, "c")
    if c.numel() != B or len(accs) != n:
        raise ValueError("c must have B elements and accs one tensor per layer")
    for k, a in enumerate(accs):
        _f32_vec(a, "accs[k]")
        if a.numel() != arr[k].d * arr[k].p:
            raise ValueError(f"accs[{k}] must have d*p elements")
    bptr = _bias_ptrs(bias_accs, arr, n, "bias_accs")
    if workspace is None:
        workspace = _scratch(lib().dp_layers_accumulate_workspace_bytes(arr, n, dt, B), c.device, stream)
    aptr = (ctypes.c_void_p * n)(*[a.data_ptr() for a in accs])
    _check("dp_clipped_sum_accumulate_layers", lib().dp_clipped_sum_accumulate_layers(
        _stream(stream), arr, n, dt, B, _ptr(c), _ptr(workspace), _ws_bytes(workspace),
        aptr, bptr, int(bool(accumulate))))


def dp_noise_mean(acc, C: float, sigma: float, denom: float, seed: int, layer_id: int, step: int, out,
                  bias_acc=None, bias_out=None, stream=None):
    """out = (acc + sigma*C*z) / denom, the noise of dp_clipped_sum_noise; acc is [d, p]."""
    _f32_vec(acc, "acc")
    _f32_vec(out, "out")
    if acc.dim() != 2 or out.shape != acc.shape:
        raise ValueError("acc and out must be [d, p]")
    d, p = int(acc.shape[0]), int(acc.shape[1])
    if (bias_acc is None) != (bias_out is None):
        raise ValueError("bias_acc and bias_out go together")
    if bias_acc is not None:
        _f32_vec(bias_acc, "bias_acc")
        _f32_vec(bias_out, "bias_out")
        if bias_acc.numel() != p or bias_out.numel() != p:
            raise ValueError("bias vectors must have p elements")
    _check("dp_noise_mean", lib().dp_noise_mean(
        _stream(stream), _ptr(acc), _ptr(bias_acc), d, p, float(C), float(sigma), float(denom),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(layer_id) & 0xFFFFFFFF, int(step) & 0xFFFFFFFF, _ptr(out),
        _ptr(bias_out)))


def dp_clip_factors(sqnorm, C: float, c, norm=None, stream=None):
    _f32_vec(sqnorm, "sqnorm")
    _f32_vec(c, "c")
    if norm is not None:
        _f32_vec(norm, "norm")
    B = sqnorm.numel()
    if c.numel() != B or (norm is not None and norm.numel() != B):
        raise ValueError("sqnorm, c and norm must have the same length")
    _check("dp_clip_factors", lib().dp_clip_factors(_stream(stream), _ptr(sqnorm), B, float(C), _ptr(c), _ptr(norm)))


def dp_clipped_sum_noise(A, G, c, C: float, sigma: float, denom: float, seed: int, layer_id: int, step: int,
                         out, bias_out=None, workspace=None, stream=None):
    dt, B, T, d, p = _layer(A, G)
    _f32_vec(c, "c")
    _f32_vec(out, "out")
    if c.numel() != B or out.numel() != d * p:
        raise ValueError("c must have B elements and out d*p")
    if bias_out is not None:
        _f32_vec(bias_out, "bias_out")
        if bias_out.numel() != p:
            raise ValueError("bias_out must have p elements")
    ws, nbytes = _workspace(workspace, dt, B, T, d, p, MODE_MIXED, 1, A.device, stream)
    _check("dp_clipped_sum_noise", lib().dp_clipped_sum_noise(
        _stream(stream), _ptr(A), _ptr(G), dt, B, T, d, p, _ptr(c), float(C), float(sigma), float(denom),
        int(seed) & 0xFFFFFFFFFFFFFFFF, int(layer_id) & 0xFFFFFFFF, int(step) & 0xFFFFFFFF, _ptr(ws), nbytes,
        _ptr(out), _ptr(bias_out)))


def dp_adaptive_threshold(norm, C_prev: float, alpha: float, beta: float, sigma_l2: float, init: bool, seed: int,
                          layer_id: int, step: int, C_next, C_l2_out=None, stream=None):
    """One update of TTP's adaptive per-layer bound into C_next (a device
    scalar). With init=True, C_l2 is the plain mean of `norm` (no noise): those
    norms must come from a data-independent batch (TTP: one iteration on
    random noise), never from private training data."""
    _f32_vec(norm, "norm")
    _f32_vec(C_next, "C_next")
    if C_l2_out is not None:
        _f32_vec(C_l2_out, "C_l2_out")
    _check("dp_adaptive_threshold", lib().dp_adaptive_threshold(
        _stream(stream), _ptr(norm), norm.numel(), float(C_prev), float(alpha), float(beta), float(sigma_l2),
        int(bool(init)), int(seed) & 0xFFFFFFFFFFFFFFFF, int(layer_id) & 0xFFFFFFFF, int(step) & 0xFFFFFFFF,
        _ptr(C_next), _ptr(C_l2_out)))


def _conv_layer(a, G, conv: DpConv2d):
    """(dtype, B, T, d, p) of a conv layer given by its folded input a [B, C_in, H, W]."""
    if a.dim() != 4 or G.dim() != 3 or a.shape[0] != G.shape[0]:
        raise ValueError(f"a [B,C_in,H,W] and G [B,T,p] expected, got {tuple(a.shape)} and {tuple(G.shape)}")
    if tuple(a.shape[1:]) != (conv.C_in, conv.H, conv.W):
        raise ValueError("a's shape does not match the geometry")
    T, d = conv_out_shape(conv)
    if G.shape[1] != T:
        raise ValueError(f"G must have T = H_out*W_out = {T} rows per sample")
    if a.dtype != G.dtype:
        raise TypeError("a and G must share one dtype")
    if not (a.is_contiguous() and G.is_contiguous() and a.is_cuda and G.is_cuda):
        raise ValueError("a and G must be contiguous GPU tensors")
    return _dtype_code(a), int(a.shape[0]), T, d, int(G.shape[2])


def dp_conv_workspace_bytes(conv: DpConv2d, dtype: int, B: int, p: int, has_bias: bool = False,
                            mode: int = MODE_MIXED, kappa: int = 1) -> int:
    return int(lib().dp_conv_workspace_bytes(ctypes.byref(conv), dtype, B, p, int(bool(has_bias)), int(mode),
                                             int(kappa)))


def _conv_ws(workspace, conv, dt, B, p, has_bias, mode, kappa, device, stream=None):
    if workspace is None:
        workspace = _scratch(dp_conv_workspace_bytes(conv, dt, B, p, has_bias, mode, kappa), device, stream)
    return workspace, _ws_bytes(workspace)


def dp_conv_norm(a, G, conv: DpConv2d, sqnorm, has_bias: bool = False, mode: int = MODE_MIXED, kappa: int = 1,
                 accumulate: bool = False, workspace=None, stream=None) -> int:
    """Per-sample squared norms of a conv layer from its folded input a
    [B, C_in, H, W] and G [B, T, p] into sqnorm; returns the path taken."""
    dt, B, T, d, p = _conv_layer(a, G, conv)
    _f32_vec(sqnorm, "sqnorm")
    if sqnorm.numel() != B:
        raise ValueError("sqnorm must have B elements")
    ws, nbytes = _conv_ws(workspace, conv, dt, B, p, has_bias, mode, kappa, a.device, stream)
    path = ctypes.c_int32(0)
    _check("dp_conv_norm", lib().dp_conv_norm(_stream(stream), _ptr(a), _ptr(G), ctypes.byref(conv), dt, B, p,
                                              int(bool(has_bias)), int(mode), int(kappa), _ptr(ws), nbytes,
                                              _ptr(sqnorm), int(bool(accumulate)), ctypes.byref(path)))
    return path.value


def dp_unfold2d(a, conv: DpConv2d, out=None, stream=None):
    """U(a) [B, T, d] of a conv layer's folded input a [B, C_in, H, W] (torch's
    unfold(a).transpose(1, 2) layout), written by the library into `out`
    (allocated when None); returns it."""
    if a.dim() != 4 or tuple(a.shape[1:]) != (conv.C_in, conv.H, conv.W):
        raise ValueError("a [B, C_in, H, W] matching the geometry expected")
    if not (a.is_contiguous() and a.is_cuda):
        raise ValueError("a must be a contiguous GPU tensor")
    T, d = conv_out_shape(conv)
    B = int(a.shape[0])
    if out is None:
        import torch
        out = torch.empty(B, T, d, dtype=a.dtype, device=a.device)
    elif tuple(out.shape) != (B, T, d) or out.dtype != a.dtype or not (out.is_contiguous() and out.is_cuda):
        raise ValueError(f"out must be a contiguous GPU tensor [B, T, d] = {(B, T, d)} of a's dtype")
    _check("dp_unfold2d", lib().dp_unfold2d(_stream(stream), _ptr(a), ctypes.byref(conv), _dtype_code(a), B,
                                            _ptr(out)))
    return out


def dp_conv_clipped_sum_noise(a, G, conv: DpConv2d, c, C: float, sigma: float, denom: float, seed: int,
                              layer_id: int, step: int, out, bias_out=None, workspace=None, stream=None):
    """Clipped noised mean of a conv layer from its folded input into out ([d, p])."""
    dt, B, T, d, p = _conv_layer(a, G, conv)
    _f32_vec(c, "c")
    _f32_vec(out, "out")
    if c.numel() != B or out.numel() != d * p:
        raise ValueError("c must have B elements and out d*p")
    if bias_out is not None:
        _f32_vec(bias_out, "bias_out")
        if bias_out.numel() != p:
            raise ValueError("bias_out must have p elements")
    ws, nbytes = _conv_ws(workspace, conv, dt, B, p, bias_out is not None, MODE_MIXED, 1, a.device, stream)
    _check("dp_conv_clipped_sum_noise", lib().dp_conv_clipped_sum_noise(
        _stream(stream), _ptr(a), _ptr(G), ctypes.byref(conv), dt, B, p, _ptr(c), float(C), float(sigma),
        float(denom), int(seed) & 0xFFFFFFFFFFFFFFFF, int(layer_id) & 0xFFFFFFFF, int(step) & 0xFFFFFFFF, _ptr(ws),
        nbytes, _ptr(out), _ptr(bias_out)))
