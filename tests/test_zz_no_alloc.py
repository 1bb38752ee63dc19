"""dp_ghost_norm_clip_layers_noalloc (the entry point for callers that cannot
allocate) against dp_ghost_norm_clip_layers with a caller's workspace, through
the C ABI: bitwise equal squared norms, norms and clip factors on two calls
in a row, the second with a smaller input (fewer samples and layers, so the
scratch array still holds the first call's partials); a request
beyond the fixed scratch is refused before any work (a CPU test in
test_abi_cpu.py)."""
import ctypes

import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W

pytestmark = pytest.mark.gpu


def _dev_layers(B, specs, seed):
    rng = np.random.default_rng(seed)
    out = []
    for (T, d, p) in specs:
        A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32))
        G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) * 3.0 / np.sqrt(p)).astype(np.float32))
        out.append(tuple(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (A, G)))
    return out


def _call(fn, layers, C, noalloc):
    """One call through the C ABI; returns (status, sqnorm, norm, c, paths)."""
    lib = dpc.lib()
    dt, B, arr = dpc._layer_table(layers, False)
    sq = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    nrm = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    c = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    paths = (ctypes.c_int32 * len(layers))()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        status = lib.dp_ghost_norm_clip_layers_noalloc(st, arr, len(layers), dt, B, dpc.MODE_MIXED, 1,
                                                       ctypes.c_void_p(sq.data_ptr()), 0, float(C),
                                                       ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(nrm.data_ptr()),
                                                       paths)
    else:
        need = lib.dp_layers_workspace_bytes(arr, len(layers), dt, B, dpc.MODE_MIXED, 1)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        status = lib.dp_ghost_norm_clip_layers(st, arr, len(layers), dt, B, dpc.MODE_MIXED, 1,
                                               ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                               ctypes.c_void_p(sq.data_ptr()), 0, float(C),
                                               ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(nrm.data_ptr()),
                                               paths)
    torch.cuda.synchronize()
    return status, sq.cpu().numpy(), nrm.cpu().numpy(), c.cpu().numpy(), list(paths)


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    dpc.lib()


def test_noalloc_matches_workspace_call_twice():
    # first call: two layers at T = 1024 sharing a long-sequence ghost launch (20 tiles per
    # sample and layer) and two T = 128 layers sharing a tiled ghost launch; second call smaller
    cases = [
        (12, [(1024, 768, 1536), (1024, 1024, 1024), (128, 768, 2304), (128, 768, 768)], 1.0, 5),
        (5, [(128, 256, 512), (128, 512, 256)], 0.5, 6),
    ]
    for B, specs, C, seed in cases:
        layers = _dev_layers(B, specs, seed)
        got = _call(None, layers, C, noalloc=True)
        want = _call(None, layers, C, noalloc=False)
        assert got[0] == dpc.DP_OK and want[0] == dpc.DP_OK, (got[0], want[0])
        for k, name in ((1, "sqnorm"), (2, "norm"), (3, "c")):
            assert np.array_equal(_bits(got[k]), _bits(want[k])), (B, name)
        assert got[4] == want[4]
        assert np.all(np.isfinite(got[1])) and np.any(got[3] < 1.0)
