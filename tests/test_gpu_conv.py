"""GPU parity of the folded-input convolution entry points (dp_conv_norm,
dp_conv_clipped_sum_noise), through the C ABI, against the oracle's unfolding
U(a) and its layer definitions.

The kernels form U(a)'s rows from the folded input a [B, C_in, H, W]; the
oracle unfolds a in fp64 (definitions.unfold2d) and applies the same per-layer
definitions as for a linear layer. Cases span several tiles, ragged tails
(d = 27, T = 121, odd p), stride, padding, dilation, rectangular kernels and
the T = 1 case; the full-size cases are ResNet-18 layers of the benchmark.
"""
import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import definitions as D
from oracle import noise as N

from gpu_util import assert_noised, assert_norms, assert_sum, dev, f32, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    dpc.lib()


GEOMS = {  # B, C_in, H, W, kernel, stride, padding, dilation, p
    "stem-3x3": (5, 3, 32, 32, (3, 3), (1, 1), (1, 1), (1, 1), 64),      # d = 27, T = 1024
    "s2-3x3": (4, 64, 16, 16, (3, 3), (2, 2), (1, 1), (1, 1), 40),       # d = 576, T = 64
    "rect-dil": (3, 16, 9, 11, (5, 3), (2, 1), (2, 0), (1, 2), 33),      # rectangular, dilated, ragged
    "1x1-s2": (6, 32, 8, 8, (1, 1), (2, 2), (0, 0), (1, 1), 48),         # downsample shortcut
    "valid-3x3": (2, 7, 13, 13, (3, 3), (1, 1), (0, 0), (1, 1), 130),    # T = 121, p ragged
    "late-3x3": (3, 20, 4, 4, (3, 3), (1, 1), (1, 1), (1, 1), 96),       # T = 16
    "t1": (4, 5, 6, 6, (6, 6), (1, 1), (0, 0), (1, 1), 24),              # one output position
    "mid-3x3": (16, 128, 16, 16, (3, 3), (1, 1), (1, 1), (1, 1), 128),   # T = 256, d = 1152: 4 row blocks
    "b1-dil2": (1, 1, 5, 5, (3, 3), (1, 1), (2, 2), (2, 2), 3),          # one sample, one channel, d = 9
    "wide-stride": (2, 3, 10, 17, (2, 5), (3, 4), (1, 2), (1, 1), 20),   # strides larger than the kernel rows
}


def _case(name, dtype):
    B, cin, H, Wd, k, s, pad, dil, p = GEOMS[name]
    geo = dpc.conv_geometry(cin, H, Wd, k, s, pad, dil)
    T, d = dpc.conv_out_shape(geo)
    r = np.random.default_rng([2024, sorted(GEOMS).index(name), dtype == "bf16"])
    a = r.standard_normal((B, cin, H, Wd), dtype=np.float32)
    G = r.standard_normal((B, T, p), dtype=np.float32) * np.float32(0.1)
    if dtype == "bf16":
        a, G = W.f32_to_bf16_bits(a), W.f32_to_bf16_bits(G)
    a64, G64 = W.as_f64(a, dtype), W.as_f64(G, dtype)
    U = D.unfold2d(a64, k, s, pad, dil)
    assert U.shape == (B, T, d)
    return geo, (U, G64), (upload(a, dtype), upload(G, dtype))


def _expected_path(T, d, p, mode):
    path = D.choose_path(T, d, p, mode)
    return D.PATH_GHOST if path == D.PATH_T1 else path


@pytest.mark.parametrize("name", sorted(GEOMS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", [dpc.MODE_GHOST, dpc.MODE_EXPLICIT, dpc.MODE_MIXED, dpc.MODE_TIME])
def test_conv_norms(name, dtype, mode):
    geo, (U, Go), (a, G) = _case(name, dtype)
    B, T, d = U.shape
    p = Go.shape[2]
    for hb in (False, True):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        path = dpc.dp_conv_norm(a, G, geo, sq, has_bias=hb, mode=mode)
        assert path == _expected_path(T, d, p, mode)
        torch.cuda.synchronize()
        ref = D.layer_sqnorms(U, Go, has_bias=hb)
        assert_norms(sq.cpu().numpy(), ref, dtype, what=f"{name} hb={hb}")
        # accumulate adds the layer's squared norms to what sqnorm holds
        dpc.dp_conv_norm(a, G, geo, sq, has_bias=hb, mode=mode, accumulate=True)
        torch.cuda.synchronize()
        assert_norms(sq.cpu().numpy(), 2.0 * ref, dtype, what=f"{name} hb={hb} accumulated")


@pytest.mark.parametrize("name", sorted(GEOMS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_clipped_sum(name, dtype):
    geo, (U, Go), (a, G) = _case(name, dtype)
    B, T, d = U.shape
    p = Go.shape[2]
    c_np = W.make_vector(B, 0.05, 1.0, tag=11)
    c = f32(c_np)
    C, denom, seed, layer, step = 1.5, float(B), 9, 3, 2
    for hb in (False, True):
        S, Sb = D.clipped_sum(U, Go, c_np, has_bias=hb)
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
        dpc.dp_conv_clipped_sum_noise(a, G, geo, c, C, 0.0, denom, seed, layer, step, out, bias_out=bout)
        torch.cuda.synchronize()
        assert_sum(out.cpu().numpy() * denom, S, dtype, what=f"{name} sum")
        if hb:
            assert_sum(bout.cpu().numpy() * denom, Sb, dtype, what=f"{name} bias sum")
        sigma = 0.8
        dpc.dp_conv_clipped_sum_noise(a, G, geo, c, C, sigma, denom, seed, layer, step, out, bias_out=bout)
        torch.cuda.synchronize()
        z = N.weight_noise(d, p, seed, layer, step)
        assert_noised(out.cpu().numpy().ravel(), D.noised_mean(S, z, C, sigma, denom).ravel(), S,
                      (sigma * C * z / denom).ravel(), dtype, denom, what=f"{name} out")
        if hb:
            zb = N.normals(p, seed, layer, 1, step)
            assert_noised(bout.cpu().numpy(), D.noised_mean(Sb, zb, C, sigma, denom), Sb, sigma * C * zb / denom,
                          dtype, denom, what=f"{name} bias out")


def test_conv_workspace_reuse_and_errors():
    """Consecutive calls share one workspace (each call's partials overwrite the
    last call's); a short workspace and a mismatched geometry are refused."""
    geo, (U, Go), (a, G) = _case("stem-3x3", "f32")  # T = 1024: 36 Gram tiles per sample
    B = U.shape[0]
    need = dpc.dp_conv_workspace_bytes(geo, dpc.DP_F32, B, Go.shape[2], False, dpc.MODE_GHOST)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    ref = D.layer_sqnorms(U, Go)
    for _ in range(3):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_conv_norm(a, G, geo, sq, mode=dpc.MODE_GHOST, workspace=ws)
        torch.cuda.synchronize()
        assert_norms(sq.cpu().numpy(), ref, "f32")
    with pytest.raises(dpc.DpError) as e:
        dpc.dp_conv_norm(a, G, geo, sq, mode=dpc.MODE_GHOST, workspace=ws[:16])
    assert e.value.status == dpc.DP_ERR_WORKSPACE
    bad = dpc.conv_geometry(3, 32, 32, 3, 2, 1)  # stride 2: T = 256, G has 1024 rows per sample
    with pytest.raises(ValueError):
        dpc.dp_conv_norm(a, G, bad, sq)


@pytest.mark.parametrize("mode", [dpc.MODE_MIXED, dpc.MODE_TIME])
@pytest.mark.parametrize("l", range(8))
def test_resnet_full_size_layer(l, mode):
    """Every ResNet-18 conv layer of the benchmark at its size (B = 256) from
    the folded input, under the space and the time path rules (from 3
    channels at 32x32, T = 1024, to 512 channels at 4x4, T = 16; explicit and
    ghost paths). Norms of sampled examples and sampled entries of the
    clipped noised sum against the oracle on U(a), formed per sample."""
    wl = W.WORKLOADS["resnet18-conv-t1024"]
    fmap, Gn = W.make_folded(wl, l)
    cin, hin, win, stride = wl.conv[l]
    geo = dpc.conv_geometry(cin, hin, win, 3, stride, 1)
    B = fmap.shape[0]
    T, d = dpc.conv_out_shape(geo)
    p = Gn.shape[2]
    a, G = upload(fmap, "f32"), upload(Gn, "f32")
    sq = torch.empty(B, dtype=torch.float32, device=dev())
    path = dpc.dp_conv_norm(a, G, geo, sq, mode=mode)
    assert path == D.choose_path(T, d, p, mode)
    c_np = W.make_vector(B, 0.05, 1.0, tag=12)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    dpc.dp_conv_clipped_sum_noise(a, G, geo, f32(c_np), wl.C, wl.sigma, float(B), wl.seed, l, 0, out)
    torch.cuda.synchronize()
    idx = np.array([0, 1, 77, 128, 255])
    Ui = D.unfold2d(fmap[idx].astype(np.float64), (3, 3), (stride, stride), (1, 1))
    assert_norms(sq.cpu().numpy()[idx], D.layer_sqnorms(Ui, Gn[idx].astype(np.float64)), "f32")
    rng = np.random.default_rng(13)
    rows, cols = rng.integers(0, d, 48), rng.integers(0, p, 48)
    S_or = np.zeros(rows.shape[0])
    for i0 in range(0, B, 32):  # the sum over samples, 32 unfolded samples at a time
        Uc = D.unfold2d(fmap[i0:i0 + 32].astype(np.float64), (3, 3), (stride, stride), (1, 1))
        S_or += D.clipped_sum_entries(Uc, Gn[i0:i0 + 32].astype(np.float64), c_np[i0:i0 + 32], rows, cols)
    z = N.weight_noise_at(rows, cols, p, wl.seed, l, 0)
    assert_noised(out.cpu().numpy()[rows, cols], D.noised_mean(S_or, z, wl.C, wl.sigma, B), S_or,
                  wl.sigma * wl.C * z / B, "f32", B)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_folded_input_at_an_element_offset(dtype):
    """The folded input needs element alignment only: the same values starting
    one element into a buffer (4- or 2-byte aligned, not 16) give the same
    norms and sums bit for bit as the aligned copy."""
    geo, (U, Go), (a, G) = _case("rect-dil", dtype)
    B = U.shape[0]
    d, p = U.shape[2], Go.shape[2]
    buf = torch.empty(a.numel() + 1, dtype=a.dtype, device=dev())
    a_off = buf[1:].view(a.shape)
    a_off.copy_(a)
    assert a_off.data_ptr() % 16 != 0
    c = f32(W.make_vector(B, 0.05, 1.0, tag=14))
    res = []
    for x in (a, a_off):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        bout = torch.empty(p, dtype=torch.float32, device=dev())
        dpc.dp_conv_norm(x, G, geo, sq, has_bias=True, mode=dpc.MODE_GHOST)
        dpc.dp_conv_clipped_sum_noise(x, G, geo, c, 1.0, 0.5, float(B), 3, 1, 0, out, bias_out=bout)
        torch.cuda.synchronize()
        res.append((sq.cpu().numpy(), out.cpu().numpy(), bout.cpu().numpy()))
    for r0, r1 in zip(res[0], res[1]):
        np.testing.assert_array_equal(r0.view(np.uint32), r1.view(np.uint32))
    assert_norms(res[0][0], D.layer_sqnorms(U, Go, has_bias=True), dtype)


def test_conv_calls_deterministic_and_on_a_given_stream():
    """Repeated calls give the same bits; a call on a side stream (stream=)
    gives the bits of the call on the current stream."""
    geo, (U, Go), (a, G) = _case("mid-3x3", "bf16")
    B, d, p = U.shape[0], U.shape[2], Go.shape[2]
    c = f32(W.make_vector(B, 0.05, 1.0, tag=15))
    side = torch.cuda.Stream(device=dev())

    def run(stream):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        dpc.dp_conv_norm(a, G, geo, sq, mode=dpc.MODE_MIXED, stream=stream)
        dpc.dp_conv_clipped_sum_noise(a, G, geo, c, 1.0, 1.0, float(B), 5, 2, 9, out, stream=stream)
        torch.cuda.synchronize()
        return sq.cpu().numpy().view(np.uint32), out.cpu().numpy().view(np.uint32)

    torch.cuda.synchronize()  # inputs are ready before the side stream reads them
    r0, r1, r2 = run(None), run(None), run(side)
    for x, y, z in zip(r0, r1, r2):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(x, z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", sorted(GEOMS))
def test_unfold2d_bit_exact(name, dtype):
    """dp_unfold2d writes U(a) itself: bit for bit the oracle's fp64 unfolding
    (every element a copy of an input element or 0) and torch's
    unfold(a).transpose(1, 2); the unfolded calls on it give dp_conv_norm's
    norms within the norm tolerance."""
    geo, (U64, G64), (a, G) = _case(name, dtype)
    U = dpc.dp_unfold2d(a, geo)
    torch.cuda.synchronize()
    want = U64.astype(np.float32)
    if dtype == "bf16":
        want = W.f32_to_bf16_bits(want).view(np.uint16)
        got = U.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = U.cpu().numpy().view(np.uint32)
        want = want.view(np.uint32)
    np.testing.assert_array_equal(got.reshape(want.shape), want)
    B, cin, H, Wd, k, s, pad, dil, p = GEOMS[name]
    ref = torch.nn.functional.unfold(a.float(), k, dilation=dil, padding=pad, stride=s).transpose(1, 2)
    assert torch.equal(U.float(), ref)
    sq = torch.empty(B, dtype=torch.float32, device=dev())
    dpc.dp_ghost_norm(U, G, sq)
    torch.cuda.synchronize()
    assert_norms(sq.cpu().numpy(), D.layer_sqnorms(U64, G64), dtype, what=f"{name} unfolded")


def test_unfold2d_resnet_layers_and_errors():
    """The ResNet-18 layers of the benchmark at B = 256 (strides 1 and 2):
    dp_unfold2d against torch's unfold, bit for bit; and the binding's checks."""
    wl = W.WORKLOADS["resnet18-conv-t1024"]
    for l, (cin, h, w, st) in enumerate(wl.conv):
        fm, _ = W.make_folded(wl, l, step=0)
        a = torch.from_numpy(fm).to(dev())
        geo = dpc.conv_geometry(cin, h, w, 3, st, 1)
        U = dpc.dp_unfold2d(a, geo)
        ref = torch.nn.functional.unfold(a, 3, padding=1, stride=st).transpose(1, 2)
        torch.cuda.synchronize()
        assert torch.equal(U.view(torch.int32), ref.contiguous().view(torch.int32)), f"layer {l}"
        del a, U, ref
    a = torch.zeros(2, 3, 8, 8, device=dev())
    geo = dpc.conv_geometry(3, 8, 8, 3, 1, 1)
    with pytest.raises(ValueError):
        dpc.dp_unfold2d(a, geo, out=torch.empty(2, 64, 26, device=dev()))
    with pytest.raises(ValueError):
        dpc.dp_unfold2d(a[:, :2].contiguous(), geo)
