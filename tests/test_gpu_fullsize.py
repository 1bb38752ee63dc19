"""Full-size parity of exactly the launches the benchmark runs, and call
patterns around them (graph replay, side streams).

The benchmark's step is two calls: dp_ghost_norm_clip_layers (every layer's
norm, the cross-layer sum and the clip factors) and
dp_clipped_sum_noise_layers (every layer's clipped noised mean under one c).
At gpt-block-t128 the four layers share one ghost launch and one contraction
launch (256 x 256 tiles with the per-sample rescale, K split, the split
tiles' partials added by one reduce launch); at gpt2large-t1024 eight
consecutive layers (two decoder blocks) share each launch, and each launch's
split reduce runs on the next launch's idle CUs. The oracle computes each layer's
per-example gradients in fp64 and everything from them ("Scalable and
Efficient Training of Large CNNs with DP", eq. (2.1) and Sec. 3.2; "Scaling up
DP Deep Learning with Fast Per-Example Gradient Clipping", clipped mean plus
Gaussian noise).
"""
import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import definitions as D
from oracle import drivers
from oracle import noise as N

from gpu_util import assert_clip, assert_noised, assert_norms, dev, f32, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    dpc.lib()


def _benched_step(devs, wl, step, workspace=None, stream=None):
    """The benchmark's two calls on a layer set; returns device tensors."""
    B = devs[0][0].shape[0]
    sq = torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
    c = torch.empty(B, dtype=torch.float32, device=dev())
    nrm = torch.empty(B, dtype=torch.float32, device=dev())
    paths = dpc.dp_ghost_norm_clip_layers(devs, sq, wl.C, c, nrm, workspace=workspace, stream=stream)
    outs = [torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev()) for (A, G) in devs]
    dpc.dp_clipped_sum_noise_layers(devs, c, wl.C, wl.sigma, float(B), wl.seed, step, outs, workspace=workspace,
                                    stream=stream)
    return sq, c, nrm, outs, paths


def test_gpt_block_t128_benched_calls_every_entry():
    """gpt-block-t128 at full size (B = 64, T = 128, the four layers) through
    the benchmark's call pair: every norm, every clip factor and every entry
    of all four noised means against the oracle's global step."""
    wl = W.WORKLOADS["gpt-block-t128"]
    host, devs = [], []
    for l in range(wl.n_layers):
        A, G = W.make_layer(wl, l, step=0)
        host.append((W.as_f64(A, "bf16"), W.as_f64(G, "bf16")))
        devs.append((upload(A, "bf16"), upload(G, "bf16")))
    sq, c, nrm, outs, paths = _benched_step(devs, wl, step=0)
    torch.cuda.synchronize()
    assert paths == [dpc.PATH_GHOST] * 4
    ref = drivers.global_clip_step(host, wl.C, wl.sigma, wl.seed, step=0)
    assert_norms(nrm.cpu().numpy(), ref["norms"], "bf16")
    assert_norms(np.sqrt(sq.cpu().numpy().astype(np.float64)), ref["norms"], "bf16", what="sqrt(sqnorm)")
    assert_clip(c.cpu().numpy(), ref["c"], ref["norms"], wl.C, "bf16")
    for l, out in enumerate(outs):
        S = ref["sums"][l]
        noise = wl.sigma * wl.C * N.weight_noise(S.shape[0], S.shape[1], wl.seed, l, 0) / wl.B
        assert_noised(out.cpu().numpy(), ref["outs"][l], S, noise, "bf16", wl.B, what=f"out[{l}]")


def _device_layers(wl, layers, step):
    """Inputs drawn on the device (the benchmark's generator for this stack)
    and their exact values widened to fp64 for the oracle."""
    devs, host = [], []
    for l in layers:
        A, G = W.make_layer_device(wl, l, dev(), step=step)
        devs.append((A, G))
        host.append(tuple(x.float().cpu().numpy().astype(np.float64) for x in (A, G)))
    return devs, host


def test_gpt2large_block_pair_benched_launches():
    """Two GPT-2-large decoder blocks (8 layers, B = 32, T = 1024) through the
    benchmark's call pair: the eight layers share one long-sequence ghost
    launch and one contraction launch, as every pair of blocks does in the
    benchmark. Every norm and clip factor, and 4096 sampled entries of each
    layer's noised mean, against the oracle."""
    wl = W.WORKLOADS["gpt2large-t1024"]
    devs, host = _device_layers(wl, range(8), step=0)
    B = wl.B
    sq, c, nrm, outs, paths = _benched_step(devs, wl, step=4)
    torch.cuda.synchronize()
    assert paths == [dpc.PATH_GHOST] * 8
    sqs = [D.layer_sqnorms(A, G) for (A, G) in host]
    norms = D.total_norms(sqs)
    c_or = D.clip_factors(norms, wl.C)
    assert_norms(nrm.cpu().numpy(), norms, "bf16")
    assert_clip(c.cpu().numpy(), c_or, norms, wl.C, "bf16")
    c_gpu = c.cpu().numpy()
    rng = np.random.default_rng(2024)
    for l, ((A, G), out) in enumerate(zip(host, outs)):
        d, p = out.shape
        rows, cols = rng.integers(0, d, 4096), rng.integers(0, p, 4096)
        # the same clip factors on both sides: the sum is checked on its own bar
        S_or = D.clipped_sum_entries(A, G, c_gpu.astype(np.float64), rows, cols)
        z = N.weight_noise_at(rows, cols, p, wl.seed, l, 4)
        out_or = D.noised_mean(S_or, z, wl.C, wl.sigma, B)
        assert_noised(out.cpu().numpy()[rows, cols], out_or, S_or, wl.sigma * wl.C * z / B, "bf16", B,
                      what=f"out[{l}]")


@pytest.mark.parametrize("unaligned", [False, True])
def test_gpt2large_reduce_in_next_launch_bitwise(unaligned):
    """Six GPT-2-large decoder blocks (24 layers: three shared contraction
    launches) in one call, where each launch's split reduce runs on the idle
    CUs of the next launch and the last one's on its own: every layer's noised
    mean equals, bit for bit, that of one call per block pair (whose reduce
    runs on its own), with the same layer ids. With one output of the first
    launch only 4-byte aligned, that launch's reduce cannot go to the next
    launch (it runs on its own after it, the odd layer in the scalar reduce):
    the same bits."""
    wl = W.WORKLOADS["gpt2large-t1024"]
    layers = [W.make_layer_device(wl, l, dev()) for l in range(24)]
    B = wl.B
    gen = torch.Generator(device=dev()).manual_seed(3)
    c = torch.rand(B, device=dev(), generator=gen) * 0.8 + 0.2
    outs = [torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev()) for (A, G) in layers]
    if unaligned:
        d, p = outs[3].shape
        buf = torch.empty(d * p + 4, dtype=torch.float32, device=dev())
        outs[3] = buf[1:1 + d * p].view(d, p)
        assert outs[3].data_ptr() % 16 == 4
    dpc.dp_clipped_sum_noise_layers(layers, c, 1.0, 1.0, float(B), 7, 2, outs)
    for k in range(3):
        ids = list(range(8 * k, 8 * k + 8))
        ref = [torch.empty_like(outs[l]) for l in ids]
        dpc.dp_clipped_sum_noise_layers([layers[l] for l in ids], c, 1.0, 1.0, float(B), 7, 2, ref, layer_ids=ids)
        torch.cuda.synchronize()
        for l, r in zip(ids, ref):
            assert torch.equal(outs[l].view(torch.int32), r.view(torch.int32)), f"layer {l}"
    del layers


def test_wide_tile_extreme_clip_factors():
    """The 256 x 256 tile keeps its running sum divided by the current clip
    factor. Factors from 1 down to 2e-38 and a subnormal one, next to zeros,
    on samples whose inputs are scaled by powers of two so that c_i A_i^T G_i
    stays of order one (huge per-sample norms clipped to a bound C < 1): the
    GPT-2-large qkv layer (which takes that tile) against the oracle on
    sampled entries, and no non-finite output."""
    wl = W.WORKLOADS["gpt2large-t1024"]
    A_raw, G_raw = W.make_layer(wl, 0, step=7)
    B = wl.B
    c_np = np.random.default_rng(31).uniform(0.2, 1.0, B).astype(np.float32)
    tiny = {1: 2.0e-38, 2: 0.0, 3: 5.0e-39, 4: 1.0e-30, 6: 1.0e-20, 9: 3.0e-38, 10: 1.0, 13: 1.0e-36,
            20: 0.0, 21: 4.0e-38, 30: 1.0e-25, 31: 2.5e-38}
    for i, v in tiny.items():
        c_np[i] = np.float32(v)
    A64, G64 = W.as_f64(A_raw, "bf16"), W.as_f64(G_raw, "bf16")
    for i, v in tiny.items():
        if v > 0:
            k = int(np.floor(-np.log2(float(np.float32(v))) / 2))     # 2^(2k) ~ 1/c_i: exact in bf16
            A64[i] *= 2.0 ** k
            G64[i] *= 2.0 ** k
    A_bits = W.f32_to_bf16_bits(A64.astype(np.float32))
    G_bits = W.f32_to_bf16_bits(G64.astype(np.float32))
    assert np.array_equal(W.as_f64(A_bits, "bf16"), A64) and np.array_equal(W.as_f64(G_bits, "bf16"), G64)
    A, G = upload(A_bits, "bf16"), upload(G_bits, "bf16")
    d, p = A.shape[2], G.shape[2]
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    C, denom = 0.25, float(B)
    dpc.dp_clipped_sum_noise(A, G, f32(c_np), C, 0.0, denom, 5, 0, 0, out)
    # the multi-layer call with this layer twice shares a launch (and its plan)
    outs2 = [torch.empty_like(out), torch.empty_like(out)]
    dpc.dp_clipped_sum_noise_layers([(A, G), (A, G)], f32(c_np), C, 0.0, denom, 5, 0, outs2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows, cols = rng.integers(0, d, 512), rng.integers(0, p, 512)
    S_or = D.clipped_sum_entries(A64, G64, c_np.astype(np.float64), rows, cols)
    for what, o in (("single", out), ("layers[0]", outs2[0]), ("layers[1]", outs2[1])):
        got = o.cpu().numpy()
        assert np.isfinite(got).all(), what
        assert_noised(got[rows, cols], S_or / denom, S_or, np.zeros(rows.size), "bf16", denom, what=what)


def test_graph_capture_replays_match_eager_calls():
    """The benchmark's two calls captured in a HIP graph (torch.cuda.CUDAGraph)
    and replayed three times with new inputs copied in, eager work and
    synchronisations in between: every replay gives the eager calls' bits
    (norms, clip factors, noised means): a call's kernels read from the
    workspace only what the same call wrote there."""
    wl = W.WORKLOADS["gpt-block-t128"]
    B = 16
    specs = [(128, 256, 384), (128, 256, 256), (128, 384, 256)]
    rng = np.random.default_rng(3)

    def draw():
        out = []
        for (T, d, p) in specs:
            A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32))
            G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) * 4.0 / np.sqrt(p)).astype(np.float32))
            out.append((upload(A, "bf16"), upload(G, "bf16")))
        return out

    static = draw()
    ws = torch.empty(dpc.dp_layers_workspace_bytes(static) + 256, dtype=torch.uint8, device=dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm up on the capture stream
        _benched_step(static, wl, 0, workspace=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = _benched_step(static, wl, 0, workspace=ws, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        fresh = draw()
        for (A, G), (A2, G2) in zip(static, fresh):
            A.copy_(A2)
            G.copy_(G2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [cap[0].cpu(), cap[1].cpu(), cap[2].cpu()] + [o.cpu() for o in cap[3]]
        eager = _benched_step(fresh, wl, 0, workspace=ws)
        torch.cuda.synchronize()
        want = [eager[0].cpu(), eager[1].cpu(), eager[2].cpu()] + [o.cpu() for o in eager[3]]
        for k, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {rep}, output {k}"
        assert (want[1] < 1.0).any()


def test_graph_capture_of_a_multi_launch_sum_call():
    """A clipped-sum call of four GPT-2-large decoder blocks (two shared
    launches: the second runs the first one's split reduce in its tail, the
    last reduce runs on its own) captured in a HIP graph and replayed three
    times with new inputs copied in: every replay gives the eager call's bits."""
    wl = W.WORKLOADS["gpt2large-t1024"]
    B = wl.B
    static = [W.make_layer_device(wl, l, dev(), step=0) for l in range(16)]
    gen = torch.Generator(device=dev()).manual_seed(5)
    c = torch.rand(B, device=dev(), generator=gen) * 0.8 + 0.2
    ws = torch.empty(dpc.dp_layers_workspace_bytes(static) + 256, dtype=torch.uint8, device=dev())
    outs = [torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev()) for (A, G) in static]

    def call(layers, o, stream=None):
        dpc.dp_clipped_sum_noise_layers(layers, c, wl.C, wl.sigma, float(B), wl.seed, 3, o, workspace=ws,
                                        stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        call(static, outs, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(static, outs, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager_outs = [torch.empty_like(o) for o in outs]
    for rep in range(3):
        for l, (A, G) in enumerate(static):
            A2, G2 = W.make_layer_device(wl, l, dev(), step=rep + 1)
            A.copy_(A2)
            G.copy_(G2)
            del A2, G2
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        call(static, eager_outs)
        torch.cuda.synchronize()
        for l, (x, y) in enumerate(zip(got, eager_outs)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {rep}, layer {l}"
    del static


def test_side_stream_call_keeps_its_workspace():
    """A call on a side stream with a workspace the binding allocates, then an
    allocation on the current stream written with garbage right away: the
    side-stream call's results are the serial ones bit for bit (the binding
    keeps the block in use until the side stream has passed the call)."""
    wl = W.WORKLOADS["gpt-block-t128"]
    B = 32
    specs = [(128, 768, 2304), (128, 768, 768)]
    rng = np.random.default_rng(17)
    devs = []
    for (T, d, p) in specs:
        A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32))
        G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32))
        devs.append((upload(A, "bf16"), upload(G, "bf16")))
    c = f32(np.linspace(0.1, 1.0, B))
    need = dpc.dp_layers_workspace_bytes(devs)
    assert need > 0
    ref = [torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev()) for (A, G) in devs]
    dpc.dp_clipped_sum_noise_layers(devs, c, 1.0, 1.0, float(B), 9, 2, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = [torch.empty_like(r) for r in ref]
        # keep the side stream busy first so that the call's kernels start late
        with torch.cuda.stream(side):
            busy = torch.randn(4096, 4096, device=dev())
            for _ in range(8):
                busy = busy @ busy * 1e-3
        dpc.dp_clipped_sum_noise_layers(devs, c, 1.0, 1.0, float(B), 9, 2, got, stream=side)
        junk = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device=dev())
        junk.fill_(3.0e38)
        torch.cuda.synchronize()
        for x, y in zip(got, ref):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"rep {rep}"
        del junk, busy
