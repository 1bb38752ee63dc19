"""Virtual step on the GPU: a logical batch fed as physical batches
(dp_clipped_sum_accumulate per physical batch, dp_noise_mean once) against
the oracle's virtual step, the noise bit for bit, and one physical batch
against dp_clipped_sum_noise bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import definitions as D
from oracle import drivers
from oracle import noise as N

from gpu_util import assert_noised, dev, f32, upload

pytestmark = pytest.mark.gpu

CASES = {
    # name: (dtype, physical batch sizes, T, d, p, has_bias)
    "bf16-direct-engine": ("bf16", (5, 3, 8), 64, 128, 192, False),
    "f32-bias": ("f32", (4, 7), 20, 40, 24, True),
    "bf16-ragged": ("bf16", (2, 9, 1), 37, 24, 40, False),
}


def _batches(dtype, sizes, T, d, p, seed):
    rng = np.random.default_rng(seed)
    host, devs = [], []
    for B in sizes:
        A = (rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32)
        G = (rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32)
        if dtype == "bf16":
            A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
        host.append((W.as_f64(A, dtype), W.as_f64(G, dtype)))
        devs.append((upload(A, dtype), upload(G, dtype)))
    return host, devs


def _gpu_virtual(devs, cs, d, p, has_bias, C, sigma, seed, layer, step):
    acc = torch.full((d, p), float("nan"), dtype=torch.float32, device=dev())
    bacc = torch.full((p,), float("nan"), dtype=torch.float32, device=dev()) if has_bias else None
    for k, ((A, G), c) in enumerate(zip(devs, cs)):
        dpc.dp_clipped_sum_accumulate(A, G, f32(c), acc, bias_acc=bacc, accumulate=k > 0)
    n = sum(A.shape[0] for (A, _) in devs)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if has_bias else None
    dpc.dp_noise_mean(acc, C, sigma, float(n), seed, layer, step, out, bias_acc=bacc, bias_out=bout)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (bout.cpu().numpy() if has_bias else None), float(n)


@pytest.mark.parametrize("name", list(CASES))
def test_virtual_step_against_oracle(name):
    dtype, sizes, T, d, p, hb = CASES[name]
    host, devs = _batches(dtype, sizes, T, d, p, seed=len(name))
    rng = np.random.default_rng(2)
    cs = [rng.uniform(0.0, 1.0, B).astype(np.float32) for B in sizes]
    cs[0][0] = 0.0
    out, bout, n = _gpu_virtual(devs, cs, d, p, hb, 1.0, 0.0, 7, 3, 5)
    r = drivers.virtual_step(host, [c.astype(np.float64) for c in cs], 1.0, 0.0, 7, 3, 5, has_bias=hb)
    assert r["denom"] == n
    assert_noised(out, r["out"], r["sum"], np.zeros((d, p)), dtype, n)
    if hb:
        assert_noised(bout, r["bias_out"], r["bias_sum"], np.zeros(p), dtype, n, what="bias")
    # the noise alone (c = 0 everywhere), bit for bit against the oracle's fp32 replica
    zs = [np.zeros(B, dtype=np.float32) for B in sizes]
    out, bout, n = _gpu_virtual(devs, zs, d, p, hb, 1.3, 0.9, 11, 2, 6)
    zw = N.weight_noise(d, p, 11, 2, 6)
    np.testing.assert_array_equal(out, D.noised_mean_f32(np.zeros((d, p)), zw, 1.3, 0.9, n))
    if hb:
        zb = N.normals(p, 11, 2, 1, 6)
        np.testing.assert_array_equal(bout, D.noised_mean_f32(np.zeros(p), zb, 1.3, 0.9, n))


@pytest.mark.parametrize("name", list(CASES))
def test_one_physical_batch_equals_clipped_sum_noise_bitwise(name):
    """A virtual step of one physical batch is the plain step: the same sum
    (sigma = 0 makes the first call's epilogue exact), then the same noise
    operations on it."""
    dtype, sizes, T, d, p, hb = CASES[name]
    _, devs = _batches(dtype, sizes[-1:], T, d, p, seed=3)
    A, G = devs[0]
    B = A.shape[0]
    c = np.linspace(0.2, 1.0, B).astype(np.float32)
    out_v, bout_v, _ = _gpu_virtual(devs, [c], d, p, hb, 0.7, 1.1, 13, 4, 9)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
    dpc.dp_clipped_sum_noise(A, G, f32(c), 0.7, 1.1, float(B), 13, 4, 9, out, bout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_v.view(np.uint32), out.cpu().numpy().view(np.uint32))
    if hb:
        np.testing.assert_array_equal(bout_v.view(np.uint32), bout.cpu().numpy().view(np.uint32))


def test_noise_mean_in_place():
    d, p = 13, 7
    acc_np = np.random.default_rng(4).standard_normal((d, p)).astype(np.float32)
    bacc_np = np.arange(p, dtype=np.float32)
    acc, bacc = f32(acc_np).reshape(d, p), f32(bacc_np)
    ref = torch.empty(d, p, dtype=torch.float32, device=dev())
    bref = torch.empty(p, dtype=torch.float32, device=dev())
    dpc.dp_noise_mean(acc, 1.0, 0.5, 3.0, 1, 0, 2, ref, bias_acc=bacc, bias_out=bref)
    dpc.dp_noise_mean(acc, 1.0, 0.5, 3.0, 1, 0, 2, acc, bias_acc=bacc, bias_out=bacc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), ref.cpu().numpy())
    np.testing.assert_array_equal(bacc.cpu().numpy(), bref.cpu().numpy())
    zw = N.weight_noise(d, p, 1, 0, 2)
    np.testing.assert_array_equal(ref.cpu().numpy(), D.noised_mean_f32(acc_np, zw, 1.0, 0.5, 3.0))


def test_virtual_step_multi_layer():
    """Several layers per physical batch (dp_clipped_sum_accumulate_layers,
    bf16 layers sharing launches and one with a bias on another engine)
    against the oracle's virtual step per layer; the first batch alone is
    bit for bit the multi-layer clipped sum at sigma = 0, denom = 1."""
    specs = [(64, 128, 192), (64, 96, 64), (128, 64, 136), (20, 40, 24)]
    flags = [False, False, False, True]
    sizes = (4, 6, 3)
    rng = np.random.default_rng(12)
    host = [[] for _ in specs]
    devs = []
    for B in sizes:
        batch = []
        for l, (T, d, p) in enumerate(specs):
            A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32))
            G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32))
            host[l].append((W.as_f64(A, "bf16"), W.as_f64(G, "bf16")))
            batch.append((upload(A, "bf16"), upload(G, "bf16")))
        devs.append(batch)
    cs = [rng.uniform(0.0, 1.0, B).astype(np.float32) for B in sizes]
    accs = [torch.full((d, p), float("nan"), dtype=torch.float32, device=dev()) for (T, d, p) in specs]
    baccs = [torch.full((p,), float("nan"), dtype=torch.float32, device=dev()) if hb else None
             for (T, d, p), hb in zip(specs, flags)]
    for k, batch in enumerate(devs):
        dpc.dp_clipped_sum_accumulate_layers(batch, f32(cs[k]), accs, bias_accs=baccs, has_bias=flags,
                                             accumulate=k > 0)
        if k == 0:
            torch.cuda.synchronize()
            first = [a.cpu().numpy().copy() for a in accs]
            outs = [torch.empty_like(a) for a in accs]
            bouts = [torch.empty_like(b) if b is not None else None for b in baccs]
            dpc.dp_clipped_sum_noise_layers(batch, f32(cs[0]), 1.0, 0.0, 1.0, 0, 0, outs, bias_outs=bouts,
                                            has_bias=flags)
            torch.cuda.synchronize()
            for x, y in zip(first, outs):
                np.testing.assert_array_equal(x.view(np.uint32), y.cpu().numpy().view(np.uint32))
    n = float(sum(sizes))
    for l, ((T, d, p), hb) in enumerate(zip(specs, flags)):
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
        dpc.dp_noise_mean(accs[l], 1.0, 0.0, n, 3, l, 1, out, bias_acc=baccs[l], bias_out=bout)
        torch.cuda.synchronize()
        r = drivers.virtual_step(host[l], [c.astype(np.float64) for c in cs], 1.0, 0.0, 3, l, 1, has_bias=hb)
        assert_noised(out.cpu().numpy(), r["out"], r["sum"], np.zeros((d, p)), "bf16", n, what=f"layer {l}")
        if hb:
            assert_noised(bout.cpu().numpy(), r["bias_out"], r["bias_sum"], np.zeros(p), "bf16", n, what="bias")


def test_virtual_step_gpt_block_accumulates_bit_for_bit():
    """The transformer-block layers at B = 64, T = 128 (one shared bf16
    launch whose split partials are added to the accumulators by the reduce
    kernel itself): after each physical batch the accumulators equal, bit for
    bit, the previous accumulators plus that batch's multi-layer clipped sum at
    sigma = 0, denom = 1, added in fp32."""
    wl = W.WORKLOADS["gpt-block-t128"]
    B = wl.B
    rng = np.random.default_rng(21)
    batches = []
    for k in range(3):
        batch = []
        for (T, d, p) in wl.layers:
            A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32))
            G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32))
            batch.append((upload(A, "bf16"), upload(G, "bf16")))
        batches.append(batch)
    cs = [rng.uniform(0.0, 1.0, B).astype(np.float32) for _ in batches]
    accs = [torch.full((d, p), float("nan"), dtype=torch.float32, device=dev()) for (T, d, p) in wl.layers]
    sums = [torch.empty_like(a) for a in accs]
    prev = None
    for k, batch in enumerate(batches):
        dpc.dp_clipped_sum_accumulate_layers(batch, f32(cs[k]), accs, accumulate=k > 0)
        dpc.dp_clipped_sum_noise_layers(batch, f32(cs[k]), 1.0, 0.0, 1.0, 0, 0, sums)
        torch.cuda.synchronize()
        got = [a.cpu().numpy() for a in accs]
        s = [x.cpu().numpy() for x in sums]
        want = s if prev is None else [np.add(a, b, dtype=np.float32) for a, b in zip(prev, s)]
        for l, (x, y) in enumerate(zip(got, want)):
            assert np.isfinite(x).all(), f"batch {k} layer {l}"
            np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32), err_msg=f"batch {k} layer {l}")
        prev = got
