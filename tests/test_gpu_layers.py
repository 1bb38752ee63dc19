"""Multi-layer calls (dp_ghost_norm_layers, dp_clipped_sum_noise_layers) on the GPU.

The norm call must give, bit for bit, what per-layer dp_ghost_norm calls with
accumulate give (same fold order: each layer's tile partials in tile order,
then the layers in call order), whether its layers share one launch or not;
and the sum over layers must match the oracle's within the norm tolerance.
The clipped-sum call must match the oracle per layer within the sum
tolerance (its K splits may differ from a single-layer call's) and give the
noise bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import definitions as D

from gpu_util import assert_norms, dev, upload

pytestmark = pytest.mark.gpu


def _inputs(B, specs, dtype, seed):
    """specs: (T, d, p) per layer; seeded normal inputs scaled like the workloads."""
    rng = np.random.default_rng(seed)
    host, devs = [], []
    for (T, d, p) in specs:
        A = (rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32)
        G = (rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32)
        if dtype == "bf16":
            A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
        host.append((W.as_f64(A, dtype), W.as_f64(G, dtype)))
        devs.append((upload(A, dtype), upload(G, dtype)))
    return host, devs


def _sequential(devs, flags, mode, start=None):
    B = devs[0][0].shape[0]
    sq = start.clone() if start is not None else torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
    paths = []
    for l, ((A, G), hb) in enumerate(zip(devs, flags)):
        paths.append(dpc.dp_ghost_norm(A, G, sq, has_bias=hb, mode=mode, accumulate=(l > 0 or start is not None)))
    torch.cuda.synchronize()
    return sq.cpu().numpy(), paths


def _grouped(devs, flags, mode, start=None):
    B = devs[0][0].shape[0]
    sq = start.clone() if start is not None else torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
    paths = dpc.dp_ghost_norm_layers(devs, sq, has_bias=flags, mode=mode, accumulate=start is not None)
    torch.cuda.synchronize()
    return sq.cpu().numpy(), paths


def _oracle(host, flags, start=None):
    tot = np.zeros(host[0][0].shape[0]) if start is None else np.asarray(start, dtype=np.float64)
    for (A, G), hb in zip(host, flags):
        tot = tot + D.layer_sqnorms(A, G, hb)
    return tot


GPT_BLOCK = [(128, 768, 2304), (128, 768, 768), (128, 768, 3072), (128, 3072, 768)]

CASES = {
    # name: (B, specs, dtype, has_bias flags, mode)
    "gpt-block": (64, GPT_BLOCK, "bf16", [False] * 4, dpc.MODE_MIXED),
    "ragged-bias-f32": (13, [(100, 96, 80), (128, 64, 200), (37, 72, 72), (64, 128, 64)], "f32",
                        [True, False, True, True], dpc.MODE_GHOST),
    "mixed-paths": (9, [(1, 64, 32), (96, 128, 128), (200, 16, 24), (96, 200, 64), (600, 64, 96), (80, 64, 128)],
                    "bf16", [False, True, False, True, False, True], dpc.MODE_MIXED),
    "ten-layers": (11, [(128, 64 + 8 * k, 128) for k in range(10)], "bf16", [k % 2 == 0 for k in range(10)],
                   dpc.MODE_GHOST),
    "wide-engine-inside": (3, [(128, 96, 128), (512, 128, 192), (64, 64, 128)], "bf16", [False, False, True],
                           dpc.MODE_GHOST),
    # consecutive long-sequence layers share one launch of that engine
    "wide-group": (3, [(512, 128, 192), (576, 64, 128), (1024, 128, 64), (512, 192, 64)], "bf16",
                   [False, True, False, True], dpc.MODE_GHOST),
    # short and long samples in one launch of that engine (128 x 128 tiles beside 256 x 128)
    "wide-short-long": (5, [(128, 128, 192), (100, 64, 64), (512, 64, 128), (65, 128, 64)], "bf16",
                        [True, False, False, True], dpc.MODE_GHOST),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layers_match_sequential_and_oracle(name):
    B, specs, dtype, flags, mode = CASES[name]
    host, devs = _inputs(B, specs, dtype, seed=len(name))
    seq, p_seq = _sequential(devs, flags, mode)
    grp, p_grp = _grouped(devs, flags, mode)
    assert p_grp == p_seq
    np.testing.assert_array_equal(grp.view(np.uint32), seq.view(np.uint32))
    assert_norms(np.sqrt(grp), np.sqrt(_oracle(host, flags)), dtype)


def test_layers_accumulate_onto_existing_values():
    B, specs, dtype, flags, mode = CASES["ragged-bias-f32"]
    host, devs = _inputs(B, specs, dtype, seed=5)
    start_np = np.linspace(0.5, 3.0, B).astype(np.float32)
    start = torch.from_numpy(start_np).to(dev())
    seq, _ = _sequential(devs, flags, mode, start=start)
    grp, _ = _grouped(devs, flags, mode, start=start)
    np.testing.assert_array_equal(grp.view(np.uint32), seq.view(np.uint32))
    assert_norms(np.sqrt(grp), np.sqrt(_oracle(host, flags, start_np)), dtype)


def test_layers_zero_and_nan_samples():
    """A sample whose inputs are all zero has norm 0; a NaN in one layer of
    one sample makes only that sample's norm NaN."""
    B, specs, dtype, flags, mode = CASES["gpt-block"]
    B = 16
    rng = np.random.default_rng(9)
    devs = []
    for k, (T, d, p) in enumerate(specs):
        A = (rng.standard_normal((B, T, d)) / np.sqrt(d)).astype(np.float32)
        G = (rng.standard_normal((B, T, p)) / np.sqrt(p)).astype(np.float32)
        A[3] = 0.0
        G[3] = 0.0
        if k == 2:
            G[7, 5, 11] = np.nan
        devs.append((upload(W.f32_to_bf16_bits(A), "bf16"), upload(W.f32_to_bf16_bits(G), "bf16")))
    grp, _ = _grouped(devs, flags, mode)
    seq, _ = _sequential(devs, flags, mode)
    np.testing.assert_array_equal(grp.view(np.uint32), seq.view(np.uint32))
    assert grp[3] == 0.0
    assert np.isnan(grp[7])
    assert np.isfinite(np.delete(grp, 7)).all()


def test_layers_repeated_calls_share_a_workspace():
    """Calls of different layer lists on one workspace (partials of other
    shapes left in it) give the same results as fresh ones."""
    B = 12
    lists = [CASES["ten-layers"][1][:5], GPT_BLOCK[:2], [(100, 96, 80), (37, 72, 72)]]
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev())
    ws.fill_(0x3F)  # float-like bytes
    for rep in range(2):
        for k, specs in enumerate(lists):
            _, devs = _inputs(B, specs, "bf16", seed=100 + k)
            flags = [False] * len(specs)
            sq = torch.empty(B, dtype=torch.float32, device=dev())
            dpc.dp_ghost_norm_layers(devs, sq, has_bias=flags, mode=dpc.MODE_GHOST, workspace=ws)
            torch.cuda.synchronize()
            ref, _ = _sequential(devs, flags, dpc.MODE_GHOST)
            np.testing.assert_array_equal(sq.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- clipped sums of several layers
from oracle import noise as N  # noqa: E402

from gpu_util import assert_noised, f32  # noqa: E402


def _sum_layers(devs, c_np, C, sigma, denom, seed, step, flags=None, layer_ids=None, workspace=None):
    B = devs[0][0].shape[0]
    flags = [False] * len(devs) if flags is None else flags
    outs = [torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev()) for (A, G) in devs]
    bouts = [torch.empty(G.shape[2], dtype=torch.float32, device=dev()) if hb else None
             for (A, G), hb in zip(devs, flags)]
    dpc.dp_clipped_sum_noise_layers(devs, f32(c_np), C, sigma, denom, seed, step, outs,
                                    bias_outs=bouts if any(flags) else None, has_bias=flags,
                                    layer_ids=layer_ids, workspace=workspace)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs], [None if b is None else b.cpu().numpy() for b in bouts]


def test_sum_layers_gpt_block_full_size():
    """The four layers of a GPT block at full size (B = 64, T = 128) in one
    call: sampled entries of every layer's clipped sum against the oracle,
    and the noise, at c = 0, bit for bit over every entry."""
    B, specs, dtype, _, _ = CASES["gpt-block"]
    host, devs = _inputs(B, specs, dtype, seed=21)
    rng = np.random.default_rng(4)
    c_np = rng.uniform(0.0, 1.0, B).astype(np.float32)
    c_np[[0, 17, 40]] = 0.0
    c_np[5] = 1.0
    C, denom, seed, step = 0.8, float(B), 12345, 3
    outs, _ = _sum_layers(devs, c_np, C, 0.0, denom, seed, step)
    for l, ((Ao, Go), out) in enumerate(zip(host, outs)):
        d, p = out.shape
        rows, cols = rng.integers(0, d, 128), rng.integers(0, p, 128)
        S_or = D.clipped_sum_entries(Ao, Go, c_np.astype(np.float64), rows, cols)
        assert_noised(out[rows, cols], S_or / denom, S_or, np.zeros(rows.size), dtype, denom, what=f"layer {l}")
    zeros = np.zeros(B, dtype=np.float32)
    outs, _ = _sum_layers(devs, zeros, C, 1.3, denom, seed, step, layer_ids=[7, 8, 9, 10])
    for l, out in enumerate(outs):
        d, p = out.shape
        zw = N.weight_noise(d, p, seed, 7 + l, step)
        np.testing.assert_array_equal(out, D.noised_mean_f32(np.zeros((d, p)), zw, C, 1.3, denom))


SUM_CASES = {
    # name: (B, specs, flags)
    "mixed-engines": (6, [(128, 64, 96), (100, 40, 24), (64, 128, 64), (128, 96, 32), (192, 136, 200)],
                      [False, False, False, True, False]),
    "ten-layers": (5, [(64, 64 + 8 * k, 128 - 8 * k) for k in range(10)], [False] * 10),
    # launches of 8 and 1: the last eligible layer takes the single-layer path
    "nine-layers": (4, [(128, 64 + 16 * k, 64) for k in range(9)], [False] * 9),
    "one-eligible": (7, [(100, 40, 24), (128, 136, 64)], [False, False]),
}


@pytest.mark.parametrize("name", list(SUM_CASES))
def test_sum_layers_against_oracle_and_single_calls(name):
    """Every layer of a mixed list (grouped engine, other engines, a bias)
    against the oracle's full clipped noised mean, and against the
    single-layer call within the same tolerance."""
    B, specs, flags = SUM_CASES[name]
    host, devs = _inputs(B, specs, "bf16", seed=33 + len(name))
    c_np = np.linspace(0.05, 1.0, B).astype(np.float32)
    c_np[1] = 0.0
    C, sigma, denom, seed, step = 1.1, 0.0, 2.0 * B, 99, 6
    outs, bouts = _sum_layers(devs, c_np, C, sigma, denom, seed, step, flags=flags)
    for l, ((Ao, Go), (A, G), hb) in enumerate(zip(host, devs, flags)):
        S_or, Sb = D.clipped_sum(Ao, Go, c_np.astype(np.float64), has_bias=hb)
        assert_noised(outs[l], S_or / denom, S_or, np.zeros_like(S_or), "bf16", denom, what=f"layer {l}")
        if hb:
            assert_noised(bouts[l], Sb / denom, Sb, np.zeros_like(Sb), "bf16", denom, what=f"bias {l}")
        one = torch.empty(A.shape[2], G.shape[2], dtype=torch.float32, device=dev())
        bone = torch.empty(G.shape[2], dtype=torch.float32, device=dev()) if hb else None
        dpc.dp_clipped_sum_noise(A, G, f32(c_np), C, sigma, denom, seed, l, step, one, bone)
        torch.cuda.synchronize()
        assert_noised(outs[l], one.cpu().numpy(), S_or, np.zeros_like(S_or), "bf16", denom, what=f"single {l}")


def test_sum_layers_repeatable_bitwise():
    """Two calls with the same inputs give the same bits, also when the
    workspace holds another call's partials in between."""
    B, specs, _ = SUM_CASES["ten-layers"]
    _, devs = _inputs(B, specs, "bf16", seed=8)
    c_np = np.linspace(0.1, 0.9, B).astype(np.float32)
    ws = torch.empty(dpc.dp_layers_workspace_bytes(devs) + 256, dtype=torch.uint8, device=dev())
    a, _ = _sum_layers(devs, c_np, 1.0, 0.5, float(B), 5, 1, workspace=ws)
    _, other = _inputs(B, specs[:3], "bf16", seed=9)
    _sum_layers(other, c_np, 1.0, 0.5, float(B), 5, 1, workspace=ws)
    b, _ = _sum_layers(devs, c_np, 1.0, 0.5, float(B), 5, 1, workspace=ws)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_sum_layers_unaligned_outputs_bitwise():
    """Outputs (and accumulators) only 4-byte aligned take the scalar reduce
    for their layer while the others share the grouped one: every layer's
    result equals, bit for bit, that of the call with 16-byte aligned
    outputs, with noise and in the accumulating form."""
    B, specs, dtype, _, _ = CASES["gpt-block"]
    _, devs = _inputs(B, specs, dtype, seed=41)
    c_np = np.random.default_rng(6).uniform(0.0, 1.0, B).astype(np.float32)
    want, _ = _sum_layers(devs, c_np, 0.9, 1.2, float(B), 77, 2)
    # layers 1 and 3 written at a 4-byte offset into a larger buffer
    bufs = [torch.empty(A.shape[2] * G.shape[2] + 4, dtype=torch.float32, device=dev()) for (A, G) in devs]
    outs = [b[1:1 + A.shape[2] * G.shape[2]].view(A.shape[2], G.shape[2]) if l % 2 else
            b[:A.shape[2] * G.shape[2]].view(A.shape[2], G.shape[2]) for l, (b, (A, G)) in enumerate(zip(bufs, devs))]
    assert outs[1].data_ptr() % 16 == 4
    dpc.dp_clipped_sum_noise_layers(devs, f32(c_np), 0.9, 1.2, float(B), 77, 2, outs)
    torch.cuda.synchronize()
    for l, (x, y) in enumerate(zip(outs, want)):
        np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32), y.view(np.uint32), err_msg=f"layer {l}")
    # accumulating form: acc + sum at sigma = 0, denom = 1, against fp32 adds of the plain sums
    plain, _ = _sum_layers(devs, c_np, 1.0, 0.0, 1.0, 0, 0)
    start = [np.random.default_rng(50 + l).standard_normal(x.shape).astype(np.float32) for l, x in enumerate(plain)]
    for l, o in enumerate(outs):
        o.copy_(torch.from_numpy(start[l]))
    dpc.dp_clipped_sum_accumulate_layers(devs, f32(c_np), outs, accumulate=True)
    torch.cuda.synchronize()
    for l, (x, s0, s) in enumerate(zip(outs, start, plain)):
        np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32), np.add(s0, s, dtype=np.float32).view(np.uint32),
                                      err_msg=f"accumulated layer {l}")


def test_time_rule_on_conv_layers():
    """The time rule (DP_MODE_TIME) on the conv layer set (B = 5): the paths
    the oracle's rule picks (explicit on the four early layers), and the norm
    summed over layers against the oracle's."""
    wl = W.WORKLOADS["resnet18-conv-t1024"]
    host, devs = [], []
    for l in range(wl.n_layers):
        A, G = W.make_layer(wl, l, B=5)
        host.append((W.as_f64(A, wl.dtype), W.as_f64(G, wl.dtype)))
        devs.append((upload(A, wl.dtype), upload(G, wl.dtype)))
    flags = [False] * wl.n_layers
    grp, paths = _grouped(devs, flags, dpc.MODE_TIME)
    want = [D.choose_path(*wl.layer_shape(l), D.MODE_TIME) for l in range(wl.n_layers)]
    assert paths == want
    assert paths[:4] == [dpc.PATH_EXPLICIT] * 4 and paths[4:] == [dpc.PATH_GHOST] * 4
    seq, _ = _sequential(devs, flags, dpc.MODE_TIME)
    np.testing.assert_array_equal(grp.view(np.uint32), seq.view(np.uint32))
    assert_norms(np.sqrt(grp), np.sqrt(_oracle(host, flags)), wl.dtype)


FUSED_CLIP_CASES = ["gpt-block", "ragged-bias-f32", "mixed-paths", "ten-layers", "wide-engine-inside", "wide-group"]


@pytest.mark.parametrize("name", FUSED_CLIP_CASES)
def test_norm_clip_layers_equal_separate_clip(name):
    """Clip factors formed in the norm kernels' sinks (dp_ghost_norm_clip_layers)
    equal dp_clip_factors applied after dp_ghost_norm_layers, bit for bit,
    whatever path the last layer takes; so do the squared norms."""
    B, specs, dtype, flags, mode = CASES[name]
    host, devs = _inputs(B, specs, dtype, seed=40 + len(name))
    sq_ref, _ = _grouped(devs, flags, mode)
    sq_ref_t = torch.from_numpy(sq_ref).to(dev())
    norms = np.sqrt(_oracle(host, flags))
    for C in (float(np.median(norms)), 1e-3, 1e9):
        c_ref = torch.empty(B, dtype=torch.float32, device=dev())
        n_ref = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_clip_factors(sq_ref_t, C, c_ref, n_ref)
        sq = torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
        c = torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
        n = torch.full((B,), float("nan"), dtype=torch.float32, device=dev())
        dpc.dp_ghost_norm_clip_layers(devs, sq, C, c, n, has_bias=flags, mode=mode)
        torch.cuda.synchronize()
        for got, want in ((sq, sq_ref_t), (c, c_ref), (n, n_ref)):
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("last", [dpc.PATH_T1, dpc.PATH_EXPLICIT])
def test_norm_clip_layers_last_layer_path(last):
    """A last layer with T = 1 has no per-sample sink: its call is followed
    by the clip kernel; an explicit last layer forms the factors in its own
    sink. Either way the factors are the same bits."""
    B = 7
    specs = [(96, 128, 128), (1, 64, 32) if last == dpc.PATH_T1 else (200, 16, 24)]
    _, devs = _inputs(B, specs, "bf16", seed=77)
    flags = [False, True]
    sq_ref, paths = _grouped(devs, flags, dpc.MODE_MIXED)
    assert paths[-1] == last
    c_ref = torch.empty(B, dtype=torch.float32, device=dev())
    dpc.dp_clip_factors(torch.from_numpy(sq_ref).to(dev()), 0.5, c_ref)
    sq = torch.empty(B, dtype=torch.float32, device=dev())
    c = torch.empty(B, dtype=torch.float32, device=dev())
    dpc.dp_ghost_norm_clip_layers(devs, sq, 0.5, c, has_bias=flags)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint32), c_ref.cpu().numpy().view(np.uint32))
