"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every case is seeded and synthetic (workloads.py). Reduced cases run the whole
path and compare every output; full-size cases use the launch configuration
of the benchmark and compare everything the oracle computes in seconds, else
sampled outputs.
"""
import math

import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import definitions as D
from oracle import drivers
from oracle import noise as N

from gpu_util import (TAU_NORM, TAU_SUM, assert_clip, assert_noised, assert_norms, assert_sum, dev, f32,
                      gpu_global_step, layer_inputs, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    dpc.lib()


def _check_global(wl, oracle_layers, res, has_bias=False, denom=None, seed=0, step=0):
    B = oracle_layers[0][0].shape[0]
    denom = float(B) if denom is None else denom
    ref = drivers.global_clip_step(oracle_layers, wl.C, wl.sigma, seed, step=step, has_bias=has_bias, denom=denom)
    assert_norms(res["norm"], ref["norms"], wl.dtype)
    assert_clip(res["c"], ref["c"], ref["norms"], wl.C, wl.dtype)
    for l in range(len(oracle_layers)):
        S = ref["sums"][l]
        noise = wl.sigma * wl.C * N.weight_noise(S.shape[0], S.shape[1], seed, l, step) / denom
        assert_noised(res["outs"][l], ref["outs"][l], S, noise, wl.dtype, denom, what=f"out[{l}]")
    for l, (A, G) in enumerate(oracle_layers):
        path = D.choose_path(A.shape[1], A.shape[2], G.shape[2])
        assert res["paths"][l] == path
    return ref


# ------------------------------------------------------------------ whole-path cases
def test_single_linear_t1_full():
    wl = W.WORKLOADS["single-linear-t1"]
    _, o, g = layer_inputs(wl, 0)
    res = gpu_global_step([g], False, wl.C, wl.sigma, wl.seed)
    ref = _check_global(wl, [o], res)
    assert np.all(ref["c"] < 1.0)  # every sample clips here (norms ~ 45 and ~ 4500 vs C = 1)


REDUCED = {
    # (workload, B, shapes): several tiles per dimension and ragged tails
    "gpt-block-t128": (5, [(128, 192, 200), (100, 72, 136), (128, 3072 // 16, 768 // 8), (37, 40, 24)]),
    "gpt2large-t1024": (3, [(300, 160, 480), (1024, 64, 72), (129, 136, 64)]),
    "resnet18-conv-t1024": (5, None),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_workload_reduced(name):
    wl = W.WORKLOADS[name]
    B, shapes = REDUCED[name]
    n_layers = len(shapes) if shapes else wl.n_layers
    ors, gps = [], []
    for l in range(n_layers):
        _, o, g = layer_inputs(wl, l, B=B, shape=shapes[l] if shapes else None)
        ors.append(o)
        gps.append(g)
    res = gpu_global_step(gps, False, wl.C, wl.sigma, wl.seed)
    _check_global(wl, ors, res)


def test_gpt_block_t128_full():
    """The benchmark's workload at full size, every output compared."""
    wl = W.WORKLOADS["gpt-block-t128"]
    ors, gps = [], []
    for l in range(wl.n_layers):
        _, o, g = layer_inputs(wl, l)
        ors.append(o)
        gps.append(g)
    res = gpu_global_step(gps, False, wl.C, wl.sigma, wl.seed)
    assert all(p == dpc.PATH_GHOST for p in res["paths"])
    _check_global(wl, ors, res)


def test_resnet18_conv_full():
    wl = W.WORKLOADS["resnet18-conv-t1024"]
    ors, gps = [], []
    for l in range(wl.n_layers):
        _, o, g = layer_inputs(wl, l)
        ors.append(o)
        gps.append(g)
    res = gpu_global_step(gps, False, wl.C, wl.sigma, wl.seed)
    assert res["paths"][:2] == [dpc.PATH_EXPLICIT] * 2 and res["paths"][2:] == [dpc.PATH_GHOST] * 6
    _check_global(wl, ors, res)


def _adaptive_gpu_step(gps, C_t, wl, step, denom):
    """Per-layer clipping with bound C_t[l], then the bound update."""
    outs, bouts, norms, cs, C_next = [], [], [], [], []
    for l, (A, G) in enumerate(gps):
        B, d, p = A.shape[0], A.shape[2], G.shape[2]
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_ghost_norm(A, G, sq, has_bias=True)
        c = torch.empty_like(sq)
        nrm = torch.empty_like(sq)
        dpc.dp_clip_factors(sq, C_t[l], c, nrm)
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        bout = torch.empty(p, dtype=torch.float32, device=dev())
        dpc.dp_clipped_sum_noise(A, G, c, C_t[l], wl.sigma, denom, wl.seed, l, step, out, bout)
        cn = torch.empty(1, dtype=torch.float32, device=dev())
        dpc.dp_adaptive_threshold(nrm, C_t[l], wl.alpha, wl.beta, wl.sigma_l2, False, wl.seed, l, step + 1, cn)
        outs.append(out); bouts.append(bout); norms.append(nrm); cs.append(c); C_next.append(cn)
    torch.cuda.synchronize()
    return dict(outs=[o.cpu().numpy() for o in outs], bias_outs=[b.cpu().numpy() for b in bouts],
                norms=[n.cpu().numpy() for n in norms], c=[c.cpu().numpy() for c in cs],
                C_next=[float(c.item()) for c in C_next])


def test_mlp_adaptive_chain_reduced():
    """Per-layer adaptive clipping, init batch + 4 steps, free running: the GPU
    carries its own bounds from step to step, the oracle its own."""
    wl = W.WORKLOADS["mlp-b65536-adaptive"]
    B = 300
    shapes = [(1, 96, 128), (1, 128, 128), (1, 128, 40)]
    denom = float(B)
    # init batch (step -1)
    ors, gps = [], []
    for l, s in enumerate(shapes):
        _, o, g = layer_inputs(wl, l, step=-1, B=B, shape=s)
        ors.append(o)
        gps.append(g)
    C_l2_or, C_or = drivers.adaptive_init(ors, wl.alpha, wl.beta, wl.sigma_l2, wl.seed)
    C_gpu = []
    for l, (A, G) in enumerate(gps):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_ghost_norm(A, G, sq, has_bias=True)
        nrm, cdummy = torch.empty_like(sq), torch.empty_like(sq)
        dpc.dp_clip_factors(sq, 3.0e38, cdummy, nrm)
        cn = torch.empty(1, dtype=torch.float32, device=dev())
        cl2 = torch.empty(1, dtype=torch.float32, device=dev())
        dpc.dp_adaptive_threshold(nrm, 1.0, wl.alpha, wl.beta, wl.sigma_l2, True, wl.seed, l, 0, cn, cl2)
        assert abs(cl2.item() - C_l2_or[l]) <= 1e-4 * C_l2_or[l]
        C_gpu.append(float(cn.item()))
    np.testing.assert_allclose(C_gpu, C_or, rtol=1e-4)
    for step in range(4):
        ors, gps = [], []
        for l, s in enumerate(shapes):
            _, o, g = layer_inputs(wl, l, step=step, B=B, shape=s)
            ors.append(o)
            gps.append(g)
        ref = drivers.adaptive_step(ors, C_or, wl.sigma, wl.alpha, wl.beta, wl.sigma_l2, wl.seed, step,
                                    has_bias=True, denom=denom)
        res = _adaptive_gpu_step(gps, C_gpu, wl, step, denom)
        for l in range(len(shapes)):
            assert_norms(res["norms"][l], ref["norms"][l], "f32", what=f"step{step} norm[{l}]")
            assert_clip(res["c"][l], ref["c"][l], ref["norms"][l], C_or[l], "f32")
            S = ref["sums"][l]
            nz = wl.sigma * C_or[l] * N.weight_noise(S.shape[0], S.shape[1], wl.seed, l, step) / denom
            crel = abs(C_gpu[l] - C_or[l]) / C_or[l] + 1e-7
            assert_noised(res["outs"][l], ref["outs"][l], S, nz, "f32", denom, what=f"step{step} out[{l}]",
                          noise_rtol=crel)
            assert np.any(res["c"][l] < 1.0) and np.any(res["c"][l] == 1.0)  # both branches exercised
        np.testing.assert_allclose(res["C_next"], ref["C_next"], rtol=1e-4)
        C_gpu, C_or = res["C_next"], ref["C_next"]


# ------------------------------------------------------------------ full-size sampled cases
def test_mlp_full_size_sampled():
    """B = 65536, the 4096 -> 4096 layer with bias: norms of sampled examples,
    sampled entries of the clipped noised sum (seeded clip factors), and the
    adaptive bound of the full batch."""
    wl = W.WORKLOADS["mlp-b65536-adaptive"]
    l = 1
    A_raw, G_raw = W.make_layer(wl, l, step=0)
    A, G = upload(A_raw, "f32"), upload(G_raw, "f32")
    B, T, d = A.shape
    p = G.shape[2]
    sq = torch.empty(B, dtype=torch.float32, device=dev())
    assert dpc.dp_ghost_norm(A, G, sq, has_bias=True) == dpc.PATH_T1
    rng = np.random.default_rng(77)
    idx = np.sort(rng.choice(B, 48, replace=False))
    sq_or = D.layer_sqnorms(A_raw[idx].astype(np.float64), G_raw[idx].astype(np.float64), has_bias=True)
    assert_norms(np.sqrt(sq.cpu().numpy()[idx]), np.sqrt(sq_or), "f32")
    c_np = W.make_vector(B, 0.05, 1.0, tag=1)
    c = f32(c_np)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev())
    dpc.dp_clipped_sum_noise(A, G, c, 2.0, wl.sigma, float(B), wl.seed, l, 3, out, bout)
    torch.cuda.synchronize()
    rows = rng.integers(0, d, 96)
    cols = rng.integers(0, p, 96)
    S_or = D.clipped_sum_entries(A_raw, G_raw, c_np, rows, cols)
    z = N.weight_noise_at(rows, cols, p, wl.seed, l, 3)
    out_or = D.noised_mean(S_or, z, 2.0, wl.sigma, B)
    # the scale of S is estimated from the sampled entries (random signs: entries share one scale)
    assert_noised(out.cpu().numpy()[rows, cols], out_or, S_or, wl.sigma * 2.0 * z / B, "f32", B)
    # bias entries: S_b[n] = sum_i c_i G_i[0, n]
    bcols = rng.integers(0, p, 64)
    Sb_or = np.array([np.dot(c_np.astype(np.float64), G_raw[:, 0, n].astype(np.float64)) for n in bcols])
    zb = N.normals_at(bcols, wl.seed, l, 1, 3)
    assert_noised(bout.cpu().numpy()[bcols], D.noised_mean(Sb_or, zb, 2.0, wl.sigma, B), Sb_or,
                  wl.sigma * 2.0 * zb / B, "f32", B)
    # adaptive bound over the full batch from the GPU's own norms vs the oracle on the same values
    nrm_np = W.make_vector(B, 100.0, 3000.0, tag=2)
    nrm = f32(nrm_np)
    cn = torch.empty(1, dtype=torch.float32, device=dev())
    for init, C_prev in ((True, 1.0), (False, 900.0)):
        dpc.dp_adaptive_threshold(nrm, C_prev, wl.alpha, wl.beta, wl.sigma_l2, init, wl.seed, l, 5, cn)
        _, ref = D.adaptive_threshold(nrm_np, C_prev, wl.alpha, wl.beta, wl.sigma_l2, init,
                                      N.threshold_normal(wl.seed, l, 5))
        assert abs(cn.item() - ref) <= 1e-4 * abs(ref)


@pytest.mark.parametrize("l", [0, 3])
def test_gpt2large_full_size_layer(l):
    """One decoder block's qkv (0) or fc2 (3) layer at full size (B=32,
    T=1024): every norm, and sampled entries of the clipped noised sum."""
    wl = W.WORKLOADS["gpt2large-t1024"]
    (A_raw, G_raw), (Ao, Go), (A, G) = layer_inputs(wl, l)
    B, T, d = A.shape
    p = G.shape[2]
    sq = torch.empty(B, dtype=torch.float32, device=dev())
    assert dpc.dp_ghost_norm(A, G, sq) == dpc.PATH_GHOST
    torch.cuda.synchronize()
    sq_or = D.layer_sqnorms(Ao, Go)
    assert_norms(np.sqrt(sq.cpu().numpy()), np.sqrt(sq_or), "bf16")
    c_np = W.make_vector(B, 0.05, 1.0, tag=3)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    dpc.dp_clipped_sum_noise(A, G, f32(c_np), 1.0, 1.0, float(B), wl.seed, l, 0, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = rng.integers(0, d, 64)
    cols = rng.integers(0, p, 64)
    S_or = D.clipped_sum_entries(Ao, Go, c_np, rows, cols)
    z = N.weight_noise_at(rows, cols, p, wl.seed, l, 0)
    assert_noised(out.cpu().numpy()[rows, cols], D.noised_mean(S_or, z, 1.0, 1.0, B), S_or, z / B, "bf16", B)


# ------------------------------------------------------------------ noise, edge cases, determinism
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T", [(3, 5), (2048, 3)])   # one K split (fused epilogue) / many (reduce kernel)
def test_noise_bit_exact(dtype, B, T):
    """With c = 0 the clipped sum is exactly 0, so out is pure noise and must
    equal the oracle's fp32 replica of the specified stream bit for bit."""
    d, p = 13, 7  # a partial last row group and a partial last bias group
    rng = np.random.default_rng(3)
    A = rng.standard_normal((B, T, d)).astype(np.float32)
    G = rng.standard_normal((B, T, p)).astype(np.float32)
    if dtype == "bf16":
        A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
    c = torch.zeros(B, dtype=torch.float32, device=dev())
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev())
    C, sigma, denom, seed, layer, step = 1.3, 0.7, 7.0, (5 << 32) | 11, 9, 4
    dpc.dp_clipped_sum_noise(upload(A, dtype), upload(G, dtype), c, C, sigma, denom, seed, layer, step, out, bout)
    torch.cuda.synchronize()
    zw = N.weight_noise(d, p, seed, layer, step)
    zb = N.normals(p, seed, layer, 1, step)
    np.testing.assert_array_equal(out.cpu().numpy(), D.noised_mean_f32(np.zeros((d, p)), zw, C, sigma, denom))
    np.testing.assert_array_equal(bout.cpu().numpy(), D.noised_mean_f32(np.zeros(p), zb, C, sigma, denom))


def test_noise_bit_exact_large():
    # a large stream: 2^20 + 3 elements
    d2, p2 = 1031, 1017   # d2 % 4 == 3: a partial last row group
    A2 = torch.zeros(1, 1, d2, dtype=torch.float32, device=dev())
    G2 = torch.zeros(1, 1, p2, dtype=torch.float32, device=dev())
    out2 = torch.empty(d2, p2, dtype=torch.float32, device=dev())
    dpc.dp_clipped_sum_noise(A2, G2, torch.zeros(1, device=dev()), 1.0, 1.0, 1.0, 0, 0, 0, out2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out2.cpu().numpy(), N.weight_noise(d2, p2, 0, 0, 0))


EDGE = [
    # dtype, B, T, d, p, has_bias, mode
    ("f32", 1, 1, 1, 1, True, dpc.MODE_MIXED),
    ("bf16", 9, 1, 24, 40, True, dpc.MODE_MIXED),       # T = 1 closed form in bf16
    ("f32", 7, 1, 33, 17, True, dpc.MODE_EXPLICIT),     # explicit forced at T = 1, odd sizes
    ("f32", 4, 70, 27, 64, False, dpc.MODE_GHOST),      # ghost forced where explicit is chosen; d % 4 != 0
    ("f32", 4, 9, 300, 200, True, dpc.MODE_EXPLICIT),   # explicit forced where ghost is chosen
    ("bf16", 3, 65, 20, 44, True, dpc.MODE_MIXED),      # bf16 rows not 16-byte aligned -> scalar loads
    ("bf16", 2, 1, 7, 3, False, dpc.MODE_EXPLICIT),
    ("f32", 17, 129, 130, 129, True, dpc.MODE_GHOST),   # ragged everywhere, tile 64 with 3 row blocks
    ("bf16", 2, 513, 72, 40, False, dpc.MODE_GHOST),    # tile 128, ragged 5th block
]


@pytest.mark.parametrize("dtype,B,T,d,p,hb,mode", EDGE)
def test_edge_shapes(dtype, B, T, d, p, hb, mode):
    rng = np.random.default_rng(B * 1000 + T)
    A = rng.standard_normal((B, T, d)).astype(np.float32)
    G = rng.standard_normal((B, T, p)).astype(np.float32)
    if dtype == "bf16":
        A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
    Ao, Go = W.as_f64(A, dtype), W.as_f64(G, dtype)
    Ad, Gd = upload(A, dtype), upload(G, dtype)
    sq = torch.full((B,), 5.0, dtype=torch.float32, device=dev())
    path = dpc.dp_ghost_norm(Ad, Gd, sq, has_bias=hb, mode=mode, accumulate=True)
    assert path == D.choose_path(T, d, p, mode)
    sq_or = D.layer_sqnorms(Ao, Go, hb)
    torch.cuda.synchronize()
    assert_norms(sq.cpu().numpy() - 5.0, sq_or, dtype, what="accumulated sqnorm")
    c_np = rng.uniform(0.0, 1.0, B).astype(np.float32)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
    dpc.dp_clipped_sum_noise(Ad, Gd, f32(c_np), 1.0, 0.0, 3.0, 0, 0, 0, out, bout)
    torch.cuda.synchronize()
    S, Sb = D.clipped_sum(Ao, Go, c_np.astype(np.float64), hb)
    assert_sum(out.cpu().numpy() * 3.0, S, dtype)
    if hb:
        assert_sum(bout.cpu().numpy() * 3.0, Sb, dtype, what="bias sum")


def test_clip_factor_special_values():
    C = 2.0
    sq = np.array([0.0, 4.0, 4.0000005, 1e30, -1e-12, 9.0, np.inf, np.nan], dtype=np.float32)
    c = torch.empty(len(sq), dtype=torch.float32, device=dev())
    nrm = torch.empty_like(c)
    dpc.dp_clip_factors(f32(sq), C, c, nrm)
    torch.cuda.synchronize()
    cg, ng = c.cpu().numpy(), nrm.cpu().numpy()
    fin = np.isfinite(sq)
    n_or = np.sqrt(np.maximum(sq[fin].astype(np.float64), 0.0))
    np.testing.assert_allclose(ng[fin], n_or, rtol=1e-6)
    np.testing.assert_allclose(cg[fin], D.clip_factors(n_or, C), rtol=1e-6)
    assert cg[1] == 1.0 and cg[0] == 1.0          # norm == C and norm == 0 are not clipped
    assert cg[6] == 0.0 and np.isnan(cg[7]) and np.isnan(ng[7])


def test_deterministic_bitwise():
    wl = W.WORKLOADS["gpt-block-t128"]
    B, shapes = REDUCED["gpt-block-t128"]
    gps = [layer_inputs(wl, l, B=B, shape=s)[2] for l, s in enumerate(shapes)]
    r1 = gpu_global_step(gps, False, wl.C, wl.sigma, 3)
    r2 = gpu_global_step(gps, False, wl.C, wl.sigma, 3)
    np.testing.assert_array_equal(r1["sq"], r2["sq"])
    for a, b in zip(r1["outs"], r2["outs"]):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ direct-to-LDS bf16 contraction engine
# bf16 layers without bias whose T is a multiple of 64 and whose d, p are
# multiples of 8 take this engine. The cases reach its plans: 128x128 and
# 256x128 tiles, one K split (noise in the contraction's epilogue) and many
# (partials + reduce kernel), splits that start inside a sample, ragged
# last tiles and widths below one 16-byte piece per tile.
DL_CASES = [
    # B, T, d, p
    (1, 64, 200, 328),      # 128x128, one split, ragged d and p
    (64, 64, 8, 8),         # 128x128, 64 splits; every tile column past d/p
    (6, 128, 264, 392),     # 128x128, splits on sample boundaries
    (40, 128, 264, 136),    # 128x128, 3 chunks per split: splits start mid-sample
    (32, 128, 776, 2312),   # 256x128, 3 splits, ragged
    (4, 64, 2056, 4104),    # 256x128, one split, ragged
]


@pytest.mark.parametrize("B,T,d,p", DL_CASES)
def test_dl_engine_clipped_sum(B, T, d, p):
    rng = np.random.default_rng(B * 7919 + d)
    A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / math.sqrt(d)).astype(np.float32))
    G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / math.sqrt(p)).astype(np.float32))
    c_np = rng.uniform(0.0, 1.0, B).astype(np.float32)
    c_np[0] = 1.0
    if B > 2:
        c_np[2] = 0.0
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    dpc.dp_clipped_sum_noise(upload(A, "bf16"), upload(G, "bf16"), f32(c_np), 1.0, 0.0, 1.0, 0, 0, 0, out)
    torch.cuda.synchronize()
    S, _ = D.clipped_sum(W.as_f64(A, "bf16"), W.as_f64(G, "bf16"), c_np.astype(np.float64), False)
    assert_sum(out.cpu().numpy(), S, "bf16")


@pytest.mark.parametrize("B", [2, 512])   # one K split / 256 splits (reduce kernel)
def test_dl_engine_noise_bit_exact(B):
    T, d, p = 64, 24, 16
    rng = np.random.default_rng(11)
    A = W.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32))
    G = W.f32_to_bf16_bits(rng.standard_normal((B, T, p)).astype(np.float32))
    c = torch.zeros(B, dtype=torch.float32, device=dev())
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    C, sigma, denom, seed, layer, step = 0.9, 1.7, 3.0, (7 << 32) | 5, 3, 12
    dpc.dp_clipped_sum_noise(upload(A, "bf16"), upload(G, "bf16"), c, C, sigma, denom, seed, layer, step, out)
    torch.cuda.synchronize()
    zw = N.weight_noise(d, p, seed, layer, step)
    np.testing.assert_array_equal(out.cpu().numpy(), D.noised_mean_f32(np.zeros((d, p)), zw, C, sigma, denom))


def test_dl_engine_workspace_reuse():
    """Split-K tiles leave partials in the workspace for the reduce kernel. A
    workspace full of arbitrary bytes, and one reused by earlier calls, must
    both give the oracle's sums, bit-identically for identical inputs."""
    B, T, d, p = 40, 128, 264, 136
    rng = np.random.default_rng(5)
    A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / math.sqrt(d)).astype(np.float32))
    G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / math.sqrt(p)).astype(np.float32))
    Ad, Gd = upload(A, "bf16"), upload(G, "bf16")
    Ao, Go = W.as_f64(A, "bf16"), W.as_f64(G, "bf16")
    nbytes = dpc.dp_workspace_bytes(dpc.DP_BF16, B, T, d, p)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev())
    outs = []
    for k in range(3):
        c_np = (rng.uniform(0.0, 1.0, B) if k < 2 else c_first).astype(np.float32)
        if k == 0:
            c_first = c_np.copy()
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        dpc.dp_clipped_sum_noise(Ad, Gd, f32(c_np), 1.0, 0.0, 1.0, 0, 0, 0, out, workspace=ws)
        torch.cuda.synchronize()
        S, _ = D.clipped_sum(Ao, Go, c_np.astype(np.float64), False)
        assert_sum(out.cpu().numpy(), S, "bf16", what=f"call {k}")
        outs.append(out.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[2])


# ------------------------------------------------------------------ bf16 256 x 256 tiles
# Large bf16 layers with long K per work item (here the GPT-2-large qkv
# linear) take 256 x 256 tiles with one accumulator set: the running sum is
# kept divided by the current sample's clip factor and rescaled at each
# sample; zero factors are skipped and a NaN factor propagates. Sampled
# entries are compared with the oracle's definition.
def _clip_pattern(kind, B, rng):
    if kind == "zeros-and-range":
        c = rng.uniform(0.0, 1.0, B)
        c[:3] = 0.0
        c[B // 2] = 0.0
        c[-1] = 0.0
        c[5] = 1e-4
        c[6] = 1.0
        c[9] = 3e-3
        return c.astype(np.float32)
    if kind == "all-zero":
        return np.zeros(B, dtype=np.float32)
    c = rng.uniform(0.2, 1.0, B).astype(np.float32)
    c[7] = np.nan
    return c


@pytest.fixture(scope="module")
def gpt2large_qkv():
    wl = W.WORKLOADS["gpt2large-t1024"]
    return layer_inputs(wl, 0)


@pytest.mark.parametrize("kind", ["zeros-and-range", "all-zero", "nan"])
def test_wide_tile_clip_patterns(kind, gpt2large_qkv):
    (A_raw, G_raw), (Ao, Go), (A, G) = gpt2large_qkv
    B, T, d = A.shape
    p = G.shape[2]
    assert dpc.dp_workspace_bytes(dpc.DP_BF16, B, T, d, p) > 0
    rng = np.random.default_rng(23)
    c_np = _clip_pattern(kind, B, rng)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    sigma = 1.0 if kind == "all-zero" else 0.0
    C, denom, seed, l, step = 0.7, 3.0, 11, 0, 2
    dpc.dp_clipped_sum_noise(A, G, f32(c_np), C, sigma, denom, seed, l, step, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = rng.integers(0, d, 96)
    cols = rng.integers(0, p, 96)
    if kind == "all-zero":
        z = N.weight_noise_at(rows, cols, p, seed, l, step)
        np.testing.assert_array_equal(got[rows, cols],
                                      D.noised_mean_f32(np.zeros(rows.shape[0]), z, C, sigma, denom))
        return
    if kind == "nan":
        assert np.isnan(got).all()
        return
    S_or = D.clipped_sum_entries(Ao, Go, c_np.astype(np.float64), rows, cols)
    assert_noised(got[rows, cols], S_or / denom, S_or, np.zeros(rows.shape[0]), "bf16", denom)


# ------------------------------------------------------------------ fp32 direct-to-LDS engine
# fp32 layers with d, p >= 128, multiples of 4, and B*T a multiple of 32 go to
# the direct-to-LDS fp32 engine (32-row chunks, 256x128 tiles, bias summed on
# the side in the tiles that hold output row 0).
DL32_CASES = [
    # B, T, d, p, has_bias
    (256, 1, 128, 128, True),     # T = 1: one sample per chunk row; 8 chunks -> K splits + reduce
    (64, 16, 260, 132, True),     # two samples per chunk; ragged d (2 m-tiles) and p (clamped columns)
    (8, 48, 384, 256, False),     # chunks straddle samples (48 rows per sample)
    (2048, 1, 512, 640, True),    # 64 chunks, bias with several n-tiles
    (4, 1024, 1152, 128, False),  # one sample per chunk, long K per sample
    (32, 1, 4096, 1000, True),    # one chunk: one split, fused epilogue; 16 m-tiles, ragged last n-tile
]


@pytest.mark.parametrize("B,T,d,p,hb", DL32_CASES)
def test_dl32_engine_clipped_sum(B, T, d, p, hb):
    rng = np.random.default_rng(B * 104729 + d * 31 + p)
    A = rng.standard_normal((B, T, d)).astype(np.float32)
    G = rng.standard_normal((B, T, p)).astype(np.float32)
    c_np = rng.uniform(0.0, 1.0, B).astype(np.float32)
    c_np[0] = 1.0
    if B > 2:
        c_np[2] = 0.0
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
    dpc.dp_clipped_sum_noise(upload(A, "f32"), upload(G, "f32"), f32(c_np), 1.0, 0.0, 1.0, 0, 0, 0, out, bout)
    torch.cuda.synchronize()
    S, Sb = D.clipped_sum(A.astype(np.float64), G.astype(np.float64), c_np.astype(np.float64), bool(hb))
    assert_sum(out.cpu().numpy(), S, "f32")
    if hb:
        assert_sum(bout.cpu().numpy(), Sb, "f32", what="bias sum")


@pytest.mark.parametrize("B", [32, 8192])   # one chunk (fused epilogue) / 256 chunks (K splits + reduce)
def test_dl32_engine_noise_bit_exact(B):
    T, d, p = 1, 128, 132
    rng = np.random.default_rng(13)
    A = rng.standard_normal((B, T, d)).astype(np.float32)
    G = rng.standard_normal((B, T, p)).astype(np.float32)
    c = torch.zeros(B, dtype=torch.float32, device=dev())
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev())
    C, sigma, denom, seed, layer, step = 1.3, 0.725, 7.0, (3 << 32) | 9, 2, 4
    dpc.dp_clipped_sum_noise(upload(A, "f32"), upload(G, "f32"), c, C, sigma, denom, seed, layer, step, out, bout)
    torch.cuda.synchronize()
    zw = N.weight_noise(d, p, seed, layer, step)
    np.testing.assert_array_equal(out.cpu().numpy(), D.noised_mean_f32(np.zeros((d, p)), zw, C, sigma, denom))
    zb = N.normals(p, seed, layer, 1, step)
    np.testing.assert_array_equal(bout.cpu().numpy(), D.noised_mean_f32(np.zeros(p), zb, C, sigma, denom))


# ------------------------------------------------------------------ one- and two-block ghost samples
# Samples of one or two Gram row blocks with wide and narrow feature counts on
# either side, bias on and off, accumulation into sqnorm.
SPLIT_CASES = [
    # dtype, B, T, d, p, has_bias
    ("bf16", 5, 128, 1024, 192, True),   # d >> p, bias
    ("bf16", 7, 128, 128, 640, True),    # p >> d, bias
    ("bf16", 3, 100, 256, 384, False),   # rows past T
    ("bf16", 20, 128, 64, 64, True),     # 20 samples over 3 XCD groups
    ("bf16", 4, 128, 1024, 256, True),   # two row blocks, d >> p, bias
    ("f32", 3, 128, 320, 64, True),      # the same in fp32
    ("f32", 6, 64, 320, 64, True),
    ("f32", 4, 128, 96, 224, True),
]


@pytest.mark.parametrize("dtype,B,T,d,p,hb", SPLIT_CASES)
def test_ghost_single_tile_samples(dtype, B, T, d, p, hb):
    rng = np.random.default_rng(B * 977 + d + p)
    A = (rng.standard_normal((B, T, d)) / math.sqrt(d)).astype(np.float32)
    G = (rng.standard_normal((B, T, p)) / math.sqrt(p)).astype(np.float32)
    if dtype == "bf16":
        A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
    Ad, Gd = upload(A, dtype), upload(G, dtype)
    sq = torch.full((B,), 3.0, dtype=torch.float32, device=dev())
    assert dpc.dp_ghost_norm(Ad, Gd, sq, has_bias=hb, mode=dpc.MODE_GHOST, accumulate=True) == dpc.PATH_GHOST
    torch.cuda.synchronize()
    sq_or = D.layer_sqnorms(W.as_f64(A, dtype), W.as_f64(G, dtype), hb)
    assert_norms(sq.cpu().numpy() - 3.0, sq_or, dtype, what="accumulated sqnorm")
    sq2 = torch.empty(B, dtype=torch.float32, device=dev())
    dpc.dp_ghost_norm(Ad, Gd, sq2, has_bias=hb, mode=dpc.MODE_GHOST)
    torch.cuda.synchronize()
    assert_norms(sq2.cpu().numpy(), sq_or, dtype)


# ------------------------------------------------------------------ many K splits, small outputs
# Narrow layers split K into >= 64 parts; the reduce then runs split lanes in
# parallel (16 lanes per 4 x 16 output block, summed in lane order).
WIDE_REDUCE_CASES = [
    # dtype, B, T, d, p, has_bias
    ("f32", 64, 1024, 27, 64, True),   # the unfolded 3-channel 3x3 conv layer shape
    ("f32", 4096, 4, 29, 36, False),   # partial last row group, partial last 16-column block
    ("bf16", 2048, 2, 13, 12, True),
]


def _wide_case(dtype, B, T, d, p, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((B, T, d)).astype(np.float32)
    G = rng.standard_normal((B, T, p)).astype(np.float32)
    if dtype == "bf16":
        A, G = W.f32_to_bf16_bits(A), W.f32_to_bf16_bits(G)
    nbytes = dpc.dp_workspace_bytes(dpc.DP_BF16 if dtype == "bf16" else dpc.DP_F32, B, T, d, p)
    assert nbytes >= 64 * (d + 1) * p * 4, "expected at least 64 K splits"
    return A, G, rng


@pytest.mark.parametrize("dtype,B,T,d,p,hb", WIDE_REDUCE_CASES)
def test_wide_reduce_clipped_sum(dtype, B, T, d, p, hb):
    A, G, rng = _wide_case(dtype, B, T, d, p, B + d)
    c_np = rng.uniform(0.0, 1.0, B).astype(np.float32)
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
    dpc.dp_clipped_sum_noise(upload(A, dtype), upload(G, dtype), f32(c_np), 1.0, 0.0, 1.0, 0, 0, 0, out, bout)
    torch.cuda.synchronize()
    S, Sb = D.clipped_sum(W.as_f64(A, dtype), W.as_f64(G, dtype), c_np.astype(np.float64), hb)
    assert_sum(out.cpu().numpy(), S, dtype)
    if hb:
        assert_sum(bout.cpu().numpy(), Sb, dtype, what="bias sum")


@pytest.mark.parametrize("dtype,B,T,d,p,hb", WIDE_REDUCE_CASES)
def test_wide_reduce_noise_bit_exact(dtype, B, T, d, p, hb):
    A, G, _ = _wide_case(dtype, B, T, d, p, 17)
    c = torch.zeros(B, dtype=torch.float32, device=dev())
    out = torch.empty(d, p, dtype=torch.float32, device=dev())
    bout = torch.empty(p, dtype=torch.float32, device=dev()) if hb else None
    C, sigma, denom, seed, layer, step = 0.8, 1.1, 5.0, (9 << 32) | 2, 6, 3
    dpc.dp_clipped_sum_noise(upload(A, dtype), upload(G, dtype), c, C, sigma, denom, seed, layer, step, out, bout)
    torch.cuda.synchronize()
    zw = N.weight_noise(d, p, seed, layer, step)
    np.testing.assert_array_equal(out.cpu().numpy(), D.noised_mean_f32(np.zeros((d, p)), zw, C, sigma, denom))
    if hb:
        zb = N.normals(p, seed, layer, 1, step)
        np.testing.assert_array_equal(bout.cpu().numpy(), D.noised_mean_f32(np.zeros(p), zb, C, sigma, denom))


# ------------------------------------------------------------------ concurrent calls
def test_concurrent_streams_bitwise():
    """Clipped sums of several layers issued on separate HIP streams at once
    (each with its own workspace) equal the same calls issued one after
    another, bit for bit."""
    wl = W.WORKLOADS["gpt-block-t128"]
    B = 16
    shapes = [(128, 256, 512), (128, 384, 256), (64, 512, 384)]
    layers = []
    for l, sh in enumerate(shapes):
        A, G = W.make_layer(wl, l, B=B, shape=sh)
        layers.append((upload(A, "bf16"), upload(G, "bf16")))
    c = f32(W.make_vector(B, 0.1, 1.0, tag=5))

    def run(concurrent):
        outs = [torch.empty(sh[1], sh[2], dtype=torch.float32, device=dev()) for sh in shapes]
        wss = [torch.empty(max(256, dpc.dp_workspace_bytes(dpc.DP_BF16, B, *sh)), dtype=torch.uint8, device=dev())
               for sh in shapes]
        streams = [torch.cuda.Stream() for _ in shapes] if concurrent else [torch.cuda.current_stream()] * 3
        torch.cuda.synchronize()
        for l, (A, G) in enumerate(layers):
            with torch.cuda.stream(streams[l]):
                dpc.dp_clipped_sum_noise(A, G, c, 1.0, 1.0, float(B), 3, l, 7, outs[l], workspace=wss[l])
        torch.cuda.synchronize()
        return [o.cpu().numpy() for o in outs]

    serial = run(False)
    for _ in range(3):
        for a_, b_ in zip(run(True), serial):
            np.testing.assert_array_equal(a_, b_)


# ------------------------------------------------------------------ ghost path shapes
# bf16 ghost norms over 64-row tiles (T <= 384), 128-row tiles (T > 384) and
# the long-sequence engine's 256 x 128 tiles (T > 64 with d and p multiples
# of 64; at T <= 128 one 128 x 128 tile per sample): one tile with most rows
# past T, ragged T, up to 36 tiles per sample, several short samples stacked
# in one tile, bias on and off, accumulation into sqnorm.
GHOST_CASES = [
    # B, T, d, p, has_bias
    (3, 5, 128, 256, True),      # 1 tile of 64
    (4, 100, 200, 128, False),   # 3 tiles, ragged
    (5, 128, 136, 128, True),    # 3 tiles
    (9, 64, 128, 128, True),     # 1 tile
    (3, 200, 136, 256, True),    # 10 tiles, ragged
    (2, 300, 232, 128, False),   # 15 tiles, ragged
    (2, 385, 72, 192, True),     # 128-row tiles: 10, ragged
    (4, 100, 256, 128, False),   # long-sequence engine: one 128 x 128 tile, 28 rows past T
    (5, 128, 384, 128, False),   # one 128 x 128 tile: the gpt-block T
    (3, 65, 64, 192, True),      # one tile, one row of its second half
    (3, 200, 128, 256, True),    # 2 tiles (128 x 128, 256 x 128), ragged
    (2, 300, 256, 128, False),   # 4 tiles, ragged
    (2, 385, 64, 192, True),     # 6 tiles, ragged
    (1, 1000, 128, 64, False),   # 28 tiles, ragged
    (2, 512, 64, 128, True),     # 6 tiles
    (3, 600, 128, 192, False),   # 9 tiles, last row block 88 rows
    (1, 1100, 192, 64, True),    # 25 tiles, ragged
    (4, 1024, 64, 64, False),    # 20 tiles
    (9, 520, 64, 64, True),      # 9 tiles; samples on two XCD rounds
    (9, 16, 128, 64, True),      # 4 samples per 64-row tile: packs of 4, 4, 1
    (5, 32, 64, 128, False),     # 2 samples per tile, the last pack half full
    (7, 20, 96, 64, True),       # 3 samples per tile (60 of 64 rows), packs of 3, 3, 1
]


@pytest.mark.parametrize("B,T,d,p,hb", GHOST_CASES)
def test_ghost_norms_shapes(B, T, d, p, hb):
    rng = np.random.default_rng(B * 131 + T)
    A = W.f32_to_bf16_bits((rng.standard_normal((B, T, d)) / math.sqrt(d)).astype(np.float32))
    G = W.f32_to_bf16_bits((rng.standard_normal((B, T, p)) / math.sqrt(p)).astype(np.float32))
    Ad, Gd = upload(A, "bf16"), upload(G, "bf16")
    sq = torch.full((B,), 2.0, dtype=torch.float32, device=dev())
    path = dpc.dp_ghost_norm(Ad, Gd, sq, has_bias=hb, mode=dpc.MODE_GHOST, accumulate=True)
    assert path == dpc.PATH_GHOST
    torch.cuda.synchronize()
    sq_or = D.layer_sqnorms(W.as_f64(A, "bf16"), W.as_f64(G, "bf16"), hb)
    assert_norms(sq.cpu().numpy() - 2.0, sq_or, "bf16", what="accumulated sqnorm")
    sq2 = torch.empty(B, dtype=torch.float32, device=dev())
    dpc.dp_ghost_norm(Ad, Gd, sq2, has_bias=hb, mode=dpc.MODE_GHOST)
    torch.cuda.synchronize()
    assert_norms(sq2.cpu().numpy(), sq_or, "bf16")
