"""The adaptive per-layer clipping schedule of "Three Tools for Practical
Differential Privacy" on the GPU, as the MLP workload configures it: an
initialisation batch of random-noise inputs, then 10 steps on fresh inputs,
layer l clipped with its bound C_t[l] and C_{t+1}[l] produced from step t's
norms (C_l2 = beta * C_t). The layers keep the MLP's structure (T = 1, bias,
three layers, alpha = 1.1, beta = 2, sigma = 0.725, sigma_l2 = 2.5) at a
reduced width and batch so that the fp64 oracle materialises every
per-example gradient of all 10 steps in seconds.

Three checks: free running (each side carries its own bounds), teacher
forced (the oracle's step t uses the GPU's C_t, so a mismatch cannot hide in
accumulated drift), and resume (restarting the GPU schedule from a saved
(C_t, t, seed) reproduces steps t..9 bit for bit).
"""
import numpy as np
import pytest
import torch

import sample_gradient_clipping_layer_amd as dpc
import workloads as W
from oracle import drivers
from oracle import noise as N

from gpu_util import assert_clip, assert_noised, assert_norms, dev, layer_inputs

pytestmark = pytest.mark.gpu

WL = W.WORKLOADS["mlp-b65536-adaptive"]
B = 1024
SHAPES = [(1, 160, 192), (1, 192, 192), (1, 192, 56)]
STEPS = WL.steps


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    dpc.lib()


@pytest.fixture(scope="module")
def batches():
    """Inputs of the init batch (step -1) and of steps 0..9, host fp64 and device."""
    out = {}
    for step in range(-1, STEPS):
        ors, gps = [], []
        for l, s in enumerate(SHAPES):
            _, o, g = layer_inputs(WL, l, step=step, B=B, shape=s)
            ors.append(o)
            gps.append(g)
        out[step] = (ors, gps)
    return out


def _gpu_init(gps):
    C = []
    for l, (A, G) in enumerate(gps):
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_ghost_norm(A, G, sq, has_bias=True)
        nrm, cdummy = torch.empty_like(sq), torch.empty_like(sq)
        dpc.dp_clip_factors(sq, 3.0e38, cdummy, nrm)
        cn = torch.empty(1, dtype=torch.float32, device=dev())
        dpc.dp_adaptive_threshold(nrm, 1.0, WL.alpha, WL.beta, WL.sigma_l2, True, WL.seed, l, 0, cn)
        C.append(float(cn.item()))
    return C


def _gpu_step(gps, C_t, step):
    """Step `step` of the schedule with bounds C_t: every output as numpy."""
    res = dict(outs=[], bias_outs=[], norms=[], c=[], C_next=[])
    for l, (A, G) in enumerate(gps):
        d, p = A.shape[2], G.shape[2]
        sq = torch.empty(B, dtype=torch.float32, device=dev())
        dpc.dp_ghost_norm(A, G, sq, has_bias=True)
        c, nrm = torch.empty_like(sq), torch.empty_like(sq)
        dpc.dp_clip_factors(sq, C_t[l], c, nrm)
        out = torch.empty(d, p, dtype=torch.float32, device=dev())
        bout = torch.empty(p, dtype=torch.float32, device=dev())
        dpc.dp_clipped_sum_noise(A, G, c, C_t[l], WL.sigma, float(B), WL.seed, l, step, out, bout)
        cn = torch.empty(1, dtype=torch.float32, device=dev())
        dpc.dp_adaptive_threshold(nrm, C_t[l], WL.alpha, WL.beta, WL.sigma_l2, False, WL.seed, l, step + 1, cn)
        torch.cuda.synchronize()
        res["outs"].append(out.cpu().numpy())
        res["bias_outs"].append(bout.cpu().numpy())
        res["norms"].append(nrm.cpu().numpy())
        res["c"].append(c.cpu().numpy())
        res["C_next"].append(float(cn.item()))
    return res


def _check_step(res, ref, C_or, C_gpu, step):
    for l in range(len(SHAPES)):
        assert_norms(res["norms"][l], ref["norms"][l], "f32", what=f"step {step} norm[{l}]")
        assert_clip(res["c"][l], ref["c"][l], ref["norms"][l], C_or[l], "f32")
        S = ref["sums"][l]
        nz = WL.sigma * C_or[l] * N.weight_noise(S.shape[0], S.shape[1], WL.seed, l, step) / B
        crel = abs(C_gpu[l] - C_or[l]) / C_or[l] + 1e-7
        assert_noised(res["outs"][l], ref["outs"][l], S, nz, "f32", B, what=f"step {step} out[{l}]",
                      noise_rtol=crel)


def test_adaptive_schedule_free_running_and_teacher_forced(batches):
    """Init batch + 10 steps. Free running: each side's C_t within 1e-4 of the
    other's at every step. Teacher forced: the oracle's step t run with the
    GPU's C_t gives the GPU's C_{t+1} within 1e-4 and its outputs within the
    bars."""
    ors, gps = batches[-1]
    C_l2_or, C_or = drivers.adaptive_init(ors, WL.alpha, WL.beta, WL.sigma_l2, WL.seed)
    C_gpu = _gpu_init(gps)
    np.testing.assert_allclose(C_gpu, C_or, rtol=1e-4)
    clipped_any = unclipped_any = False
    for step in range(STEPS):
        ors, gps = batches[step]
        res = _gpu_step(gps, C_gpu, step)
        free = drivers.adaptive_step(ors, C_or, WL.sigma, WL.alpha, WL.beta, WL.sigma_l2, WL.seed, step,
                                     has_bias=True, denom=float(B))
        _check_step(res, free, C_or, C_gpu, step)
        np.testing.assert_allclose(res["C_next"], free["C_next"], rtol=1e-4, err_msg=f"free running, step {step}")
        forced = drivers.adaptive_step(ors, C_gpu, WL.sigma, WL.alpha, WL.beta, WL.sigma_l2, WL.seed, step,
                                       has_bias=True, denom=float(B))
        _check_step(res, forced, C_gpu, C_gpu, step)
        np.testing.assert_allclose(res["C_next"], forced["C_next"], rtol=1e-4, err_msg=f"teacher forced, step {step}")
        for l in range(len(SHAPES)):
            clipped_any |= bool(np.any(res["c"][l] < 1.0))
            unclipped_any |= bool(np.any(res["c"][l] == 1.0))
        C_gpu, C_or = res["C_next"], free["C_next"]
    assert clipped_any and unclipped_any     # both branches of the clip factor exercised over the schedule


def test_adaptive_schedule_resumes_bit_for_bit(batches):
    """Run the GPU schedule through all 10 steps, saving (C_t, t, seed) after
    each; restarting from the state saved at t = 4 (and at t = 9) reproduces
    every later step's norms, clip factors, noised means and bounds bit for
    bit: the schedule's state is exactly the bounds, the step index and the
    noise key."""
    _, gps0 = batches[-1]
    C = _gpu_init(gps0)
    saved, results = {}, {}
    for step in range(STEPS):
        saved[step] = (list(C), step, WL.seed)
        results[step] = _gpu_step(batches[step][1], C, step)
        C = results[step]["C_next"]
    for t0 in (4, 9):
        C_t, t, seed = saved[t0]
        assert seed == WL.seed
        for step in range(t, STEPS):
            again = _gpu_step(batches[step][1], C_t, step)
            for key in ("outs", "bias_outs", "norms", "c"):
                for l in range(len(SHAPES)):
                    a, b = again[key][l], results[step][key][l]
                    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (t0, step, key, l)
            assert np.array_equal(np.float32(again["C_next"]).view(np.uint32),
                                  np.float32(results[step]["C_next"]).view(np.uint32)), (t0, step)
            C_t = again["C_next"]
