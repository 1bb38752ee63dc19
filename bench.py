"""Benchmark of the DP-SGD per-sample clipping hot path on one MI355X.

A step is one pass of the whole path over one batch of a layer set: the
per-example norms of every layer (global clipping: their sum, from one
dp_ghost_norm_layers call; per-layer clipping: dp_ghost_norm), the clip factors
(dp_clip_factors) and the clipped, noised mean gradient of every layer
(global clipping: one dp_clipped_sum_noise_layers call; per-layer clipping:
dp_clipped_sum_noise). Inputs are seeded synthetic tensors already resident
in HBM; several copies are rotated so that consecutive steps do not hit the
256 MB Infinity Cache. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "clipped examples/sec (norm+clip+noisy sum) per layer set; % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
CACHE_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sample_gradient_clipping_layer_amd", "csrc")


def _csrc_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind, workload):
    """HBM bytes per call of the dominant entry point, from the committed
    FETCH_SIZE / WRITE_SIZE counter summary of this workload; None when there
    is none or when the kernel sources changed after the counters were taken."""
    name = {"sum": "clipped_sum", "norm": "ghost_norm"}[kind]
    path = os.path.join(PROFILES, f"hbm_traffic_{name}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("|", " ", "#")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("csrc_sha256") != _csrc_sha256() or "traffic_bytes_per_call" not in fields:
        return None
    return float(fields["traffic_bytes_per_call"])


# norm path rules: the C ABI's DP_MODE_MIXED (space, kappa = 1) and DP_MODE_TIME
MODES = {"space": 0, "time": 3}


def _algorithmic(wl, T, d, p, kind, mode=0, a_elems=None):
    """Algorithmic flops and bytes of one call on one layer (no re-reads, no
    intermediate buffers). ghost: unique Gram entries B*T(T+1)(d+p) + 2BT^2;
    explicit: 2BTdp + 2Bdp; T = 1: 2B(d+p); contraction: 2BTdp. a_elems: the
    elements of one sample's layer input when the call reads a folded conv
    input (C_in*H*W) instead of the unfolded T*d."""
    B = wl.B
    eb = 2 if wl.dtype == "bf16" else 4
    hb = 1 if wl.has_bias else 0
    inp = B * (T * d if a_elems is None else a_elems) * eb + B * T * p * eb
    if kind == "norm":
        if T == 1:
            return 2.0 * B * (d + p), inp + 4 * B
        import sample_gradient_clipping_layer_amd as dpc
        if dpc.dp_choose_path(T, d, p, mode) == dpc.PATH_EXPLICIT:
            return 2.0 * B * T * d * p + 2.0 * B * d * p, inp + 4 * B
        return float(B) * T * (T + 1) * (d + p) + 2.0 * B * T * T, inp + 4 * B
    flops = 2.0 * B * T * (d + hb) * p
    return flops, inp + 4 * (d + hb) * p + 4 * B


DEVICE_GEN_BYTES = 8 << 30
BREAKDOWN_STEPS = 50


def run_gpu(wl, steps, warmup, nstreams=1, per_layer_norms=False, per_layer_sums=False, virtual_steps=1,
            mode=0, implicit_conv=False, unfold_in_step=False):
    """Times `steps` whole steps of the workload after `warmup` untimed ones.

    Global clipping (one norm per example over all layers): every layer's
    norms accumulate into one buffer, then one clip-factor call, then every
    layer's clipped noised sum. Per-layer adaptive clipping: per layer, its
    norms, its clip factors under its current bound C_t[l], its clipped noised
    sum with noise scale sigma * C_t[l], and the update of its bound from this
    step's norms; the new bounds are read back to the host once per step
    (they are host arguments of the next step's calls), inside the timed
    region. The throughput steps run with nothing else on the stream; then
    up to BREAKDOWN_STEPS more steps run with a HIP event pair around every
    call, for the per-call durations. Returns the wall seconds and the GPU
    milliseconds (events on the stream) of the throughput steps, per-call
    event times [breakdown steps, calls], the kinds and layers of the calls,
    the number of rotated input sets and whether inputs were drawn on the
    device. implicit_conv (conv workloads): the layers are given by their
    folded inputs, one dp_conv_norm per layer into the global norm, the clip
    factors, one dp_conv_clipped_sum_noise per layer. unfold_in_step (conv
    workloads): the layers are given by their folded inputs too, and each step
    first unfolds every one with torch (F.unfold, laid out [B, T, D]) into a
    buffer, then runs the unfolded path on the buffers: what a caller holding
    only folded inputs pays for the unfolded path."""
    import torch
    import sample_gradient_clipping_layer_amd as dpc

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    shapes = W.layer_list(wl)
    B = wl.B
    eb = 2 if wl.dtype == "bf16" else 4
    set_bytes = sum(B * T * (d + p) * eb for (T, d, p) in shapes)
    n_sets = max(1, min(4, math.ceil(2 * CACHE_BYTES / set_bytes) + 1)) if set_bytes < 4 * CACHE_BYTES else 1
    on_device = set_bytes > DEVICE_GEN_BYTES
    if wl.per_layer and wl.steps > 1:
        # the adaptive schedule draws fresh inputs every step: one set per step of the
        # schedule, drawn on the device (4.8 GB each for the B = 65536 MLP)
        n_sets, on_device = wl.steps, True

    def up(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    geos = None
    folded = implicit_conv or unfold_in_step
    if folded:
        geos = [dpc.conv_geometry(cin, h, w, 3, st, 1) for (cin, h, w, st) in wl.conv]
        set_bytes = sum(B * (g.C_in * g.H * g.W + T * p) * eb for g, (T, d, p) in zip(geos, shapes))
        n_sets = max(1, min(4, math.ceil(2 * CACHE_BYTES / set_bytes) + 1))
        on_device = False
    sets = []
    for s in range(n_sets):
        layers = []
        for l in range(len(shapes)):
            if folded:
                fm, G = W.make_folded(wl, l, step=s)
                layers.append((up(fm), up(G)))
                del fm, G
            elif on_device:
                layers.append(W.make_layer_device(wl, l, dev, step=s))
            else:
                A, G = W.make_layer(wl, l, step=s)
                layers.append((up(A), up(G)))
                del A, G
        sets.append(layers)
    unf = None
    if unfold_in_step:
        # the unfolded inputs U(a) [B, T, D], rewritten every step
        unf = [torch.empty(B, T, d, dtype=sets[0][l][0].dtype, device=dev) for l, (T, d, p) in enumerate(shapes)]
    torch.cuda.synchronize()
    dt = dpc.DP_BF16 if wl.dtype == "bf16" else dpc.DP_F32
    # one workspace per distinct shape (calls on one stream run one at a time)
    ws_by_shape = {}
    for sh in set(shapes):
        nbytes = dpc.dp_workspace_bytes(dt, B, *sh, mode=mode)
        ws_by_shape[sh] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    ws = [ws_by_shape[sh] for sh in shapes]
    outs = [torch.empty(d, p, dtype=torch.float32, device=dev) for (T, d, p) in shapes]
    bouts = [torch.empty(p, dtype=torch.float32, device=dev) if wl.has_bias else None for (T, d, p) in shapes]
    stream = torch.cuda.current_stream()
    # with nstreams > 1 (global clipping, throughput steps) the clipped sums of the layers
    # go round-robin to side streams once the clip factors are ready; each layer keeps
    # its own stream, output and workspace, and the next step's clip factors wait for them
    side = [torch.cuda.Stream(device=dev) for _ in range(nstreams)] if nstreams > 1 and not wl.per_layer else []
    ws_sum = ([torch.empty_like(w) for w in ws] if side else ws)
    L = len(shapes)
    if implicit_conv:
        ws = [torch.empty(max(256, dpc.dp_conv_workspace_bytes(g, dt, B, p, wl.has_bias, mode)), dtype=torch.uint8,
                          device=dev) for g, (T, d, p) in zip(geos, shapes)]

    if wl.per_layer:
        sq = [torch.empty(B, dtype=torch.float32, device=dev) for _ in range(L)]
        c = [torch.empty(B, dtype=torch.float32, device=dev) for _ in range(L)]
        nrm = [torch.empty(B, dtype=torch.float32, device=dev) for _ in range(L)]
        C_next = torch.empty(L, dtype=torch.float32, device=dev)
        # initial bounds: one adaptive-threshold init call per layer on an initialisation batch of
        # random-noise inputs (step -1 of the generator), apart from the training sets: the first
        # bound then depends on no training data
        for l in range(L):
            A, G = W.make_layer_device(wl, l, dev, step=-1)
            dpc.dp_ghost_norm(A, G, sq[l], has_bias=wl.has_bias, mode=mode, workspace=ws[l])
            dpc.dp_clip_factors(sq[l], 3.0e38, c[l], nrm[l])
            dpc.dp_adaptive_threshold(nrm[l], 1.0, wl.alpha, wl.beta, wl.sigma_l2, True, wl.seed, l, 0,
                                      C_next[l:l + 1])
            del A, G
        C_t = [float(v) for v in C_next.tolist()]
        kinds = [(kd, l) for l in range(L) for kd in ("norm", "clip", "sum", "thr")]
    else:
        sq = torch.empty(B, dtype=torch.float32, device=dev)
        c = torch.empty(B, dtype=torch.float32, device=dev)
        # the global norm: one multi-layer call (layers sharing a kernel share a launch),
        # or one call per layer with accumulate
        per_layer_norms = per_layer_norms or L == 1  # one layer: the plain call costs less host time
        norm_kinds = [("norm", l) for l in range(L)] if per_layer_norms else [("norm", -1)]
        sum_kinds = [("sum", l) for l in range(L)] if per_layer_sums else [("sum", -1)]
        # the clip factors come out of the norm call when both calls are multi-layer
        clip_kinds = [] if not (per_layer_norms or per_layer_sums) else [("clip", -1)]
        kinds = norm_kinds + clip_kinds + sum_kinds
        if implicit_conv:
            kinds = [("norm", l) for l in range(L)] + [("clip", -1)] + [("sum", l) for l in range(L)]
        # one workspace for the multi-layer calls (they run one after another on the stream)
        ws_layers = None if implicit_conv else torch.empty(
            max(256, dpc.dp_layers_workspace_bytes(
                [(unf[l], G) for l, (_, G) in enumerate(sets[0])] if unfold_in_step else sets[0],
                has_bias=wl.has_bias, mode=mode)), dtype=torch.uint8, device=dev)
        if unfold_in_step:
            kinds = [("unfold", l) for l in range(L)] + kinds
        if virtual_steps > 1:
            # a logical batch of `virtual_steps` physical batches: per physical batch the norms, the
            # clip factors and each layer's clipped sum added to its accumulator; once per logical
            # batch each layer's noise and mean
            acc_kinds = [("sum", l) for l in range(L)] if per_layer_sums else [("sum", -1)]
            kinds = (norm_kinds + [("clip", -1)] + acc_kinds) * virtual_steps + [("noise", l) for l in range(L)]
            ws_acc_layers = torch.empty(max(256, dpc.lib().dp_layers_accumulate_workspace_bytes(
                dpc._layer_table(sets[0], wl.has_bias)[2], L, dt, B)), dtype=torch.uint8, device=dev)
            accs = [torch.empty(d, p, dtype=torch.float32, device=dev) for (T, d, p) in shapes]
            baccs = [torch.empty(p, dtype=torch.float32, device=dev) if wl.has_bias else None
                     for (T, d, p) in shapes]
            ws_acc = [torch.empty(max(256, dpc.lib().dp_accumulate_workspace_bytes(
                dt, B, T, d, p, int(wl.has_bias))), dtype=torch.uint8, device=dev) for (T, d, p) in shapes]

    ncalls = len(kinds)
    bsteps = min(steps, BREAKDOWN_STEPS)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ncalls)]
          for _ in range(bsteps)]

    sum_done = [None] * len(shapes)
    # events are recorded again every step (created once: creating them costs host time)
    ready = torch.cuda.Event()
    done_ev = [torch.cuda.Event() for _ in shapes]

    def unfold_into(l, a):
        cin, h, w, st = wl.conv[l]
        if unfold_in_step == "library":
            dpc.dp_unfold2d(a, geos[l], out=unf[l])
        else:
            unf[l].copy_(torch.nn.functional.unfold(a, 3, padding=1, stride=st).transpose(1, 2))

    def step(k, e=None):
        nonlocal C_t
        layers = sets[k % n_sets]
        j = 0
        use_side = bool(side) and e is None

        def call(fn, *args, **kw):
            nonlocal j
            if e: e[j][0].record(stream)
            fn(*args, **kw)
            if e: e[j][1].record(stream)
            j += 1

        if unfold_in_step:
            join()  # the previous step's clipped sums still read the buffers
            for l, (a, G) in enumerate(layers):
                call(unfold_into, l, a)
            layers = [(unf[l], G) for l, (a, G) in enumerate(layers)]

        if wl.per_layer:
            for l, (A, G) in enumerate(layers):
                call(dpc.dp_ghost_norm, A, G, sq[l], has_bias=wl.has_bias, mode=mode, workspace=ws[l])
                call(dpc.dp_clip_factors, sq[l], C_t[l], c[l], nrm[l])
                call(dpc.dp_clipped_sum_noise, A, G, c[l], C_t[l], wl.sigma, float(B), wl.seed, l, k, outs[l],
                     bouts[l], workspace=ws[l])
                call(dpc.dp_adaptive_threshold, nrm[l], C_t[l], wl.alpha, wl.beta, wl.sigma_l2, False, wl.seed,
                     l, k + 1, C_next[l:l + 1])
            C_t = [float(v) for v in C_next.tolist()]
            return
        if implicit_conv:
            for l, (a, G) in enumerate(layers):
                call(dpc.dp_conv_norm, a, G, geos[l], sq, has_bias=wl.has_bias, mode=mode, accumulate=l > 0,
                     workspace=ws[l])
            call(dpc.dp_clip_factors, sq, wl.C, c)
            for l, (a, G) in enumerate(layers):
                call(dpc.dp_conv_clipped_sum_noise, a, G, geos[l], c, wl.C, wl.sigma, float(B), wl.seed, l, k,
                     outs[l], bouts[l], workspace=ws[l])
            return
        if virtual_steps > 1:
            for v in range(virtual_steps):
                layers = sets[(k * virtual_steps + v) % n_sets]
                if per_layer_norms:
                    for l, (A, G) in enumerate(layers):
                        call(dpc.dp_ghost_norm, A, G, sq, has_bias=wl.has_bias, mode=mode, accumulate=l > 0, workspace=ws[l])
                else:
                    call(dpc.dp_ghost_norm_layers, layers, sq, has_bias=wl.has_bias, mode=mode, workspace=ws_layers)
                call(dpc.dp_clip_factors, sq, wl.C, c)
                if per_layer_sums:
                    for l, (A, G) in enumerate(layers):
                        call(dpc.dp_clipped_sum_accumulate, A, G, c, accs[l], bias_acc=baccs[l], accumulate=v > 0,
                             workspace=ws_acc[l])
                else:
                    call(dpc.dp_clipped_sum_accumulate_layers, layers, c, accs,
                         bias_accs=baccs if wl.has_bias else None, has_bias=wl.has_bias, accumulate=v > 0,
                         workspace=ws_acc_layers)
            for l in range(L):
                call(dpc.dp_noise_mean, accs[l], wl.C, wl.sigma, float(B * virtual_steps), wl.seed, l, k, outs[l],
                     bias_acc=baccs[l], bias_out=bouts[l])
            return
        if per_layer_norms:
            for l, (A, G) in enumerate(layers):
                call(dpc.dp_ghost_norm, A, G, sq, has_bias=wl.has_bias, mode=mode, accumulate=l > 0, workspace=ws[l])
        elif per_layer_sums:
            call(dpc.dp_ghost_norm_layers, layers, sq, has_bias=wl.has_bias, mode=mode, workspace=ws_layers)
        else:  # the clip factors come out of the norm kernels
            call(dpc.dp_ghost_norm_clip_layers, layers, sq, wl.C, c, has_bias=wl.has_bias, mode=mode,
                 workspace=ws_layers)
        if not per_layer_sums:
            if per_layer_norms:
                call(dpc.dp_clip_factors, sq, wl.C, c)
            call(dpc.dp_clipped_sum_noise_layers, layers, c, wl.C, wl.sigma, float(B), wl.seed, k, outs,
                 bias_outs=bouts if wl.has_bias else None, has_bias=wl.has_bias, workspace=ws_layers)
            return
        if not use_side:
            join()
            call(dpc.dp_clip_factors, sq, wl.C, c)
            for l, (A, G) in enumerate(layers):
                call(dpc.dp_clipped_sum_noise, A, G, c, wl.C, wl.sigma, float(B), wl.seed, l, k, outs[l], bouts[l],
                     workspace=ws[l])
            return
        join()  # the previous step's sums still read c
        dpc.dp_clip_factors(sq, wl.C, c)
        ready.record(stream)
        for l, (A, G) in enumerate(layers):
            s_l = side[l % len(side)]
            s_l.wait_event(ready)
            dpc.dp_clipped_sum_noise(A, G, c, wl.C, wl.sigma, float(B), wl.seed, l, k, outs[l], bouts[l],
                                     workspace=ws_sum[l], stream=s_l)
            done_ev[l].record(s_l)
            sum_done[l] = done_ev[l]

    def join():
        for l, ev_l in enumerate(sum_done):
            if ev_l is not None:
                stream.wait_event(ev_l)
                sum_done[l] = None

    if not wl.per_layer:
        C_t = None
    for k in range(warmup):
        step(k)
    # throughput: `steps` steps with nothing else on the stream
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    for k in range(steps):
        step(warmup + k)
    join()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = g0.elapsed_time(g1)
    # per-call durations: further steps with an event pair around every call
    # (the markers cost a little GPU time, so these steps are timed apart)
    for k in range(bsteps):
        step(warmup + steps + k, ev[k])
    torch.cuda.synchronize()
    call_ms = np.array([[a.elapsed_time(b) for (a, b) in ev[k]] for k in range(bsteps)])  # [bsteps, ncalls]
    for o in outs:
        assert torch.isfinite(o).all().item(), "non-finite output"
    if wl.per_layer:
        assert all(math.isfinite(v) and v > 0 for v in C_t), f"adaptive bounds {C_t}"
    return wall, gpu_ms, call_ms, shapes, kinds, n_sets, on_device, geos


def cpu_baseline(wl, budget_s=12.0, step_s=3.0, max_step_s=25.0):
    """The fp64 oracle as it stands, timed on the host cores on a bounded
    sample of the same workload: whole steps (norms, clip factors, clipped
    sums, noise; with per-layer clipping also the bound updates) over all
    layers, or over the first decoder block when the set repeats blocks, on
    the first b examples. b is calibrated so that one step takes about
    `step_s` seconds and the per-example work is at least three times the
    step's fixed cost (its noise draw), within `max_step_s` per step. The
    oracle's cost is linear in the examples and, for a repeated block, in the
    blocks, so the rate is scaled to the whole set; the fixed cost is amortised
    over b examples, not the full batch, which makes the reported rate an
    underestimate when b is smaller than the batch."""
    from threadpoolctl import threadpool_info
    from oracle import drivers

    nl = len(wl.layers) if wl.blocks > 1 else wl.n_layers
    scale = nl / wl.n_layers

    def sample(b):
        layers = []
        for l in range(nl):
            A, G = W.make_layer(wl, l, step=0, B=b)
            layers.append((W.as_f64(A, wl.dtype), W.as_f64(G, wl.dtype)))
        return layers

    def one_step(layers, n):
        if wl.per_layer:
            drivers.adaptive_step(layers, [wl.C] * len(layers), wl.sigma, wl.alpha, wl.beta, wl.sigma_l2,
                                  wl.seed, step=n, has_bias=wl.has_bias, denom=float(wl.B))
        else:
            drivers.global_clip_step(layers, wl.C, wl.sigma, wl.seed, step=n, has_bias=wl.has_bias,
                                     denom=float(wl.B))

    def timed(b):
        layers = sample(b)
        t0 = time.perf_counter()
        one_step(layers, 0)
        return layers, time.perf_counter() - t0

    # two calibration steps give the per-example and the fixed (noise) cost of a step
    b0 = min(wl.B, 2)
    layers, t0 = timed(b0)
    b = b0
    if b0 < wl.B:
        b1 = min(wl.B, 4 * b0)
        layers, t1 = timed(b1)
        slope = max((t1 - t0) / (b1 - b0), 1e-9)
        fixed = max(t0 - slope * b0, 0.0)
        # enough examples for one step of about step_s, and for the per-example work to be
        # at least three times the fixed cost, within max_step_s per step
        want = max((step_s - fixed) / slope, 3.0 * fixed / slope)
        b = int(min(wl.B, max(b1, min(want, (max_step_s - fixed) / slope))))
        layers = sample(b) if b != b1 else layers
    n = 0
    t0 = time.perf_counter()
    while True:
        one_step(layers, n)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    host_cores = len(os.sched_getaffinity(0))
    what = f"first {nl} of {wl.n_layers} layers" if nl < wl.n_layers else f"all {nl} layers"
    # cores: the threads the oracle actually ran on (its BLAS pool; the rest of it is one Python thread)
    return {"value": b * n / dt * scale, "unit": "examples/s", "cores": int(min(threads, host_cores)),
            "host_cores": int(host_cores), "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{n} whole step(s) of {wl.name} on {b} of {wl.B} examples, {what} "
                      f"(fp64 numpy, materialised per-example gradients), {dt:.1f} s"
                      + (f"; rate scaled by {nl}/{wl.n_layers} layers" if nl < wl.n_layers else "")}


COPY_PROBE_BYTES = 256 << 20


def copy_probe(reps=5):
    """A plain copy of known size: reads and writes COPY_PROBE_BYTES per
    launch. Profiling counters of this launch give the factor between a
    counter's reading and the bytes that really moved."""
    import torch
    src = torch.full((COPY_PROBE_BYTES // 4,), 1.5, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert dst[-1].item() == 1.5
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": reps}), flush=True)


def noise_fill(reps=3):
    """The noise and the mean alone (dp_noise_mean, k_noise_mean) over the
    outputs of every layer of the GPT-2-large stack: 144 layers, 708 M fp32
    elements, out-of-place (read acc, write out: 8 bytes per element). HIP
    events around each pass; prints one JSON line with the rate."""
    import torch
    import sample_gradient_clipping_layer_amd as dpc
    wl = W.WORKLOADS["gpt2large-t1024"]
    dev = torch.device("cuda", 0)
    shapes = [(d, p) for (T, d, p) in wl.layers]
    accs = [torch.randn(d, p, device=dev) for (d, p) in shapes]
    outs = [torch.empty_like(a) for a in accs]
    elems = wl.blocks * sum(d * p for (d, p) in shapes)

    def one_pass(step):
        for b in range(wl.blocks):
            for k, (d, p) in enumerate(shapes):
                dpc.dp_noise_mean(accs[k], wl.C, wl.sigma, float(wl.B), wl.seed, 4 * b + k, step, outs[k])

    one_pass(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        one_pass(r + 1)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    for o in outs:
        assert torch.isfinite(o).all().item()
    print(json.dumps({"noise_fill_elements": elems, "launches_per_pass": wl.blocks * len(shapes),
                      "ms_per_pass": round(ms, 4), "algorithmic_bytes_per_pass": 8 * elems,
                      "GB_per_s": round(8 * elems / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # default: the largest configuration that fits one GPU (GPT-2-large-shaped decoder stack)
    ap.add_argument("--workload", default="gpt2large-t1024", choices=W.WORKLOAD_ORDER)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="print per-call times to stderr")
    ap.add_argument("--per-layer-norms", action="store_true",
                    help="global clipping: one dp_ghost_norm call per layer instead of one multi-layer call")
    ap.add_argument("--path-rule", choices=("space", "time"), default="space",
                    help="norm path per layer: the space rule p*d < T^2 (default) or the time rule "
                         "(DP_MODE_TIME: the smaller per-sample matrix-core work)")
    ap.add_argument("--virtual-steps", type=int, default=1,
                    help="global clipping: each step is a logical batch of this many physical batches "
                         "(gradient accumulation; noise and mean once per logical batch)")
    ap.add_argument("--per-layer-sums", action="store_true",
                    help="global clipping: one dp_clipped_sum_noise call per layer (on --streams side streams) "
                         "instead of one multi-layer call")
    ap.add_argument("--streams", type=int, default=None,
                    help="side streams for the layers' clipped sums in the throughput steps (global clipping); "
                         "default 3 for layer sets of at most 8 layers, else 1")
    ap.add_argument("--implicit-conv", action="store_true",
                    help="conv workloads: pass each layer's folded input (dp_conv_* calls) instead of its unfolding")
    ap.add_argument("--unfold-in-step", nargs="?", const="torch", default=None, choices=("torch", "library"),
                    help="conv workloads: the layers given by their folded inputs, unfolded inside every step "
                         "(by torch's F.unfold, or by the library's dp_unfold2d) before the unfolded path runs "
                         "(the alternatives to --implicit-conv)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (HBM counter calibration)")
    ap.add_argument("--noise-fill", action="store_true",
                    help="only run the noise and the mean (dp_noise_mean) over all 144 GPT-2-large layer outputs")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the clipping path on a single MI355X "
              "and has no multi-GPU path. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if a.copy_probe:
        copy_probe()
        return
    if a.noise_fill:
        noise_fill()
        return
    wl = W.WORKLOADS[a.workload]
    # the multi-layer clipped-sum call shares launches among bf16 layers without bias whose T is a
    # multiple of 64 and d, p multiples of 8; a set with none of those runs per-layer calls on side
    # streams instead (the library runs them one after another within one call)
    shapes0 = [wl.layer_shape(l) for l in range(wl.n_layers)]
    groupable = (wl.dtype == "bf16" and not wl.has_bias and
                 sum(1 for (T, d, p) in shapes0 if T % 64 == 0 and d % 8 == 0 and p % 8 == 0) >= 2)
    per_layer_sums = a.per_layer_sums or not groupable
    if per_layer_sums and not wl.per_layer:
        nstreams = a.streams if a.streams is not None else (3 if 2 <= wl.n_layers <= 8 else 1)
    else:
        nstreams = 1
    if a.virtual_steps > 1 and wl.per_layer:
        print("--virtual-steps applies to global clipping workloads", file=sys.stderr)
        sys.exit(2)
    if a.virtual_steps > 1:
        nstreams = 1
    if a.implicit_conv:
        if not wl.conv or a.virtual_steps > 1 or a.per_layer_norms or a.per_layer_sums:
            print("--implicit-conv applies to conv workloads, alone", file=sys.stderr)
            sys.exit(2)
        nstreams, per_layer_sums = 1, True
    if a.unfold_in_step and (not wl.conv or a.implicit_conv or a.virtual_steps > 1):
        print("--unfold-in-step applies to conv workloads, without --implicit-conv or --virtual-steps",
              file=sys.stderr)
        sys.exit(2)
    wall, gpu_ms, call_ms, shapes, kinds, n_sets, on_device, geos = run_gpu(
        wl, a.steps, a.warmup, nstreams, a.per_layer_norms, per_layer_sums, a.virtual_steps, MODES[a.path_rule],
        a.implicit_conv, a.unfold_in_step)
    L = len(shapes)
    ms_per_step = 1e3 * wall / a.steps
    value = wl.B * a.virtual_steps * a.steps / wall

    # dominant entry point by total event time: the norm calls or the clipped-sum calls
    mean_ms = call_ms.mean(axis=0)
    by_kind = {}
    for j, (kd, l) in enumerate(kinds):
        by_kind[kd] = by_kind.get(kd, 0.0) + mean_ms[j]
    dom = max(("norm", "sum"), key=lambda k: by_kind[k])
    flops = byts = t_ms = 0.0
    ndom = 0
    for j, (kd, l) in enumerate(kinds):
        if kd != dom:
            continue
        for ll in (range(L) if l < 0 else (l,)):  # l < 0: one call over all layers
            T, d, p = shapes[ll]
            a_el = None if geos is None else geos[ll].C_in * geos[ll].H * geos[ll].W
            f, b = _algorithmic(wl, T, d, p, kd, MODES[a.path_rule], a_el)
            flops += f
            byts += b
        t_ms += mean_ms[j]
        ndom += 1
    if dom == "sum" or (flops / byts > (PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS)
                        / PEAK_HBM_GBS * 1e3):
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = flops / (t_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = byts / (t_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    traffic = measured_traffic(dom, wl.name + ("-implicit-conv" if a.implicit_conv else ""))
    roof["traffic"] = None if traffic is None else round(traffic)
    roof["algorithmic_bytes_per_call"] = round(byts / ndom)
    roof["kernel"] = ("dp_ghost_norm[_layers]: k_ghost_tiles / k_ghost_wide / k_explicit_tiles / k_norm_t1"
                      if dom == "norm"
                      else "dp_clipped_sum_noise[_layers]: k_contract_dl (+ k_reduce_noise_group / _vec for split tiles), "
                           "k_contract_dl32 / k_contract_tiles (+ k_reduce_noise[_vec|_wide] when K is split)")
    if a.implicit_conv:
        roof["kernel"] = ("dp_conv_norm: k_ghost_tiles / k_explicit_tiles on folded inputs" if dom == "norm" else
                          "dp_conv_clipped_sum_noise: k_contract_tiles on folded inputs (+ k_reduce_noise[_vec|_wide])")
    roof["avg_call_us"] = round(1e3 * t_ms / ndom, 2)
    if a.breakdown:
        for (kd, l), m in zip(kinds, mean_ms):
            nm = kd if l < 0 else f"{kd}[{l}]"
            print(f"{nm:10s} {m * 1e3:9.2f} us", file=sys.stderr)
        for kd, m in by_kind.items():
            print(f"total {kd:5s} {m * 1e3:9.2f} us", file=sys.stderr)
    cfg = {"workload": wl.name, "global_batch": wl.B, "seq_len": shapes[0][0],
           "layers": [list(s) for s in shapes] if L <= 8 else f"{wl.blocks} x {[list(s) for s in wl.layers]}",
           "parallelism": "single-gpu", "input_sets_rotated": n_sets,
           "clipping": "per-layer adaptive" if wl.per_layer else "global",
           "norm_call": "per-layer" if (wl.per_layer or a.per_layer_norms or L == 1) else "multi-layer",
           "sum_call": ("per-layer" if (wl.per_layer or per_layer_sums) else "multi-layer"),
           "sum_streams": nstreams, "path_rule": a.path_rule}
    if a.implicit_conv:
        cfg["conv_input"] = "folded [B, C_in, H, W]; unfolded rows formed in the kernels"
        cfg["norm_call"] = cfg["sum_call"] = "per-layer (dp_conv_*)"
    if a.unfold_in_step:
        cfg["conv_input"] = ("folded [B, C_in, H, W], unfolded inside every step to [B, T, D] by "
                             + ("torch's F.unfold" if a.unfold_in_step == "torch" else "the library's dp_unfold2d"))
    if a.virtual_steps > 1:
        cfg["virtual_steps"] = a.virtual_steps
        cfg["logical_batch"] = wl.B * a.virtual_steps
    if on_device:
        cfg["inputs"] = "drawn on the device (torch generator), distinct for every layer"
    if wl.per_layer and wl.steps > 1:
        cfg["inputs"] = (f"drawn on the device (torch generator): fresh A and G for each of the {wl.steps} "
                         f"steps of the adaptive schedule (step k uses set k mod {n_sets}); the initial bounds "
                         f"from a separate random-noise batch")
        cfg["schedule_steps"] = wl.steps
    # layer-GB/s: the algorithmic bytes of a step's calls (per layer and physical batch: A and G read by the
    # norm pass and again by the clipped sum, 4 bytes per norm, the d x p fp32 output) over the step time
    step_bytes = 0.0
    for ll, (T, d, p) in enumerate(shapes):
        a_el = None if geos is None else geos[ll].C_in * geos[ll].H * geos[ll].W
        step_bytes += _algorithmic(wl, T, d, p, "norm", MODES[a.path_rule], a_el)[1]
        step_bytes += _algorithmic(wl, T, d, p, "sum", MODES[a.path_rule], a_el)[1]
    step_bytes *= max(1, a.virtual_steps)
    layer_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "examples/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic", "config": cfg,
        "roofline": roof,
        "gpu_ms_per_step": round(gpu_ms / a.steps, 4),
        "calls_ms_per_step": round(float(call_ms.sum(axis=1).mean()), 4),
        "breakdown_steps": int(call_ms.shape[0]),
        "layer_GB_per_s": round(layer_gbs, 1),
        "layer_GB_per_s_frac_hbm": round(layer_gbs / PEAK_HBM_GBS, 4),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
