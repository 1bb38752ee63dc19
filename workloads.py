"""Seeded synthetic workloads for the per-sample clipping hot path.

This module is shared by the tests, the benchmark and the oracle-side drivers.
It holds the five layer-set workloads (shapes, number type, clipping and noise
hyperparameters) and the seeded generators of their inputs. It contains none
of the method's arithmetic: no gradient, norm, clip factor, sum or noise is
computed here. Each generator returns the exact values the GPU path consumes
(fp32 arrays, or bf16 bit patterns as uint16); ``as_f64`` widens those exact
values for the fp64 oracle.

Input recipes (every draw from ``np.random.default_rng([base, wl, layer, step, tensor])``):

* single-linear-t1: A, G ~ N(0, 1) fp32; samples 0 and 5 have both A_i and G_i
  multiplied by 10 so that they clip.
* gpt-block-t128 and gpt2large-t1024: A ~ N(0, 1)/sqrt(d), G ~ N(0, 1)/sqrt(p)
  drawn in fp32, then rounded to bf16 (round-to-nearest-even).
* resnet18-conv-t1024: A is the unfold (kernel 3, padding 1, stride 1 or 2) of
  N(0, 1) feature maps [B, C_in, H_in, W_in], laid out [B, H_out*W_out, C_in*9]
  (the conv-as-linear equivalence of "Scalable and Efficient Training of Large
  CNNs with DP", eqs. (2.5)-(2.6)); G ~ N(0, 1) * 10**u with one u ~ U(-2, 0)
  per layer.
* mlp-b65536-adaptive: A, G ~ N(0, 1) fp32, fresh for every step; step -1 is the
  initialisation batch of the adaptive threshold.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

BASE_SEED = 0


@dataclass(frozen=True)
class Workload:
    name: str
    wl_id: int
    B: int
    layers: Tuple[Tuple[int, int, int], ...]  # (T, d, p) per layer, d = unfolded input width
    dtype: str  # "f32" or "bf16"
    C: float
    sigma: float
    has_bias: bool = False
    per_layer: bool = False  # per-layer (adaptive) clipping instead of one global norm
    adaptive: bool = False
    alpha: float = 1.1
    beta: float = 2.0
    sigma_l2: float = 2.5
    steps: int = 1
    seed: int = 0  # Philox key for the noise streams
    blocks: int = 1  # layer set repeated this many times (decoder blocks)
    conv: Tuple[Tuple[int, int, int, int], ...] = field(default_factory=tuple)  # (C_in, H_in, W_in, stride)
    description: str = ""

    @property
    def n_layers(self) -> int:
        return len(self.layers) * self.blocks

    def layer_shape(self, l: int) -> Tuple[int, int, int]:
        return self.layers[l % len(self.layers)]


WORKLOADS = {
    "single-linear-t1": Workload(
        name="single-linear-t1", wl_id=1, B=8, layers=((1, 64, 32),), dtype="f32",
        C=1.0, sigma=1.0, seed=0,
        description="one linear layer, B=8, T=1, 64->32, fp32, samples 0 and 5 scaled by 10"),
    "gpt-block-t128": Workload(
        name="gpt-block-t128", wl_id=2, B=64,
        layers=((128, 768, 2304), (128, 768, 768), (128, 768, 3072), (128, 3072, 768)),
        dtype="bf16", C=1.0, sigma=1.0, seed=0,
        description="transformer block linears qkv/out/fc1/fc2, B=64, T=128, d_model=768, bf16"),
    "resnet18-conv-t1024": Workload(
        name="resnet18-conv-t1024", wl_id=3, B=256,
        layers=((1024, 27, 64), (1024, 576, 64), (256, 576, 128), (256, 1152, 128),
                (64, 1152, 256), (64, 2304, 256), (16, 2304, 512), (16, 4608, 512)),
        conv=((3, 32, 32, 1), (64, 32, 32, 1), (64, 32, 32, 2), (128, 16, 16, 1),
              (128, 16, 16, 2), (256, 8, 8, 1), (256, 8, 8, 2), (512, 4, 4, 1)),
        dtype="f32", C=1.0, sigma=1.0, seed=0,
        description="ResNet-18 3x3 convs at 32x32 input, unfolded, B=256, fp32"),
    "mlp-b65536-adaptive": Workload(
        name="mlp-b65536-adaptive", wl_id=4, B=65536,
        layers=((1, 1024, 4096), (1, 4096, 4096), (1, 4096, 1000)),
        dtype="f32", C=1.0, sigma=0.725, has_bias=True, per_layer=True, adaptive=True,
        alpha=1.1, beta=2.0, sigma_l2=2.5, steps=10, seed=0,
        description="MLP 1024->4096->4096->1000 with biases, B=65536, T=1, fp32, "
                    "per-layer adaptive threshold over 10 steps"),
    "gpt2large-t1024": Workload(
        name="gpt2large-t1024", wl_id=5, B=32,
        layers=((1024, 1280, 3840), (1024, 1280, 1280), (1024, 1280, 5120), (1024, 5120, 1280)),
        blocks=36, dtype="bf16", C=1.0, sigma=1.0, seed=0,
        description="GPT-2-large decoder linears, 36 blocks x (qkv/out/fc1/fc2), B=32, T=1024, bf16"),
}

# The order in which the workloads are listed by the pages-derived scope table.
WORKLOAD_ORDER = ["single-linear-t1", "gpt-block-t128", "resnet18-conv-t1024",
                  "mlp-b65536-adaptive", "gpt2large-t1024"]


def rng_for(wl_id: int, layer: int, step: int, tensor: int, base: int = BASE_SEED) -> np.random.Generator:
    """Independent stream per (workload, layer, step, tensor); step -1 maps to 0."""
    return np.random.default_rng([base, wl_id, layer, step + 1, tensor])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact values of a generated tensor, widened to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def unfold3x3(x: np.ndarray, stride: int) -> np.ndarray:
    """[B, C, H, W] -> [B, H_out*W_out, C*9] (kernel 3, padding 1), channel-major
    then kernel row then kernel column, the same flattening as a conv weight
    [C_out, C_in, 3, 3]. Pure data movement (im2col)."""
    B, C, H, W = x.shape
    Ho = (H + 2 - 3) // stride + 1
    Wo = (W + 2 - 3) // stride + 1
    xp = np.zeros((B, C, H + 2, W + 2), dtype=x.dtype)
    xp[:, :, 1:H + 1, 1:W + 1] = x
    cols = np.empty((B, C, 3, 3, Ho, Wo), dtype=x.dtype)
    for kh in range(3):
        for kw in range(3):
            cols[:, :, kh, kw] = xp[:, :, kh:kh + stride * (Ho - 1) + 1:stride,
                                    kw:kw + stride * (Wo - 1) + 1:stride]
    return np.ascontiguousarray(cols.reshape(B, C * 9, Ho * Wo).transpose(0, 2, 1))


def make_layer(wl: Workload, layer: int, step: int = 0, B: int | None = None,
               shape: Tuple[int, int, int] | None = None, base: int = BASE_SEED):
    """Inputs (A, G) of one layer at one step, as the GPU consumes them.

    ``B`` and ``shape`` override the workload's batch and (T, d, p) for reduced
    test sizes; the recipe is otherwise unchanged.
    """
    B = wl.B if B is None else B
    T, d, p = wl.layer_shape(layer) if shape is None else shape
    ra = rng_for(wl.wl_id, layer, step, 0, base)
    rg = rng_for(wl.wl_id, layer, step, 1, base)
    if wl.name == "resnet18-conv-t1024" and shape is None:
        cin, hin, win, stride = wl.conv[layer]
        fmap = _normal(ra, (B, cin, hin, win))
        A = unfold3x3(fmap, stride)
        assert A.shape == (B, T, d), (A.shape, (B, T, d))
        u = rng_for(wl.wl_id, layer, step, 2, base).uniform(-2.0, 0.0)
        G = (_normal(rg, (B, T, p)) * np.float32(10.0 ** u)).astype(np.float32)
    else:
        A = _normal(ra, (B, T, d))
        G = _normal(rg, (B, T, p))
        if wl.name == "resnet18-conv-t1024":
            u = rng_for(wl.wl_id, layer, step, 2, base).uniform(-2.0, 0.0)
            G = (G * np.float32(10.0 ** u)).astype(np.float32)
    if wl.dtype == "bf16":
        A = A * np.float32(1.0 / math.sqrt(d))
        G = G * np.float32(1.0 / math.sqrt(p))
        return f32_to_bf16_bits(A), f32_to_bf16_bits(G)
    if wl.name == "single-linear-t1":
        for i in (0, 5):
            if i < B:
                A[i] *= np.float32(10.0)
                G[i] *= np.float32(10.0)
    return np.ascontiguousarray(A), np.ascontiguousarray(G)


def make_folded(wl: Workload, layer: int, step: int = 0, B: int | None = None, base: int = BASE_SEED):
    """The folded input fmap [B, C_in, H, W] and output gradients G [B, T, p]
    of one convolution layer of a workload with conv geometry: the same seeded
    values make_layer unfolds (make_layer's A is unfold3x3(fmap, stride))."""
    B = wl.B if B is None else B
    T, d, p = wl.layer_shape(layer)
    cin, hin, win, stride = wl.conv[layer]
    fmap = _normal(rng_for(wl.wl_id, layer, step, 0, base), (B, cin, hin, win))
    u = rng_for(wl.wl_id, layer, step, 2, base).uniform(-2.0, 0.0)
    G = (_normal(rng_for(wl.wl_id, layer, step, 1, base), (B, T, p)) * np.float32(10.0 ** u)).astype(np.float32)
    return np.ascontiguousarray(fmap), G


def make_vector(n: int, lo: float, hi: float, tag: int, base: int = BASE_SEED) -> np.ndarray:
    """Seeded fp32 vector in [lo, hi): free inputs of an entry point (clip factors,
    norm vectors) for tests that exercise one entry point on its own."""
    r = np.random.default_rng([base, 99, tag])
    return r.uniform(lo, hi, size=n).astype(np.float32)


def layer_list(wl: Workload) -> List[Tuple[int, int, int]]:
    return [wl.layer_shape(l) for l in range(wl.n_layers)]


def device_seed(wl_id: int, layer: int, step: int, tensor: int, base: int = BASE_SEED) -> int:
    """64-bit seed of torch's device generator for one (workload, layer, step, tensor)."""
    m = (1 << 64) - 1
    h = base & m
    for v in (wl_id, layer, step + 1, tensor):
        h = (h + (v & 0xFFFFFFFF) + 0x9E3779B97F4A7C15) & m   # splitmix64 step per field
        h = ((h ^ (h >> 30)) * 0xBF58476D1CE4E5B9) & m
        h = ((h ^ (h >> 27)) * 0x94D049BB133111EB) & m
        h ^= h >> 31
    return h >> 1


def make_layer_device(wl: Workload, layer: int, device, step: int = 0):
    """Inputs (A, G) of a layer drawn on the device with torch's generator:
    the same distributions as ``make_layer``, not the same values. bf16
    transformer layers: N(0, 1)/sqrt(d) and N(0, 1)/sqrt(p) in fp32, rounded
    to bf16 to nearest even; the fp32 MLP: N(0, 1). For layer sets too large
    to draw on the host in reasonable time (the GPT-2-large stack: 48 GB per
    pass; the B = 65536 MLP: 4.8 GB per step, fresh every step)."""
    import torch
    if wl.conv or wl.name == "single-linear-t1":
        raise ValueError("device generation covers the transformer and MLP workloads only")
    B = wl.B
    T, d, p = wl.layer_shape(layer)
    out = []
    for tensor, width in enumerate((d, p)):
        g = torch.Generator(device=device)
        g.manual_seed(device_seed(wl.wl_id, layer, step, tensor))
        x = torch.randn((B, T, width), generator=g, device=device, dtype=torch.float32)
        if wl.dtype == "bf16":
            x.mul_(1.0 / math.sqrt(width))
            out.append(x.to(torch.bfloat16))
            del x
        else:
            out.append(x)
    return out[0], out[1]
