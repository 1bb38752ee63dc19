"""Whole layer-set steps composed from the oracle definitions (test infrastructure only).

A step follows the order of the DP-SGD update with per-sample clipping
("Scaling up DP Deep Learning with Fast Per-Example Gradient Clipping", the
clipped mean plus Gaussian noise; "Scalable and Efficient Training of Large
CNNs with DP", eq. (2.1) and Appendix C.6, mixed ghost clipping = norms, then
the weighted gradient): per-layer norms -> per-example clip factors ->
clipped sum per layer -> noised mean per layer. With per-layer clipping
("Three Tools for Practical DP", layers clipped independently) each layer has
its own norms, factors and bound, and the adaptive bound is updated after the
step from that step's norms.

Inputs are lists of (A, G) fp64 arrays (exact input values). Noise streams:
weight noise of layer l at step t is weight_noise(d, p, seed, l, t); bias
noise is normals(p, seed, l, 1, t); the noise of the adaptive bound C_t of
layer l is threshold_normal(seed, l, t).
"""
from __future__ import annotations

import numpy as np

from . import definitions as D
from . import noise as N


def global_clip_step(layers, C, sigma, seed, step=0, has_bias=False, denom=None,
                     layer_ids=None):
    """One step with one global per-example norm over all given layers."""
    B = layers[0][0].shape[0]
    denom = float(B) if denom is None else float(denom)
    layer_ids = list(range(len(layers))) if layer_ids is None else list(layer_ids)
    sq = [D.layer_sqnorms(A, G, has_bias) for A, G in layers]
    norms = D.total_norms(sq)
    c = D.clip_factors(norms, C)
    outs, bouts, sums = [], [], []
    for lid, (A, G) in zip(layer_ids, layers):
        d, p = A.shape[2], G.shape[2]
        S, Sb = D.clipped_sum(A, G, c, has_bias)
        z = N.weight_noise(d, p, seed, lid, step)
        outs.append(D.noised_mean(S, z, C, sigma, denom))
        sums.append(S)
        if has_bias:
            zb = N.normals(p, seed, lid, 1, step)
            bouts.append(D.noised_mean(Sb, zb, C, sigma, denom))
        else:
            bouts.append(None)
    return dict(sqnorms=sq, norms=norms, c=c, sums=sums, outs=outs, bias_outs=bouts)


def adaptive_init(layers, alpha, beta, sigma_l2, seed, has_bias=True):
    """Initial per-layer bounds from one batch of random-noise inputs
    ("Three Tools for Practical DP": C_l2,0 is the mean l2 norm of one
    iteration on random noise). Returns lists (C_l2_0, C_0)."""
    C_l2, C_0 = [], []
    for lid, (A, G) in enumerate(layers):
        norms = np.sqrt(D.layer_sqnorms(A, G, has_bias))
        z = N.threshold_normal(seed, lid, 0)
        cl2, ct = D.adaptive_threshold(norms, 0.0, alpha, beta, sigma_l2, True, z)
        C_l2.append(cl2)
        C_0.append(ct)
    return C_l2, C_0


def adaptive_step(layers, C_t, sigma, alpha, beta, sigma_l2, seed, step, has_bias=True,
                  denom=None):
    """Step t of per-layer adaptive clipping: clip layer l with its bound
    C_t[l], add noise N(0, sigma^2 C_t[l]^2), then produce C_{t+1}[l] from this
    step's norms with C_l2 = beta * C_t[l]."""
    B = layers[0][0].shape[0]
    denom = float(B) if denom is None else float(denom)
    res = dict(norms=[], c=[], outs=[], bias_outs=[], C_l2=[], C_next=[], sums=[])
    for lid, (A, G) in enumerate(layers):
        d, p = A.shape[2], G.shape[2]
        norms = np.sqrt(D.layer_sqnorms(A, G, has_bias))
        c = D.clip_factors(norms, C_t[lid])
        S, Sb = D.clipped_sum(A, G, c, has_bias)
        z = N.weight_noise(d, p, seed, lid, step)
        res["outs"].append(D.noised_mean(S, z, C_t[lid], sigma, denom))
        res["sums"].append(S)
        if has_bias:
            zb = N.normals(p, seed, lid, 1, step)
            res["bias_outs"].append(D.noised_mean(Sb, zb, C_t[lid], sigma, denom))
        else:
            res["bias_outs"].append(None)
        zt = N.threshold_normal(seed, lid, step + 1)
        cl2, cn = D.adaptive_threshold(norms, C_t[lid], alpha, beta, sigma_l2, False, zt)
        res["norms"].append(norms)
        res["c"].append(c)
        res["C_l2"].append(cl2)
        res["C_next"].append(cn)
    return res


def virtual_step(batches, cs, C, sigma, seed, layer_id=0, step=0, has_bias=False):
    """One layer's update over a logical batch fed as several physical batches
    ([SEDP] Performance section: the physical batch is what is fed to the GPU
    at one time, the logical batch what one update covers, with one
    back-propagation per physical batch before the update; App. E, the virtual
    step). Each physical batch's samples carry their own clip factors cs[k];
    the clipped sums of the physical batches add up and the noise and the mean
    over the logical batch (denom = its size) are applied once."""
    acc = bacc = None
    n = 0
    for (A, G), c in zip(batches, cs):
        S, Sb = D.clipped_sum(A, G, c, has_bias)
        acc = S if acc is None else acc + S
        if has_bias:
            bacc = Sb if bacc is None else bacc + Sb
        n += A.shape[0]
    d, p = acc.shape
    out = D.noised_mean(acc, N.weight_noise(d, p, seed, layer_id, step), C, sigma, n)
    bout = D.noised_mean(bacc, N.normals(p, seed, layer_id, 1, step), C, sigma, n) if has_bias else None
    return dict(sum=acc, bias_sum=bacc, out=out, bias_out=bout, denom=float(n))
