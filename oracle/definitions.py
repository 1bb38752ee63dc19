"""fp64 definitions of the per-sample clipping hot path (oracle; test infrastructure only).

Every quantity is computed from its plain definition, materialising the
per-example gradients, with no ghost identity, fusion or reordering. Inputs
are the exact values of the layer inputs, widened to fp64.

Notation (one trainable layer): A[B, T, d] holds the layer inputs a_i (for a
convolution, the unfolded input U(a_i) with d = C_in*k_H*k_W and
T = H_out*W_out), G[B, T, p] the output gradients dL/ds_i (for a convolution,
the flattened F^-1(dL/ds_i)).

Sources (page title; place on the page):
  [FPC]  "Scaling up Differentially Private Deep Learning with Fast Per-Example
         Gradient Clipping": the clip_c definition and the clipped mean of DP-SGD
         (background on DP deep learning); eq. (6) and Algorithm 2 (per-example
         gradient of a fully connected layer as an outer product, batched);
         the per-example bias gradient (the equation following Algorithm 2);
         Algorithm 3 (convolution via im2col + GEMM); the re-weighted loss
         whose gradient is exactly the clipped sum.
  [TTP]  "Three Tools for Practical Differential Privacy": the adaptive
         per-layer clipping bound C_t^l, its clip(||y||) and C_l2 schedule.
  [SEDP] "Scalable and Efficient Training of Large Convolutional Neural
         Networks with Differential Privacy": eq. (2.1) privatised gradient,
         eq. (2.4) per-sample gradient, eqs. (2.5)-(2.7) conv-as-linear and
         the ghost norm, Sec. 4 layerwise decision (4.1) with the space terms
         2T^2 vs pD of Appendix F, Appendix C complexity counts.
  [DDP]  "Privacy-Preserving Deep Learning: A Deep Dive into DP-SGD": "The
         Mathematical Foundation" (clipping g / max(1, ||g||/C), noisy aggregate).
"""
from __future__ import annotations

import numpy as np

# Path identifiers, shared meaning with the library's path report.
PATH_GHOST = 1
PATH_EXPLICIT = 2
PATH_T1 = 3

MODE_MIXED = 0
MODE_GHOST = 1
MODE_EXPLICIT = 2
MODE_TIME = 3


def per_example_weight_grad(A_i: np.ndarray, G_i: np.ndarray) -> np.ndarray:
    """g_i = dL_i/dW = sum_t a_i[t] (x) g_i[t] = A_i^T G_i, shape [d, p].

    [FPC] eq. (6) / Algorithm 2 (outer product per example; with T > 1 rows the
    outer products of all rows add up, which is [FPC] Algorithm 3's GEMM on the
    im2col matrix); [SEDP] eqs. (2.4), (2.6).
    """
    A_i = np.asarray(A_i, dtype=np.float64)
    G_i = np.asarray(G_i, dtype=np.float64)
    return A_i.T @ G_i


def per_example_bias_grad(G_i: np.ndarray) -> np.ndarray:
    """b_i = dL_i/db = sum_t G_i[t, :], shape [p] ([FPC], bias gradient)."""
    return np.asarray(G_i, dtype=np.float64).sum(axis=0)


def layer_sqnorms(A: np.ndarray, G: np.ndarray, has_bias: bool = False) -> np.ndarray:
    """Per-example squared Frobenius norm of one layer's gradient (weight, plus
    bias when the layer has one), from the materialised per-example gradients.
    [SEDP] the per-sample norm entering C_i; [DDP] ||g_t(x_i)||_2."""
    B = A.shape[0]
    out = np.zeros(B, dtype=np.float64)
    for i in range(B):
        g = per_example_weight_grad(A[i], G[i])
        s = float(np.sum(g * g))
        if has_bias:
            b = per_example_bias_grad(G[i])
            s += float(np.sum(b * b))
        out[i] = s
    return out


def total_norms(sqnorms_per_layer) -> np.ndarray:
    """Global per-example norm ||g_i|| over all layers: sqrt(sum_l ||g_{i,l}||^2)."""
    total = np.zeros_like(np.asarray(sqnorms_per_layer[0], dtype=np.float64))
    for s in sqnorms_per_layer:
        total = total + np.asarray(s, dtype=np.float64)
    return np.sqrt(total)


def choose_path(T: int, d: int, p: int, mode: int = MODE_MIXED, kappa: int = 1) -> int:
    """Layerwise decision between the ghost norm and per-sample instantiation.

    [SEDP] Sec. 4, rule (4.1) compares the space of the ghost norm (2T^2,
    Appendix F) with that of instantiation (pD). The printed rule is lost in
    the extract; the reading taken here is: instantiate (explicit) when
    p*d < kappa*T^2, otherwise ghost; kappa = 1 is the default, kappa = 2
    reproduces the 2T^2-vs-pD comparison; a tie goes to ghost. T = 1 uses the
    closed form of the ghost norm (a 1x1 Gram). mode GHOST/EXPLICIT forces
    the path ([SEDP] Appendix E: 'ghost' and 'ghost-mixed' modes).

    mode TIME decides by time instead of space: per sample, the matrix-core
    work of instantiation, 2Tdp + 2dp ([SEDP] Appendix C: the per-sample
    gradient product and its squared norm), against that of the ghost norm
    with its Grams' unique entries, T(T+1)(d+p) + 2T^2 (both Grams' s <= t
    entries, then the Frobenius product); explicit when strictly smaller,
    a tie goes to ghost.
    """
    if mode == MODE_EXPLICIT:
        return PATH_EXPLICIT
    if T == 1:
        return PATH_T1
    if mode == MODE_GHOST:
        return PATH_GHOST
    if mode == MODE_TIME:
        explicit = 2 * T * d * p + 2 * d * p
        ghost = T * (T + 1) * (d + p) + 2 * T * T
        return PATH_EXPLICIT if explicit < ghost else PATH_GHOST
    return PATH_EXPLICIT if p * d < kappa * T * T else PATH_GHOST


def clip_factors(norms: np.ndarray, C: float) -> np.ndarray:
    """c_i such that clip_C(g_i) = c_i * g_i.

    [FPC] clip_c(z) = z when ||z|| <= c, else c * z / ||z||; [DDP] g / max(1, ||g||/C);
    [SEDP] Appendix C: C_i = min(R/||g_i||, 1). A norm equal to C is not clipped.
    """
    norms = np.asarray(norms, dtype=np.float64)
    c = np.ones_like(norms)
    over = norms > C
    c[over] = C / norms[over]
    return c


def clipped_sum(A: np.ndarray, G: np.ndarray, c: np.ndarray, has_bias: bool = False):
    """S = sum_i c_i g_i (weight, [d, p]) and S_b = sum_i c_i b_i (bias, [p]),
    accumulated example by example in index order.

    [FPC] the sum of clipped per-example gradients, equal to the gradient of the
    re-weighted loss sum_i c_i L_i; [SEDP] eq. (2.1) weighted gradient
    sum_i C_i g_i.
    """
    B, T, d = A.shape
    p = G.shape[2]
    S = np.zeros((d, p), dtype=np.float64)
    Sb = np.zeros(p, dtype=np.float64)
    for i in range(B):
        S += float(c[i]) * per_example_weight_grad(A[i], G[i])
        if has_bias:
            Sb += float(c[i]) * per_example_bias_grad(G[i])
    return S, (Sb if has_bias else None)


def noised_mean(S: np.ndarray, z: np.ndarray, C: float, sigma: float, denom: float) -> np.ndarray:
    """(S + N(0, sigma^2 C^2 I)) / denom with the normal draw z given, in fp64.

    [FPC] Gaussian noise is added to the clipped sum before the update; [SEDP]
    eq. (2.1); [DDP] noisy aggregation. The noise sits inside the 1/B mean (the
    reading taken where [DDP] prints it outside).
    """
    return (np.asarray(S, dtype=np.float64) + float(sigma) * float(C) * np.asarray(z, dtype=np.float64)) / float(denom)


def noised_mean_f32(S32: np.ndarray, z32: np.ndarray, C: float, sigma: float, denom: float) -> np.ndarray:
    """The same quantity evaluated as the fp32 operation sequence
    out = (S + (sigma*C)*z) * (1/denom), every operation rounded to fp32 (the
    reciprocal of denom rounded once; exact when denom is a power of two).
    Used for the bit-exact noise check, where S is exactly zero."""
    f = np.float32
    sc = f(sigma) * f(C)
    inv = f(1.0) / f(denom)
    n = (sc * np.asarray(z32, dtype=np.float32)).astype(np.float32)
    o = (np.asarray(S32, dtype=np.float32) + n).astype(np.float32)
    return (o * inv).astype(np.float32)


def adaptive_clip_norm(norm: np.ndarray, C_l2: float) -> np.ndarray:
    """[TTP] clip(||y||) = ||y|| / max(1, ||y|| / C_l2)."""
    norm = np.asarray(norm, dtype=np.float64)
    return norm / np.maximum(1.0, norm / float(C_l2))


def adaptive_threshold(norms: np.ndarray, C_prev: float, alpha: float, beta: float,
                       sigma_l2: float, init: bool, z: float):
    """One update of the adaptive per-layer bound of [TTP]:

        C_l2 = beta * C_prev            (init: the mean l2 norm of the batch)
        C_t  = alpha * |L|^-1 * (sum_i clip(||g_i||) + N(0, sigma_l2^2 C_l2^2))

    with the normal draw z given and |L| the batch size. Returns (C_l2, C_t).
    The noise term is divided by |L| as the formula on the page is written.
    """
    norms = np.asarray(norms, dtype=np.float64)
    B = norms.shape[0]
    if init:
        C_l2 = float(np.mean(norms))
    else:
        C_l2 = float(beta) * float(C_prev)
    s = float(np.sum(adaptive_clip_norm(norms, C_l2)))
    C_t = float(alpha) / B * (s + float(sigma_l2) * C_l2 * float(z))
    return C_l2, C_t


def clipped_sum_entries(A: np.ndarray, G: np.ndarray, c: np.ndarray, rows, cols) -> np.ndarray:
    """Selected entries S[m, n] of the clipped sum, each from its definition
    sum_i c_i (A_i^T G_i)[m, n] = sum_i c_i sum_t A_i[t, m] G_i[t, n]
    ([FPC] re-weighted sum; [SEDP] eq. (2.1)). For full-size checks where the
    whole [d, p] sum is too large to materialise per example."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    c = np.asarray(c, dtype=np.float64)
    out = np.zeros(rows.shape[0], dtype=np.float64)
    for k in range(rows.shape[0]):
        g_mn = np.sum(np.asarray(A[:, :, rows[k]], dtype=np.float64) * np.asarray(G[:, :, cols[k]], dtype=np.float64),
                      axis=1)  # per-example gradient entry [B]
        out[k] = float(np.dot(c, g_mn))
    return out


def unfold2d(a: np.ndarray, kernel, stride=(1, 1), padding=(0, 0), dilation=(1, 1)) -> np.ndarray:
    """U(a): the unfolded input of a 2-D convolution, [B, T, d] in fp64 from the
    folded input a [B, C_in, H, W].

    [SEDP] Sec. 2.2 (convolution as a linear layer on U(a_i), eqs. (2.5)-(2.6));
    [FPC] Algorithm 3 (the im2col matrix). Row t = ho*W_out + wo is the receptive
    field of output position (ho, wo); its column f = (ci*kH + i)*kW + j holds
    the input at channel ci, row ho*s_h - p_h + i*dl_h, column
    wo*s_w - p_w + j*dl_w, and 0 where that lies in the zero padding. Written as
    loops over the kernel offsets: each offset (i, j) fills one column per
    channel with a strided slice of the zero-padded input.
    """
    a = np.asarray(a, dtype=np.float64)
    B, Cin, H, W = a.shape
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = kernel, stride, padding, dilation
    Ho = (H + 2 * ph - dh * (kh - 1) - 1) // sh + 1
    Wo = (W + 2 * pw - dw * (kw - 1) - 1) // sw + 1
    if Ho < 1 or Wo < 1:
        raise ValueError("the kernel does not fit the padded input")
    padded = np.zeros((B, Cin, H + 2 * ph, W + 2 * pw), dtype=np.float64)
    padded[:, :, ph:ph + H, pw:pw + W] = a
    U = np.zeros((B, Ho, Wo, Cin, kh, kw), dtype=np.float64)
    for i in range(kh):
        for j in range(kw):
            y0, x0 = i * dh, j * dw  # padded coordinates of output (0, 0)'s tap (i, j)
            U[:, :, :, :, i, j] = padded[:, :, y0:y0 + sh * (Ho - 1) + 1:sh,
                                         x0:x0 + sw * (Wo - 1) + 1:sw].transpose(0, 2, 3, 1)
    return U.reshape(B, Ho * Wo, Cin * kh * kw)
