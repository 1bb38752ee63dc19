"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names the passage it follows and the mistake it would catch.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import definitions as D
from oracle import drivers
from oracle import noise as N
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _f64_default():
    """fp64 autograd in these tests only (restored afterwards)."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _two_layer_net(rng, d, h, p):
    W1 = torch.tensor(rng.standard_normal((h, d)) / math.sqrt(d), requires_grad=True)
    b1 = torch.tensor(rng.standard_normal(h) * 0.1, requires_grad=True)
    W2 = torch.tensor(rng.standard_normal((p, h)) / math.sqrt(h), requires_grad=True)
    b2 = torch.tensor(rng.standard_normal(p) * 0.1, requires_grad=True)
    return W1, b1, W2, b2


def _per_example_losses(x, y, W1, b1, W2, b2):
    s1 = x @ W1.T + b1           # [B, T, h]
    a1 = torch.tanh(s1)
    s2 = a1 @ W2.T + b2          # [B, T, p]
    return ((s2 - y) ** 2).sum(dim=(1, 2)), s1, a1, s2


# ---------------------------------------------------------------- P1: brute force
@pytest.mark.parametrize("B,T,d,h,p", [(4, 1, 5, 7, 3), (3, 6, 4, 5, 2), (2, 9, 8, 3, 4)])
def test_per_example_grads_equal_single_example_backprop(B, T, d, h, p):
    """[FPC] loop over examples one at a time (the baseline that defines
    per-example gradients); [SEDP] eq. (2.4): the per-sample gradient of a
    linear layer is a_i^T dL/ds_i. Catches a transposed operand, a missing
    sum over T, or a wrong bias gradient."""
    rng = np.random.default_rng(1)
    x = torch.tensor(rng.standard_normal((B, T, d)))
    y = torch.tensor(rng.standard_normal((B, T, p)))
    W1, b1, W2, b2 = _two_layer_net(rng, d, h, p)
    # layer inputs and output gradients of the whole batch
    losses, s1, a1, s2 = _per_example_losses(x, y, W1, b1, W2, b2)
    s1.retain_grad(); s2.retain_grad()
    losses.sum().backward()
    A1, G1 = x.detach().numpy(), s1.grad.numpy()
    A2, G2 = a1.detach().numpy(), s2.grad.numpy()
    for i in range(B):
        Wg = [w.detach().clone().requires_grad_(True) for w in (W1, b1, W2, b2)]
        li, _, _, _ = _per_example_losses(x[i:i + 1], y[i:i + 1], *Wg)
        gW1, gb1, gW2, gb2 = torch.autograd.grad(li.sum(), Wg)
        # torch weight layout is [out, in]; the oracle's is [in, out]
        np.testing.assert_allclose(D.per_example_weight_grad(A1[i], G1[i]), gW1.numpy().T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(D.per_example_weight_grad(A2[i], G2[i]), gW2.numpy().T, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(D.per_example_bias_grad(G1[i]), gb1.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(D.per_example_bias_grad(G2[i]), gb2.numpy(), rtol=1e-12, atol=1e-12)
        sq = D.layer_sqnorms(A2[i:i + 1], G2[i:i + 1], has_bias=True)[0]
        assert sq == pytest.approx(float((gW2 ** 2).sum() + (gb2 ** 2).sum()), rel=1e-12)


@pytest.mark.parametrize("cin,H,cout,stride", [(3, 6, 4, 1), (2, 7, 3, 2), (4, 4, 5, 1)])
def test_conv_per_example_grad_via_unfold(cin, H, cout, stride):
    """[FPC] Algorithm 3 (im2col + GEMM gives the per-example conv gradient);
    [SEDP] eqs. (2.5)-(2.6): U(a_i)^T F^-1(dL/ds_i) is the conv weight gradient.
    Pins the unfold layout of the conv workload (channel, kernel row, kernel
    column) against a batch-1 conv2d backward."""
    rng = np.random.default_rng(2)
    B = 3
    x = rng.standard_normal((B, cin, H, H)).astype(np.float32)
    Wt = torch.tensor(rng.standard_normal((cout, cin, 3, 3)), requires_grad=True)
    U = W.unfold3x3(x, stride).astype(np.float64)         # [B, T, cin*9]
    for i in range(B):
        xi = torch.tensor(x[i:i + 1].astype(np.float64))
        out = F.conv2d(xi, Wt, stride=stride, padding=1)  # [1, cout, Ho, Wo]
        R = torch.tensor(rng.standard_normal(out.shape))
        (gW,) = torch.autograd.grad((out * R).sum(), [Wt])
        Gi = R[0].reshape(cout, -1).T.numpy()             # F^-1: [Ho*Wo, cout]
        g = D.per_example_weight_grad(U[i], Gi)           # [cin*9, cout]
        np.testing.assert_allclose(g, gW.reshape(cout, -1).T.numpy(), rtol=1e-10, atol=1e-10)


CONV_GEOMETRIES = [  # (C_in, H, W, kernel, stride, padding, dilation)
    (3, 7, 9, (3, 3), (1, 1), (1, 1), (1, 1)),
    (2, 8, 8, (3, 3), (2, 2), (1, 1), (1, 1)),
    (4, 6, 5, (5, 3), (2, 1), (2, 0), (1, 2)),
    (3, 4, 4, (1, 1), (2, 2), (0, 0), (1, 1)),
    (2, 9, 7, (2, 4), (3, 2), (0, 3), (2, 1)),
]


@pytest.mark.parametrize("cin,H,Wd,k,s,pad,dil", CONV_GEOMETRIES)
def test_unfold2d_gives_conv_weight_grad(cin, H, Wd, k, s, pad, dil):
    """[SEDP] Sec. 2.2, eqs. (2.5)-(2.6); [FPC] Algorithm 3: the oracle's
    unfolding U(a_i) times F^-1(dL/ds_i) is the per-example conv weight
    gradient, here from a batch-1 conv2d backward with stride, padding,
    dilation and a rectangular kernel. A wrong column order, tap offset or
    padding fill fails it."""
    rng = np.random.default_rng(7)
    B, cout = 2, 3
    x = rng.standard_normal((B, cin, H, Wd))
    Wt = torch.tensor(rng.standard_normal((cout, cin) + k), requires_grad=True)
    U = D.unfold2d(x, k, s, pad, dil)
    for i in range(B):
        out = F.conv2d(torch.tensor(x[i:i + 1]), Wt, stride=s, padding=pad, dilation=dil)
        assert U.shape[1] == out.shape[2] * out.shape[3]
        R = torch.tensor(rng.standard_normal(out.shape))
        (gW,) = torch.autograd.grad((out * R).sum(), [Wt])
        Gi = R[0].reshape(cout, -1).T.numpy()
        np.testing.assert_allclose(D.per_example_weight_grad(U[i], Gi), gW.reshape(cout, -1).T.numpy(),
                                   rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("cin,H,Wd,k,s,pad,dil", CONV_GEOMETRIES)
def test_unfold2d_matches_torch_unfold(cin, H, Wd, k, s, pad, dil):
    """The unfolding is torch's im2col (F.unfold) laid out [B, T, d]; a
    library routine of the same definition ([FPC] Algorithm 3)."""
    x = np.random.default_rng(8).standard_normal((2, cin, H, Wd))
    ref = F.unfold(torch.tensor(x), k, dilation=dil, padding=pad, stride=s).transpose(1, 2).numpy()
    np.testing.assert_array_equal(D.unfold2d(x, k, s, pad, dil), ref)


def test_unfold2d_closed_forms():
    """A 1x1 kernel at stride 1 is the channel-last view of the input; with a
    kernel as large as the padded input there is one row, the flattened padded
    input. Checks the row count and the zero fill of the padding."""
    x = np.random.default_rng(9).standard_normal((2, 3, 4, 5))
    np.testing.assert_array_equal(D.unfold2d(x, (1, 1)), x.reshape(2, 3, 20).transpose(0, 2, 1))
    U = D.unfold2d(x, (6, 7), padding=(1, 1))
    padded = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)))
    assert U.shape == (2, 1, 3 * 6 * 7)
    np.testing.assert_array_equal(U[:, 0, :], padded.reshape(2, -1))


# ---------------------------------------------------------------- P2/P3: identities
@pytest.mark.parametrize("B,T,d,p", [(3, 1, 7, 5), (2, 17, 9, 4), (4, 33, 3, 40), (1, 5, 64, 2)])
@pytest.mark.parametrize("has_bias", [False, True])
def test_ghost_identity(B, T, d, p, has_bias):
    """[SEDP] eq. (2.7), Sec. 3.1: ||A_i^T G_i||_F^2 = <A_i A_i^T, G_i G_i^T>.
    With a bias the input gains a constant-1 feature, so the Gram of A gains
    the all-ones matrix. Catches a dropped bias term or a wrong square."""
    rng = np.random.default_rng(3)
    A = rng.standard_normal((B, T, d))
    G = rng.standard_normal((B, T, p))
    ghost = np.einsum("bst,bst->b", np.einsum("bsd,btd->bst", A, A) + (1.0 if has_bias else 0.0),
                      np.einsum("bsp,btp->bst", G, G))
    np.testing.assert_allclose(D.layer_sqnorms(A, G, has_bias), ghost, rtol=1e-12)


def test_t1_closed_form():
    """[FPC] eq. (6): for one row the gradient is an outer product, whose
    squared norm is ||a||^2 ||g||^2; a bias adds ||g||^2."""
    rng = np.random.default_rng(4)
    A = rng.standard_normal((6, 1, 11))
    G = rng.standard_normal((6, 1, 13))
    a2 = (A[:, 0] ** 2).sum(1)
    g2 = (G[:, 0] ** 2).sum(1)
    np.testing.assert_allclose(D.layer_sqnorms(A, G, False), a2 * g2, rtol=1e-12)
    np.testing.assert_allclose(D.layer_sqnorms(A, G, True), (a2 + 1) * g2, rtol=1e-12)


def test_total_norm_sums_layers():
    """Global clipping: one norm over all parameters ([DDP] code: the norm
    over all parameter gradients; [SEDP] Sec. 3, sum over layers)."""
    rng = np.random.default_rng(5)
    layers = [(rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 3))),
              (rng.standard_normal((3, 5, 2)), rng.standard_normal((3, 5, 6)))]
    n = D.total_norms([D.layer_sqnorms(A, G) for A, G in layers])
    for i in range(3):
        flat = np.concatenate([D.per_example_weight_grad(A[i], G[i]).ravel() for A, G in layers])
        assert n[i] == pytest.approx(np.linalg.norm(flat), rel=1e-13)


# ---------------------------------------------------------------- P4: clip invariants
def test_clip_invariants():
    """[FPC] clip_c: norm <= c after clipping, unchanged when already <= c,
    exactly c when clipped; [DDP] g / max(1, ||g||/C) is the same map.
    Catches an inverted ratio, a missing min with 1, or clipping at equality."""
    rng = np.random.default_rng(6)
    B, T, d, p = 12, 3, 4, 5
    A = rng.standard_normal((B, T, d))
    G = rng.standard_normal((B, T, p))
    A[2] *= 1e-2            # well below the bound
    A[7] *= 1e-3
    sq = D.layer_sqnorms(A, G)
    norms = np.sqrt(sq)
    C = float(np.median(norms))
    c = D.clip_factors(norms, C)
    for i in range(B):
        g = D.per_example_weight_grad(A[i], G[i])
        cg = c[i] * g
        assert np.linalg.norm(cg) <= C * (1 + 1e-12)
        assert (c[i] == 1.0) == (norms[i] <= C)
        if norms[i] > C:
            assert c[i] * norms[i] == pytest.approx(C, rel=1e-14)
            assert c[i] < 1.0
        np.testing.assert_allclose(cg, g / max(1.0, np.linalg.norm(g) / C), rtol=1e-13)
    assert c[2] == 1.0 and c[7] == 1.0
    # a norm exactly at the bound is left unchanged; zero norm gives c = 1
    assert D.clip_factors(np.array([C, 0.0]), C).tolist() == [1.0, 1.0]


# ---------------------------------------------------------------- P5: contraction
def test_clipped_sum_is_gradient_of_reweighted_loss():
    """[FPC] the gradient of the re-weighted loss sum_i nu_i L_i is exactly the
    sum of the re-weighted per-example gradients; with all weights 1 it is the
    ordinary batch gradient. [SEDP] Sec. 3.2 second back-propagation on
    sum_i C_i L_i. Catches a weight applied to the wrong sample or dropped."""
    rng = np.random.default_rng(7)
    B, T, d, h, p = 5, 4, 6, 3, 2
    x = torch.tensor(rng.standard_normal((B, T, d)))
    y = torch.tensor(rng.standard_normal((B, T, p)))
    W1, b1, W2, b2 = _two_layer_net(rng, d, h, p)
    losses, s1, a1, s2 = _per_example_losses(x, y, W1, b1, W2, b2)
    s1.retain_grad()
    losses.sum().backward()
    A, G = x.detach().numpy(), s1.grad.numpy()
    for c in (np.ones(B), rng.uniform(0.1, 1.0, B)):
        Wg = [w.detach().clone().requires_grad_(True) for w in (W1, b1, W2, b2)]
        lw, _, _, _ = _per_example_losses(x, y, *Wg)
        gW1, gb1 = torch.autograd.grad((torch.tensor(c) * lw).sum(), Wg[:2])
        S, Sb = D.clipped_sum(A, G, c, has_bias=True)
        np.testing.assert_allclose(S, gW1.numpy().T, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Sb, gb1.numpy(), rtol=1e-11, atol=1e-12)


def test_clipped_sum_selects_and_is_linear():
    rng = np.random.default_rng(8)
    B, T, d, p = 4, 3, 5, 6
    A = rng.standard_normal((B, T, d))
    G = rng.standard_normal((B, T, p))
    for j in range(B):
        e = np.zeros(B); e[j] = 1.0
        S, _ = D.clipped_sum(A, G, e)
        np.testing.assert_allclose(S, A[j].T @ G[j], rtol=1e-13, atol=1e-13)
    c1, c2 = rng.uniform(size=B), rng.uniform(size=B)
    S1, _ = D.clipped_sum(A, G, c1)
    S2, _ = D.clipped_sum(A, G, c2)
    S12, _ = D.clipped_sum(A, G, 2.0 * c1 - 3.0 * c2)
    np.testing.assert_allclose(S12, 2.0 * S1 - 3.0 * S2, rtol=1e-12, atol=1e-12)


def test_global_step_without_noise_or_clipping_is_mean_gradient():
    """[FPC] with no clipping and no noise the update is the mini-batch mean
    gradient (1/tau) sum_i grad l_i."""
    rng = np.random.default_rng(9)
    B, T, d, p = 6, 2, 5, 4
    A = rng.standard_normal((B, T, d))
    G = rng.standard_normal((B, T, p))
    r = drivers.global_clip_step([(A, G)], C=1e9, sigma=0.0, seed=1)
    np.testing.assert_allclose(r["outs"][0], np.einsum("btd,btp->dp", A, G) / B, rtol=1e-12)
    assert np.all(r["c"] == 1.0)


def test_virtual_step_is_accumulated_reweighted_backprop():
    """[SEDP] gradient accumulation: back-propagating each physical batch's
    re-weighted loss sum_i c_i L_i into the same .grad before one update gives
    the logical batch's clipped sum; divided by the logical batch size it is
    the virtual step's update (sigma = 0). Catches a batch dropped or counted
    twice, factors applied to the wrong batch, or the mean taken per physical
    batch instead of over the logical one."""
    rng = np.random.default_rng(17)
    T, d, h, p = 3, 5, 4, 3
    W1, b1, W2, b2 = _two_layer_net(rng, d, h, p)
    Wg = [w.detach().clone().requires_grad_(True) for w in (W1, b1, W2, b2)]
    batches, cs = [], []
    for B in (3, 2, 4):
        x = torch.tensor(rng.standard_normal((B, T, d)))
        y = torch.tensor(rng.standard_normal((B, T, p)))
        c = rng.uniform(0.1, 1.0, B)
        losses, s1, _, _ = _per_example_losses(x, y, *Wg)
        s1.retain_grad()
        (torch.tensor(c) * losses).sum().backward()  # accumulates into Wg[k].grad
        # layer-1 output gradients of the unweighted per-example losses
        l2, s1u, _, _ = _per_example_losses(x, y, W1, b1, W2, b2)
        s1u.retain_grad()
        l2.sum().backward()
        batches.append((x.numpy(), s1u.grad.numpy()))
        cs.append(c)
    r = drivers.virtual_step(batches, cs, C=1.0, sigma=0.0, seed=3, has_bias=True)
    assert r["denom"] == 9.0
    np.testing.assert_allclose(r["out"], Wg[0].grad.numpy().T / 9.0, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["bias_out"], Wg[1].grad.numpy() / 9.0, rtol=1e-11, atol=1e-13)
    # the noise is drawn once, from the logical step's counters
    rn = drivers.virtual_step(batches, cs, C=1.5, sigma=0.5, seed=3, layer_id=2, step=4, has_bias=True)
    z = N.weight_noise(d, h, 3, 2, 4).astype(np.float64)
    np.testing.assert_allclose(rn["out"] - r["out"], 1.5 * 0.5 * z / 9.0, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P6: noise
def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


def test_philox_known_answers():
    """Salmon et al. (SC'11) known-answer vectors. Catches a swapped word, a
    wrong multiplier or Weyl constant, or a wrong number of rounds."""
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, out in rows:
        got = N.philox4x32_10(tuple(np.array([c], dtype=np.uint64) for c in ctr), key)
        assert [int(g[0]) for g in got] == out


def test_ln_sin_cos_accuracy():
    """The specified fp32 ln and quarter-turn sin/cos agree with libm to a few
    fp32 ulps over their whole input grids (catches a wrong coefficient, a
    wrong reduction branch or a wrong quadrant)."""
    u = (np.arange(1, 2 ** 24 + 1, 101, dtype=np.float64) * 2.0 ** -24).astype(np.float32)
    ref = np.log(u.astype(np.float64))
    got = N.ln_f32(u).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 4e-7 * np.abs(ref) + 1e-13)   # a few fp32 ulps
    f = (np.arange(0, 2 ** 22, 7) * 2.0 ** -22).astype(np.float32)
    s, c = N.sincos_quarter_f32(f)
    ang = np.pi / 2 * f.astype(np.float64)
    assert np.max(np.abs(s - np.sin(ang))) < 2.5e-7
    assert np.max(np.abs(c - np.cos(ang))) < 2.5e-7
    # full Box-Muller quadrant rotation against libm on random words
    rng = np.random.default_rng(10)
    xa = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    xb = rng.integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    z0, z1 = N.box_muller_f32(xa, xb)
    u1 = ((xa >> 8).astype(np.float64) + 1) * 2.0 ** -24
    u2 = (xb >> 8).astype(np.float64) * 2.0 ** -24
    r = np.sqrt(-2 * np.log(u1))
    np.testing.assert_allclose(z0, r * np.cos(2 * np.pi * u2), atol=3e-6 * max(1.0, r.max()))
    np.testing.assert_allclose(z1, r * np.sin(2 * np.pi * u2), atol=3e-6 * max(1.0, r.max()))


def test_normal_stream_statistics():
    """Sample mean, variance and KS distance of 1e7 normals from the stream
    (the pages require N(0, sigma^2 C^2 I) noise). Bounds: |mean| <= 5/sqrt(n),
    |var - 1| <= 5 sqrt(2/n), KS statistic below the 1e-6 critical value."""
    from scipy.special import ndtr
    n = 10_000_000
    z = N.normals(n, seed=12345, layer=3, which=0, step=7).astype(np.float64)
    assert abs(z.mean()) <= 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) <= 5 * math.sqrt(2 / n)
    zs = np.sort(z)
    cdf = ndtr(zs)
    ks = max(np.max(np.arange(1, n + 1) / n - cdf), np.max(cdf - np.arange(0, n) / n))
    assert ks < 2.7 / math.sqrt(n)
    # independent streams for different (layer, which, step, tag) are uncorrelated
    z2 = N.normals(n // 10, seed=12345, layer=3, which=1, step=7).astype(np.float64)
    assert abs(np.corrcoef(z[: n // 10], z2)[0, 1]) < 5 / math.sqrt(n // 10)


def test_normal_stream_layout():
    """Element e of the flat stream is lane e % 4 of group e // 4; windows of
    the stream agree with the whole stream; the threshold normal is tag 1."""
    full = N.normals(103, seed=7, layer=2, which=0, step=5)
    for s, n in [(0, 103), (1, 10), (3, 4), (50, 53), (101, 2)]:
        np.testing.assert_array_equal(N.normals(n, 7, 2, 0, 5, start=s), full[s:s + n])
    x = N.philox4x32_10(tuple(np.array([v], dtype=np.uint64) for v in (25, 4, 5, 0)), N.key_of(7))
    za, zb = N.box_muller_f32(x[0], x[1])
    zc, zd = N.box_muller_f32(x[2], x[3])
    assert full[100:103].tolist() == [za[0], zb[0], zc[0]]
    t = N.threshold_normal(7, 2, 5)
    x = N.philox4x32_10(tuple(np.array([v], dtype=np.uint64) for v in (0, 4, 5, 1)), N.key_of(7))
    assert t == N.box_muller_f32(x[0], x[1])[0][0]
    assert N.key_of((3 << 32) | 9) == (9, 3)


def test_noised_mean_forms_agree():
    rng = np.random.default_rng(11)
    S = rng.standard_normal((7, 9)).astype(np.float32)
    z = N.normals(63, 1, 0, 0, 0).reshape(7, 9)
    o32 = D.noised_mean_f32(S, z, 1.5, 0.7, 64.0)
    o64 = D.noised_mean(S.astype(np.float64), z, 1.5, 0.7, 64.0)
    np.testing.assert_allclose(o32, o64, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(D.noised_mean(np.zeros((2, 2)), np.ones((2, 2)), 2.0, 3.0, 4.0), 1.5)


# ---------------------------------------------------------------- P7: adaptive threshold
def test_adaptive_threshold_closed_forms():
    """[TTP] adaptive clipping: with no noise and every norm under C_l2 the new
    bound is alpha times the mean norm; with every norm over C_l2 it is
    alpha * C_l2 = alpha * beta * C_prev; init takes C_l2 as the mean norm;
    the noise enters as alpha * sigma_l2 * C_l2 * z / |L|."""
    rng = np.random.default_rng(12)
    n = rng.uniform(1.0, 2.0, 100)
    cl2, ct = D.adaptive_threshold(n, C_prev=5.0, alpha=1.1, beta=2.0, sigma_l2=0.0, init=False, z=0.3)
    assert cl2 == 10.0 and ct == pytest.approx(1.1 * n.mean(), rel=1e-14)
    cl2, ct = D.adaptive_threshold(n, C_prev=0.25, alpha=1.1, beta=2.0, sigma_l2=0.0, init=False, z=0.3)
    assert cl2 == 0.5 and ct == pytest.approx(1.1 * 0.5, rel=1e-14)
    cl2, ct = D.adaptive_threshold(n, C_prev=123.0, alpha=1.0, beta=2.0, sigma_l2=0.0, init=True, z=0.0)
    assert cl2 == pytest.approx(n.mean(), rel=1e-14)
    _, c0 = D.adaptive_threshold(n, 0.9, 1.1, 2.0, 0.0, False, 0.7)
    _, c1 = D.adaptive_threshold(n, 0.9, 1.1, 2.0, 2.5, False, 0.7)
    assert c1 - c0 == pytest.approx(1.1 * 2.5 * 1.8 * 0.7 / 100, rel=1e-10)
    # the page's clip(||y||) equals min(||y||, C_l2)
    np.testing.assert_allclose(D.adaptive_clip_norm(n, 1.5), np.minimum(n, 1.5), rtol=1e-15)


def test_adaptive_chain_driver():
    """Two steps of the per-layer adaptive schedule: the step uses C_t, and
    C_{t+1} comes from that step's norms with C_l2 = beta * C_t."""
    rng = np.random.default_rng(13)
    layers = [(rng.standard_normal((16, 1, 5)), rng.standard_normal((16, 1, 3)))]
    C_l2, C0 = drivers.adaptive_init(layers, 1.1, 2.0, 0.0, seed=3)
    norms = np.sqrt(D.layer_sqnorms(*layers[0], has_bias=True))
    assert C_l2[0] == pytest.approx(norms.mean(), rel=1e-14)
    r = drivers.adaptive_step(layers, C0, sigma=0.0, alpha=1.1, beta=2.0, sigma_l2=0.0, seed=3, step=0)
    assert r["C_l2"][0] == pytest.approx(2.0 * C0[0], rel=1e-15)
    np.testing.assert_allclose(r["c"][0], D.clip_factors(norms, C0[0]))


# ---------------------------------------------------------------- P8: path rule
def test_time_rule_counts_the_work_of_each_path():
    """The time rule's per-sample work figures, counted by brute force: the
    instantiated product A_i^T G_i (d*p entries of T multiply-adds) and its
    squared norm (d*p multiply-adds); the ghost Grams' unique entries (s <= t,
    d multiply-adds for A's and p for G's) and the Frobenius product over all
    T^2 entries ([SEDP] Appendix C). Catches a dropped term or a factor of 2."""
    def explicit_flops(T, d, p):
        macs = sum(T for _ in range(d) for _ in range(p)) + d * p
        return 2 * macs

    def ghost_flops(T, d, p):
        macs = sum(d + p for s_ in range(T) for t_ in range(s_, T)) + T * T
        return 2 * macs

    for (T, d, p) in [(2, 3, 5), (7, 4, 4), (16, 3, 9), (9, 40, 2), (30, 5, 6)]:
        e, g = explicit_flops(T, d, p), ghost_flops(T, d, p)
        want = D.PATH_EXPLICIT if e < g else D.PATH_GHOST
        assert D.choose_path(T, d, p, D.MODE_TIME) == want, (T, d, p, e, g)
    # both outcomes occur among these shapes
    assert {D.choose_path(T, d, p, D.MODE_TIME) for (T, d, p) in [(2, 3, 5), (30, 5, 6)]} == \
        {D.PATH_EXPLICIT, D.PATH_GHOST}


def test_path_rule_matches_the_pages_layer_pattern():
    """[SEDP] Sec. 4.2: in ResNets the early layers (large H*W, few channels)
    favour instantiation and the late layers (small H*W, many channels) the
    ghost norm; T = 1 layers use the closed form; forced modes win."""
    wl = W.WORKLOADS["resnet18-conv-t1024"]
    paths = [D.choose_path(T, d, p) for (T, d, p) in wl.layers]
    assert paths[:2] == [D.PATH_EXPLICIT] * 2 and paths[2:] == [D.PATH_GHOST] * 6
    # the 2T^2-vs-pD space comparison flips the third layer (T=256, D=576, p=128)
    assert D.choose_path(256, 576, 128, kappa=2) == D.PATH_EXPLICIT
    for (T, d, p) in W.WORKLOADS["gpt-block-t128"].layers + W.WORKLOADS["gpt2large-t1024"].layers:
        assert D.choose_path(T, d, p) == D.PATH_GHOST
    assert D.choose_path(1, 64, 32) == D.PATH_T1
    assert D.choose_path(1, 64, 32, mode=D.MODE_EXPLICIT) == D.PATH_EXPLICIT
    assert D.choose_path(1024, 27, 64, mode=D.MODE_GHOST) == D.PATH_GHOST
    assert D.choose_path(4, 2, 8) == D.PATH_GHOST      # tie p*d == T^2 goes to ghost


# ---------------------------------------------------------------- inputs
def test_workload_inputs_shapes_and_recipe():
    for name in W.WORKLOAD_ORDER:
        wl = W.WORKLOADS[name]
        T, d, p = wl.layer_shape(0)
        B = min(wl.B, 4)
        shape = None if name == "resnet18-conv-t1024" else (T, min(d, 64), min(p, 64))
        A, G = W.make_layer(wl, 0, B=B, shape=shape)
        exp_dt = np.uint16 if wl.dtype == "bf16" else np.float32
        assert A.dtype == exp_dt and G.dtype == exp_dt
        A2, _ = W.make_layer(wl, 0, B=B, shape=shape)
        np.testing.assert_array_equal(A, A2)            # seeded
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e-3], dtype=np.float32)
    b = W.f32_to_bf16_bits(x)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(b),
                                  torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy())


def test_entrywise_helpers_agree_with_whole_forms():
    """The entry-wise clipped sum and the indexed noise lookup used by
    full-size checks equal the corresponding entries of the whole forms."""
    rng = np.random.default_rng(14)
    A = rng.standard_normal((5, 3, 7))
    G = rng.standard_normal((5, 3, 6))
    c = rng.uniform(size=5)
    S, _ = D.clipped_sum(A, G, c)
    rows = rng.integers(0, 7, 20)
    cols = rng.integers(0, 6, 20)
    np.testing.assert_allclose(D.clipped_sum_entries(A, G, c, rows, cols), S[rows, cols], rtol=1e-13)
    full = N.normals(42, 9, 4, 1, 3)
    idx = rng.integers(0, 42, 30)
    np.testing.assert_array_equal(N.normals_at(idx, 9, 4, 1, 3), full[idx])


def test_weight_noise_layout():
    """Weight noise element (m, n) is lane m % 4 of the Philox block at group
    (m // 4) * p + n; rows past d in the last group are simply not used."""
    d, p, seed, layer, step = 7, 5, 11, 2, 3
    z = N.weight_noise(d, p, seed, layer, step)
    assert z.shape == (d, p)
    for m in range(d):
        for n in range(p):
            j = (m // 4) * p + n
            x = N.philox4x32_10(tuple(np.array([v], dtype=np.uint64) for v in (j, 2 * layer, step, 0)),
                                N.key_of(seed))
            za, zb = N.box_muller_f32(x[0], x[1])
            zc, zd = N.box_muller_f32(x[2], x[3])
            assert z[m, n] == [za[0], zb[0], zc[0], zd[0]][m % 4]
    rows = np.array([0, 3, 4, 6, 6])
    cols = np.array([4, 0, 2, 1, 4])
    np.testing.assert_array_equal(N.weight_noise_at(rows, cols, p, seed, layer, step), z[rows, cols])


def test_newton_reciprocal_and_rsqrt():
    """The division- and sqrt-free helpers of the noise spec agree with the
    exact reciprocal and square root to 2e-7 relative over their ranges."""
    b = np.linspace(1.7071, 2.41422, 100001).astype(np.float32)
    assert np.max(np.abs(N.rcp_f32(b).astype(np.float64) * b - 1.0)) < 2e-7
    t = np.concatenate([np.linspace(1.19e-7, 1e-3, 50001), np.linspace(1e-3, 33.3, 50001)]).astype(np.float32)
    y = N.rsqrt_f32(t).astype(np.float64)
    assert np.max(np.abs(y * np.sqrt(t.astype(np.float64)) - 1.0)) < 2e-7
    z0, z1 = N.box_muller_f32(np.array([0xFFFFFFFF], dtype=np.uint32), np.array([5], dtype=np.uint32))
    assert z0[0] == 0.0 and z1[0] == 0.0   # u1 = 1 gives r = 0


def _stream_positions(values, stream):
    """Position in `stream` of every entry of `values`, found by value (no
    index formula): a dict from fp32 bit pattern to the list of positions
    where it occurs. Returns (positions, ambiguous) where ambiguous counts
    the values that occur more than once in the stream."""
    where = {}
    for k, b in enumerate(stream.view(np.uint32).tolist()):
        where.setdefault(b, []).append(k)
    pos, amb = [], 0
    for b in values.reshape(-1).view(np.uint32).tolist():
        ks = where.get(b)
        assert ks is not None, "a noise value that the stream does not hold"
        amb += len(ks) > 1
        pos.append(ks[0])
    return np.array(pos, dtype=np.int64), amb


@pytest.mark.parametrize("d,p", [(7, 5), (8, 1), (1, 9), (13, 3), (64, 32), (5, 17)])
def test_weight_noise_draws_distinct_normals_of_its_stream(d, p):
    """[FPC] Gaussian mechanism and [SEDP] eq. (2.1): the noise added to the
    [d, p] clipped sum is N(0, sigma^2 C^2 I), every coordinate its own
    independent normal. Located by value in the flat weight stream
    (which = 0) of the first ceil(d/4)*p blocks: every entry of
    weight_noise(d, p) is there, no two entries share one position (a map
    that reused a normal fails), and the entries touch exactly those
    ceil(d/4)*p blocks (a map that skipped or overran blocks fails). The bias
    noise of [p] is the first p normals of the which = 1 stream, in order, and
    shares no value with the weight noise."""
    seed, layer, step = 0xABCDEF12345, 3, 9
    nq = -(-d // 4)
    z = N.weight_noise(d, p, seed, layer, step)
    assert z.shape == (d, p) and z.dtype == np.float32
    stream = N.normals(4 * nq * p + 64, seed, layer, 0, step)
    pos, amb = _stream_positions(z, stream)
    assert amb == 0
    assert len(set(pos.tolist())) == d * p                       # injective
    assert pos.max() < 4 * nq * p                                # nothing past the blocks it needs
    assert set((pos // 4).tolist()) == set(range(nq * p))        # every needed block used
    zb = N.normals(p, seed, layer, 1, step)
    bstream = N.normals(p + 8, seed, layer, 1, step)
    bpos, bamb = _stream_positions(zb, bstream)
    assert bamb == 0 and bpos.tolist() == list(range(p))
    assert not (set(zb.view(np.uint32).tolist()) & set(z.reshape(-1).view(np.uint32).tolist()))


def test_weight_noise_array_has_the_gaussian_law():
    """The [d, p] weight-noise array (and the [p] bias noise) as a sample of
    N(0, I): mean, variance and KS distance of all entries, and lag-1
    correlations along rows, along columns and across the 4-row groups that
    share a Philox block, each within 5/sqrt(n). Sizes are ragged (d % 4 != 0)
    so the partial last group is included. A layout that repeated or
    correlated normals within the array would fail the lag tests; one that
    biased the lanes would fail the moments."""
    from scipy.special import ndtr
    d, p = 2051, 997
    z = N.weight_noise(d, p, 77, 5, 2).astype(np.float64)
    n = z.size
    assert abs(z.mean()) <= 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) <= 5 * math.sqrt(2 / n)
    zs = np.sort(z.reshape(-1))
    cdf = ndtr(zs)
    ks = max(np.max(np.arange(1, n + 1) / n - cdf), np.max(cdf - np.arange(0, n) / n))
    assert ks < 2.7 / math.sqrt(n)

    def lag_corr(x, y):
        x = x.reshape(-1) - x.mean()
        y = y.reshape(-1) - y.mean()
        return float(np.dot(x, y) / math.sqrt(np.dot(x, x) * np.dot(y, y))), x.size

    for a, b in [(z[:, :-1], z[:, 1:]),          # along rows (neighbouring columns)
                 (z[:-1, :], z[1:, :]),          # along columns (neighbouring rows)
                 (z[0:-4:4, :], z[3::4, :][: (d - 1) // 4]),   # first and last lane of a block
                 (z[:-4, :], z[4:, :])]:         # the same lane of consecutive blocks
        r, m = lag_corr(a, b)
        assert abs(r) <= 5 / math.sqrt(m), r
    # per-lane moments: no lane of the 4-row groups is biased
    for lane in range(4):
        zl = z[lane::4, :]
        assert abs(zl.mean()) <= 5 / math.sqrt(zl.size)
        assert abs(zl.var() - 1.0) <= 5 * math.sqrt(2 / zl.size)
    zb = N.normals(200_003, 77, 5, 1, 2).astype(np.float64)
    assert abs(zb.mean()) <= 5 / math.sqrt(zb.size)
    assert abs(zb.var() - 1.0) <= 5 * math.sqrt(2 / zb.size)
    r, m = lag_corr(zb[:-1], zb[1:])
    assert abs(r) <= 5 / math.sqrt(m)
    r, m = lag_corr(zb[:100_000], z.reshape(-1)[:100_000])   # bias vs weight stream
    assert abs(r) <= 5 / math.sqrt(m)
