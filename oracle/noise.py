"""Counter-based Gaussian noise stream (oracle side; test infrastructure only).

The pages fix only the distribution of the noise, N(0, sigma^2 C^2 I) ("Scaling
up DP Deep Learning with Fast Per-Example Gradient Clipping", Gaussian
mechanism; "Scalable and Efficient Training ... with DP", eq. (2.1)); they name
no generator. The stream specified here is:

Generator: Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter and
a 2x32-bit key; each of the 10 rounds multiplies words 0 and 2 by the round
multipliers M0 = 0xD2511F53 and M1 = 0xCD9E8D57 (64-bit products split into
hi/lo halves) and mixes the halves with words 1 and 3 and the round key; the
key is bumped by the Weyl constants W0 = 0x9E3779B9, W1 = 0xBB67AE85 between
rounds.

Stream layout: key = (seed mod 2^32, seed div 2^32). Element e of a flat
stream belongs to group j = e // 4 and takes lane e % 4 of the block
Philox(counter = (j, 2*layer + which, step, tag), key); which = 0 for weight
noise, 1 for bias noise; tag = 0 for gradient noise, 1 for the noise of the
adaptive threshold (element 0 of group 0). The weight noise of a [d, p]
output groups 4 consecutive rows of one column: element (m, n) takes lane
m % 4 of group (m // 4) * p + n (weight_noise); the bias noise of a [p]
output is the flat stream (element n: lane n % 4 of group n // 4).

Normals: one block (x0, x1, x2, x3) gives four normals by Box-Muller on the
pairs (x0, x1) and (x2, x3):
  u1 = ((x >> 8) + 1) * 2^-24  in (0, 1]      (exact in fp32)
  v  = x' >> 8;  q = v >> 22 (quadrant);  f = (v & (2^22 - 1)) * 2^-22  (exact)
  r  = sqrt(-2 ln u1);  (z_a, z_b) = r * (cos 2 pi u2, sin 2 pi u2), u2 = v 2^-24
All arithmetic is fp32 with every operation rounded (no fused multiply-add)
and no division or square root: both are replaced by fixed Newton sequences
from integer-bit initial guesses, so that the two implementations can follow
the same operations exactly. ln and sin/cos are evaluated as below with the
constants given as hex floats; the tails of the series beyond the kept terms
are below 1e-9 relative, under the fp32 rounding of the result.
  rcp(b), b in [1.7, 2.5]:  r = bits(0x7EF311C3 - bits(b)); 3 times
          r = r * (2 - b*r).                       (max rel. error 1.5e-7)
  rsqrt(t), t > 0:  y = bits(0x5F3759DF - (bits(t) >> 1)), h = 0.5*t; 3 times
          y = y * (1.5 - h*(y*y)).                  (max rel. error 1.6e-7)
  ln u1:  u1 = m * 2^e with m in [2^-1/2, 2^1/2] (m halved and e raised when
          m > SQRT2); s = (m - 1) * rcp(m + 1); ln m = 2s * (1 + s^2/3 + ... +
          s^10/11) by Horner in s^2; ln u1 = e*LN2 + ln m   (atanh series).
  r = t * rsqrt(t) for t = -2 ln u1 > 0, and r = 0 for t = 0 (u1 = 1).
  sin/cos of (pi/2)*f: if f > 1/2 use g = 1 - f and swap sin and cos; phi = g*HALF_PI;
          sin phi = phi + phi*(phi^2*P_s(phi^2)), cos phi = 1 + phi^2*P_c(phi^2),
          Taylor polynomials to phi^9 and phi^10; then the quadrant q rotates
          (cos, sin) by q quarter turns.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)

_f = np.float32


def _hx(s: str) -> np.float32:
    return np.float32(float.fromhex(s))


LN2 = _hx("0x1.62e430p-1")
SQRT2 = _hx("0x1.6a09e6p+0")
HALF_PI = _hx("0x1.921fb6p+0")
K3 = _hx("0x1.555556p-2")
K5 = _hx("0x1.99999ap-3")
K7 = _hx("0x1.24924ap-3")
K9 = _hx("0x1.c71c72p-4")
K11 = _hx("0x1.745d18p-4")
S3 = _hx("-0x1.555556p-3")
S5 = _hx("0x1.111112p-7")
S7 = _hx("-0x1.a01a02p-13")
S9 = _hx("0x1.71de3ap-19")
C2 = _hx("-0x1.000000p-1")
C4 = _hx("0x1.555556p-5")
C6 = _hx("-0x1.6c16c2p-10")
C8 = _hx("0x1.a01a02p-16")
C10 = _hx("-0x1.27e4fcp-22")
TWO_M24 = np.float32(2.0 ** -24)
TWO_M22 = np.float32(2.0 ** -22)


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays: ctr is a tuple of four uint32-valued arrays,
    key a pair of ints. Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in ctr)
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for r in range(10):
        if r > 0:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


RCP_MAGIC = np.uint32(0x7EF311C3)
RSQRT_MAGIC = np.uint32(0x5F3759DF)


def rcp_f32(b: np.ndarray) -> np.ndarray:
    """Reciprocal of b in [1.7, 2.5] as the specified Newton sequence."""
    b = np.asarray(b, dtype=np.float32)
    r = (RCP_MAGIC - b.view(np.uint32)).view(np.float32)
    for _ in range(3):
        t = (b * r).astype(np.float32)
        t = (_f(2.0) - t).astype(np.float32)
        r = (r * t).astype(np.float32)
    return r


def rsqrt_f32(t: np.ndarray) -> np.ndarray:
    """1/sqrt(t) for t > 0 as the specified Newton sequence."""
    t = np.asarray(t, dtype=np.float32)
    y = (RSQRT_MAGIC - (t.view(np.uint32) >> np.uint32(1))).view(np.float32)
    h = (_f(0.5) * t).astype(np.float32)
    for _ in range(3):
        y2 = (y * y).astype(np.float32)
        pr = (h * y2).astype(np.float32)
        q = (_f(1.5) - pr).astype(np.float32)
        y = (y * q).astype(np.float32)
    return y


def ln_f32(u: np.ndarray) -> np.ndarray:
    """Natural log of u in (0, 1] as the specified fp32 operation sequence."""
    u = np.asarray(u, dtype=np.float32)
    bits = u.view(np.uint32)
    e = ((bits >> np.uint32(23)).astype(np.int32) - 127)
    m = ((bits & np.uint32(0x007FFFFF)) | np.uint32(0x3F800000)).view(np.float32)
    big = m > SQRT2
    m = np.where(big, (m * _f(0.5)).astype(np.float32), m)
    e = np.where(big, e + 1, e)
    s = ((m - _f(1.0)).astype(np.float32) * rcp_f32((m + _f(1.0)).astype(np.float32))).astype(np.float32)
    s2 = (s * s).astype(np.float32)
    p = np.full_like(s2, K11)
    for k in (K9, K7, K5, K3, _f(1.0)):
        p = ((p * s2).astype(np.float32) + k).astype(np.float32)
    lnm = ((s + s).astype(np.float32) * p).astype(np.float32)
    return ((e.astype(np.float32) * LN2).astype(np.float32) + lnm).astype(np.float32)


def sincos_quarter_f32(frac: np.ndarray):
    """(sin, cos) of (pi/2)*frac for frac in [0, 1), specified fp32 sequence."""
    f = np.asarray(frac, dtype=np.float32)
    swap = f > _f(0.5)
    g = np.where(swap, (_f(1.0) - f).astype(np.float32), f)
    phi = (g * HALF_PI).astype(np.float32)
    p2 = (phi * phi).astype(np.float32)
    ps = np.full_like(p2, S9)
    for k in (S7, S5, S3):
        ps = ((ps * p2).astype(np.float32) + k).astype(np.float32)
    sin_phi = (phi + (phi * (p2 * ps).astype(np.float32)).astype(np.float32)).astype(np.float32)
    pc = np.full_like(p2, C10)
    for k in (C8, C6, C4, C2):
        pc = ((pc * p2).astype(np.float32) + k).astype(np.float32)
    cos_phi = (_f(1.0) + (p2 * pc).astype(np.float32)).astype(np.float32)
    s = np.where(swap, cos_phi, sin_phi)
    c = np.where(swap, sin_phi, cos_phi)
    return s, c


def box_muller_f32(xa: np.ndarray, xb: np.ndarray):
    """Two normals from two uint32 words, the specified fp32 sequence."""
    xa = np.asarray(xa, dtype=np.uint32)
    xb = np.asarray(xb, dtype=np.uint32)
    u1 = (((xa >> np.uint32(8)) + np.uint32(1)).astype(np.float32) * TWO_M24).astype(np.float32)
    v = xb >> np.uint32(8)
    q = (v >> np.uint32(22)).astype(np.int32)
    frac = ((v & np.uint32(0x3FFFFF)).astype(np.float32) * TWO_M22).astype(np.float32)
    t = (_f(-2.0) * ln_f32(u1)).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.where(t > _f(0.0), (t * rsqrt_f32(np.where(t > 0, t, _f(1.0)))).astype(np.float32), _f(0.0))
    s, c = sincos_quarter_f32(frac)
    # rotate (cos, sin) of the in-quadrant angle by q quarter turns
    cos_t = np.select([q == 0, q == 1, q == 2], [c, -s, -c], default=s).astype(np.float32)
    sin_t = np.select([q == 0, q == 1, q == 2], [s, c, -s], default=-c).astype(np.float32)
    return (r * cos_t).astype(np.float32), (r * sin_t).astype(np.float32)


def key_of(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & 0xFFFFFFFF, seed >> 32)


def normals(n: int, seed: int, layer: int, which: int, step: int, tag: int = 0,
            start: int = 0) -> np.ndarray:
    """Elements [start, start+n) of the flat normal stream of (seed, layer,
    which, step, tag) as fp32."""
    if n <= 0:
        return np.zeros(0, dtype=np.float32)
    g0 = start // 4
    g1 = (start + n + 3) // 4
    j = np.arange(g0, g1, dtype=np.uint64)
    w1 = np.full_like(j, (2 * int(layer) + int(which)) & 0xFFFFFFFF)
    w2 = np.full_like(j, int(step) & 0xFFFFFFFF)
    w3 = np.full_like(j, int(tag) & 0xFFFFFFFF)
    x0, x1, x2, x3 = philox4x32_10((j, w1, w2, w3), key_of(seed))
    z0, z1 = box_muller_f32(x0, x1)
    z2, z3 = box_muller_f32(x2, x3)
    z = np.stack([z0, z1, z2, z3], axis=1).reshape(-1)
    off = start - 4 * g0
    return z[off:off + n].copy()


def threshold_normal(seed: int, layer: int, step: int) -> np.float32:
    """The single normal of the adaptive-threshold noise (tag 1)."""
    return normals(1, seed, layer, 0, step, tag=1)[0]


def normals_at(indices, seed: int, layer: int, which: int, step: int, tag: int = 0) -> np.ndarray:
    """Elements at the given flat indices of the stream of (seed, layer,
    which, step, tag): element e is lane e % 4 of the group e // 4."""
    idx = np.asarray(indices, dtype=np.int64)
    j = (idx // 4).astype(np.uint64)
    w1 = np.full_like(j, (2 * int(layer) + int(which)) & 0xFFFFFFFF)
    w2 = np.full_like(j, int(step) & 0xFFFFFFFF)
    w3 = np.full_like(j, int(tag) & 0xFFFFFFFF)
    x0, x1, x2, x3 = philox4x32_10((j, w1, w2, w3), key_of(seed))
    z0, z1 = box_muller_f32(x0, x1)
    z2, z3 = box_muller_f32(x2, x3)
    z = np.stack([z0, z1, z2, z3], axis=1)
    return z[np.arange(idx.shape[0]), idx % 4].astype(np.float32)


def weight_noise(d: int, p: int, seed: int, layer: int, step: int) -> np.ndarray:
    """The [d, p] weight-noise array: element (m, n) is lane m % 4 of the
    block of group (m // 4) * p + n (which = 0, tag = 0)."""
    nq = (d + 3) // 4
    flat = normals(4 * nq * p, seed, layer, 0, step)      # group j = q * p + n, lanes 0..3
    z = flat.reshape(nq, p, 4).transpose(0, 2, 1).reshape(4 * nq, p)
    return np.ascontiguousarray(z[:d])


def weight_noise_at(rows, cols, p: int, seed: int, layer: int, step: int) -> np.ndarray:
    """Entries (rows[k], cols[k]) of weight_noise(d, p, ...)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    flat_idx = 4 * ((rows // 4) * p + cols) + rows % 4
    return normals_at(flat_idx, seed, layer, 0, step)
