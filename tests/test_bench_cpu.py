"""Host-side pieces of bench.py (CPU only): the algorithmic flop and byte
counts the roofline divides by, and the refusal of more than one GPU."""
import subprocess
import sys

import pytest

import bench
import workloads as W


def test_algorithmic_counts_follow_the_cost_formulas():
    """Ghost: the Grams' unique entries B*T(T+1)(d+p) plus 2BT^2 for the
    Frobenius product; explicit: 2BTdp + 2Bdp; T = 1: 2B(d+p); contraction:
    2BT(d + bias)p. Bytes: one read of A and G (+ the norm vector or the
    output)."""
    wl = W.WORKLOADS["gpt-block-t128"]
    B, eb = wl.B, 2
    T, d, p = 128, 768, 2304
    f, b = bench._algorithmic(wl, T, d, p, "norm", 0)           # p*d >= T^2: ghost
    assert f == B * T * (T + 1) * (d + p) + 2 * B * T * T
    assert b == B * T * (d + p) * eb + 4 * B
    f, b = bench._algorithmic(wl, T, d, p, "sum")
    assert f == 2 * B * T * d * p
    assert b == B * T * (d + p) * eb + 4 * d * p + 4 * B
    r = W.WORKLOADS["resnet18-conv-t1024"]
    f, _ = bench._algorithmic(r, 1024, 576, 64, "norm", 0)       # p*d < T^2: explicit
    assert f == 2 * r.B * 1024 * 576 * 64 + 2 * r.B * 576 * 64
    m = W.WORKLOADS["mlp-b65536-adaptive"]                       # T = 1, with a bias
    f, b = bench._algorithmic(m, 1, 1024, 4096, "norm", 0)
    assert f == 2 * m.B * (1024 + 4096) and b == m.B * (1024 + 4096) * 4 + 4 * m.B
    f, _ = bench._algorithmic(m, 1, 1024, 4096, "sum")
    assert f == 2 * m.B * (1024 + 1) * 4096


def test_algorithmic_bytes_of_a_folded_conv_input():
    """A folded conv layer reads C_in*H*W elements per sample instead of the
    unfolded T*d; the flops do not change."""
    r = W.WORKLOADS["resnet18-conv-t1024"]
    T, d, p = r.layer_shape(1)
    cin, h, w, _ = r.conv[1]
    f0, b0 = bench._algorithmic(r, T, d, p, "sum")
    f1, b1 = bench._algorithmic(r, T, d, p, "sum", a_elems=cin * h * w)
    assert f0 == f1
    assert b0 - b1 == r.B * (T * d - cin * h * w) * 4
    assert T * d == 9 * cin * h * w  # 3x3 at stride 1: nine times the folded input


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
