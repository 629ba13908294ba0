"""Pins of the oracle's HQQ-style zero refinement (the page names HQQ as its
default quantiser; the steps are the half-quadratic solver's, with the l1
norm's soft threshold as the proximal step) and of its fixed-order sum."""
import math

import numpy as np

from oracle import river_oracle as ro


def test_zero_rounds_is_the_minmax_quantiser():
    rng = np.random.default_rng(3)
    w = ro.bf16_from_f32((rng.standard_normal((16, 256)) * 0.02).astype(np.float32))
    a = ro.quantize_int4(w, 64)
    b = ro.quantize_int4_hqq(w, 64, iters=0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_tree_sum_order_by_hand():
    # eight values whose float32 sum depends on the order of the additions:
    # the fold-halves order is ((a0+a4)+(a2+a6)) + ((a1+a5)+(a3+a7))
    a = np.array([1e8, 3.0, -1e8, 5.0, 1.0, 7.0, 2.0, -4.0], dtype=np.float32)
    f = np.float32
    expect = (f(f(a[0] + a[4]) + f(a[2] + a[6])) + f(f(a[1] + a[5]) + f(a[3] + a[7])))
    assert ro.tree_sum_f32(a) == expect
    # exactly representable integers: the exact sum
    assert ro.tree_sum_f32(np.arange(128, dtype=np.float32)) == 8128.0
    x = np.random.default_rng(1).standard_normal((5, 64)).astype(np.float32)
    for row in x:
        assert abs(float(ro.tree_sum_f32(row)) - math.fsum(row.astype(np.float64))) <= 64 * 2.0 ** -24 * np.abs(row).sum()


def test_refinement_worked_example():
    """Group w = (0, 0.25, 0.5, 7.5), beta 8, kappa 2, two rounds; every
    float32 operation below is exact.
      min-max: s = bf16(7.5 / 15) = 0.5, z = 0, q = rint(0, 0.5, 1, 15) = (0, 0, 1, 15).
      round 1 (threshold 1/8): residual e = w - (q - 0) 0.5 = (0, 0.25, 0, 0);
        we = (0, 0.125, 0, 0); q - (w - we)/s = (0, -0.25, 0, 0); zf = -0.25/4 = -0.0625.
      round 2 (beta 16, threshold 1/16): w/s + zf = (-0.0625, 0.4375, 0.9375, 14.9375)
        -> q = (0, 0, 1, 15); e = w - (q + 0.0625) 0.5 = (-0.03125, 0.21875, -0.03125, -0.03125);
        we = (0, 0.15625, 0, 0); q - (w - we)/s = (0, -0.1875, 0, 0); zf = -0.046875.
      stored: z = bf16(-0.046875) = -0.046875; codes rint(w/s + z) = (0, 0, 1, 15).
    """
    w = np.array([[0.0, 0.25, 0.5, 7.5]], dtype=np.float32)
    q, s, z = ro.quantize_int4_hqq(w, 4, iters=2, beta=8.0, kappa=2.0)
    assert s[0, 0] == 0.5
    assert z[0, 0] == -0.046875
    assert list(q[0]) == [0, 0, 1, 15]
    # one round only stops at zf = -0.0625
    q1, s1, z1 = ro.quantize_int4_hqq(w, 4, iters=1, beta=8.0, kappa=2.0)
    assert z1[0, 0] == -0.0625 and list(q1[0]) == [0, 0, 1, 15]


def test_soft_threshold_is_the_l1_proximal_step():
    """The refinement's error variable minimises beta/2 (x - e)^2 + |x| (the
    proximal step of the l1 norm): with e far above and far below the
    threshold, the refined zero differs from the plain least-squares zero by
    exactly the shrunken outlier's share."""
    # one large outlier in an otherwise exactly representable group
    w = np.array([[0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 30.0]], dtype=np.float32)
    q0, s, z0 = ro.quantize_int4(w, 8)
    # brute force of the proximal problem on a grid for the group's residuals
    beta = 10.0
    for e in (-0.7, -0.05, 0.0, 0.03, 0.4):
        xs = np.linspace(-1, 1, 200001)
        obj = beta / 2 * (xs - e) ** 2 + np.abs(xs)
        best = xs[np.argmin(obj)]
        assert abs(best - np.sign(e) * max(abs(e) - 1 / beta, 0.0)) < 2e-5
    q, s2, z = ro.quantize_int4_hqq(w, 8)
    assert np.array_equal(s, s2) and q.min() >= 0 and q.max() <= 15 and np.isfinite(z).all()


def test_refinement_lowers_the_reconstruction_error():
    """On weights of the configs' distribution the refined zero points give a
    lower mean squared and mean absolute reconstruction error than min-max."""
    rng = np.random.default_rng(0)
    w = ro.bf16_from_f32((rng.standard_normal((256, 2048)) * 0.02).astype(np.float32))
    e0 = ro.dequantize_int4(*ro.quantize_int4(w, 128), 128) - w
    e1 = ro.dequantize_int4(*ro.quantize_int4_hqq(w, 128), 128) - w
    assert (e1 ** 2).mean() < 0.97 * (e0 ** 2).mean()
    assert np.abs(e1).mean() < np.abs(e0).mean()
