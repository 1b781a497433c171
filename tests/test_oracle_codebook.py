"""Pins of the oracle's Beta Lloyd-Max codebook against facts fixed by the
mathematics, not by the oracle itself.

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", technical summary, "Experimental setup" (data-oblivious Beta
Lloyd-Max codebook after a random Walsh-Hadamard transform).
"""
import math

import numpy as np
import pytest
import scipy.special as sps

from oracle import codebook as cb


# Gaussian Lloyd-Max quantisers, J. Max, "Quantizing for minimum distortion",
# IRE Trans. Information Theory, 1960, table of optimum output levels for a
# unit-variance normal input (positive half) and the resulting mean-squared
# error.  Four significant digits as printed there.
MAX_1960 = {
    1: ([0.7979], 0.3634),
    2: ([0.4528, 1.510], 0.1175),
    3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454),
    4: ([0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733], 0.009497),
}


def gaussian_lloyd(bits, iters=20000):
    """Independent Lloyd-Max for N(0,1): conditional means from the normal
    pdf/cdf (a different density and different closed forms than the oracle)."""
    L = 1 << bits
    c = np.linspace(-2.5, 2.5, L)
    phi = lambda x: np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    for _ in range(iters):
        t = np.concatenate([[-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]])
        mass = sps.ndtr(t[1:]) - sps.ndtr(t[:-1])
        pa = np.where(np.isinf(t[:-1]), 0.0, phi(np.where(np.isinf(t[:-1]), 0, t[:-1])))
        pb = np.where(np.isinf(t[1:]), 0.0, phi(np.where(np.isinf(t[1:]), 0, t[1:])))
        c_new = (pa - pb) / mass
        if np.max(np.abs(c_new - c)) < 1e-15:
            c = c_new
            break
        c = c_new
    t = 0.5 * (c[1:] + c[:-1])
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    # MSE = 1 - sum c_j^2 P_j for conditional-mean centroids of a unit-variance law
    mass = sps.ndtr(edges[1:]) - sps.ndtr(edges[:-1])
    return c, 1.0 - np.sum(c * c * mass)


@pytest.mark.parametrize("d,bits", [(64, 3), (64, 4), (128, 3), (128, 4), (16, 2), (1024, 4)])
def test_lloyd_fixed_point_and_symmetry(d, bits):
    c, t = cb.lloyd_max(d, bits)
    assert np.all(np.diff(c) > 0)
    # nearest-neighbour and centroid conditions hold simultaneously
    np.testing.assert_allclose(t, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=1e-16)
    np.testing.assert_allclose(cb.centroids_from_thresholds(t, d), c, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(c, -c[::-1])
    assert t[len(t) // 2] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_uniform_quantiser(bits):
    # d = 3: (Y+1)/2 ~ Beta(1,1), Y uniform on [-1,1] (Archimedes' hat-box
    # theorem); the Lloyd-Max quantiser of a uniform law is the uniform one.
    L = 1 << bits
    c, t = cb.lloyd_max(3, bits)
    np.testing.assert_allclose(c, (2 * np.arange(L) + 1 - L) / L, atol=1e-12)
    # uniform quantiser of step D on a unit-variance-1/3 law: MSE = D^2 / 12
    assert abs(cb.distortion(c, t, 3) - (2.0 / L) ** 2 / 12) < 1e-12
    assert abs(3 * cb.distortion(c, t, 3) - 4.0 ** (-bits)) < 1e-12


@pytest.mark.parametrize("d", [4, 8, 64, 128, 1000])
def test_one_bit_closed_form(d):
    # 1 bit: threshold 0, centroids +-E|Y| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, t = cb.lloyd_max(d, 1)
    e_abs = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert t[0] == 0.0
    np.testing.assert_allclose(c, [-e_abs, e_abs], rtol=1e-12)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_limit(bits):
    # sqrt(d) Y -> N(0,1) as d grows; at d = 2^16 the gap is O(1/d).
    d = 1 << 16
    c, t = cb.lloyd_max(d, bits)
    g, g_mse = gaussian_lloyd(bits)
    np.testing.assert_allclose(math.sqrt(d) * c, g, rtol=2e-4, atol=2e-5)
    assert abs(d * cb.distortion(c, t, d) - g_mse) < 2e-5
    levels, mse = MAX_1960[bits]
    half = math.sqrt(d) * c[len(c) // 2:]
    np.testing.assert_allclose(half, levels, rtol=1e-3)
    assert abs(d * cb.distortion(c, t, d) - mse) / mse < 2e-3


@pytest.mark.parametrize("bits", [3, 4])
def test_dmse_rises_monotonically_toward_gaussian(bits):
    _, g_mse = gaussian_lloyd(bits)
    vals = []
    for d in (8, 16, 32, 64, 128, 256, 1024):
        c, t = cb.lloyd_max(d, bits)
        vals.append(d * cb.distortion(c, t, d))
    assert all(a < b for a, b in zip(vals, vals[1:]))
    assert vals[-1] < g_mse


@pytest.mark.parametrize("d,bits,n", [(16, 3, 200000), (16, 4, 200000), (128, 4, 40000), (64, 3, 60000)])
def test_monte_carlo_marginal_and_mse(d, bits, n):
    # Coordinates of uniform unit vectors (normalised Gaussians) must fall in
    # the cells with the probabilities the Beta CDF predicts, and the
    # empirical MSE of the fp32 codebook must match the predicted distortion.
    rng = np.random.default_rng(1234 + d + bits)
    x = rng.standard_normal((n, d))
    u = (x / np.linalg.norm(x, axis=1, keepdims=True)).reshape(-1)
    c, t = cb.lloyd_max(d, bits)
    edges = np.concatenate([[-1.0], t, [1.0]])
    mass = cb.cdf(edges[1:], d) - cb.cdf(edges[:-1], d)
    counts = np.bincount(np.searchsorted(t, u, side="left"), minlength=len(c))
    expected = mass * u.size
    # coordinates of one vector are weakly dependent; allow 6 sigma of a
    # multinomial with a factor 2 for that dependence
    assert np.all(np.abs(counts - expected) < 6 * np.sqrt(2 * expected) + 1)
    q = c[np.searchsorted(t, u, side="left")]
    emp = np.mean((u - q) ** 2)
    pred = cb.distortion(c, t, d)
    assert abs(emp - pred) / pred < 0.02


@pytest.mark.parametrize("d,bits", [(128, 4), (128, 3), (64, 4), (64, 3), (128, 2), (64, 2)])
def test_stored_tables_are_the_fixed_point_in_fp32(d, bits):
    # The stored fp32 tables satisfy both Lloyd conditions to fp32 rounding:
    # each stored centroid is the fp32 value nearest to the conditional mean
    # of its cell under the fp64 thresholds, and each stored threshold is the
    # fp32 value nearest to the midpoint of the fp64 centroids.  The
    # conditional means are recomputed here by adaptive quadrature of the
    # density (scipy.integrate.quad), not by the oracle's closed forms.
    from scipy import integrate
    c, t = cb.lloyd_max(d, bits)
    c32, t32 = cb.codebook_f32(d, bits)
    k = (d - 3) / 2.0
    f = lambda y: (1.0 - y * y) ** k
    edges = np.concatenate([[-1.0], t, [1.0]])
    for j in range(len(c)):
        m0 = integrate.quad(f, edges[j], edges[j + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda y: y * f(y), edges[j], edges[j + 1], epsabs=0,
                            epsrel=1e-13, limit=200)[0]
        cond_mean = m1 / m0
        # within half an fp32 ulp (plus the quadrature's own error)
        assert abs(float(c32[j]) - cond_mean) <= 0.5 * np.spacing(np.float32(abs(cond_mean))) * 1.001 + 1e-15
    mid = 0.5 * (c[:-1] + c[1:])
    for j in range(len(t)):
        assert abs(float(t32[j]) - mid[j]) <= 0.5 * float(np.spacing(np.float32(abs(mid[j])))) + 1e-300
    # exact odd symmetry survives the rounding; middle threshold 0; order kept
    np.testing.assert_array_equal(c32, -c32[::-1])
    np.testing.assert_array_equal(t32, -t32[::-1])
    assert t32[len(t32) // 2] == 0.0 and np.all(np.diff(t32) > 0) and np.all(np.diff(c32) > 0)
    # every threshold separates its two centroids
    assert np.all((c32[:-1] < t32) & (t32 < c32[1:]))
