"""Beta Lloyd-Max codebook (oracle, fp64).  TEST INFRASTRUCTURE ONLY.

Source: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", technical summary, "Experimental setup": TurboQuant spreads a
token's energy with a random Walsh-Hadamard transform and then quantises with a
data-oblivious Beta Lloyd-Max codebook, so no calibration data is needed.

Reading taken (the page names the codebook but gives no parameters): after the
rotation, one coordinate Y of a uniformly random unit vector in R^d has density

    f_d(y) = (1 - y^2)^k / Z,   k = (d - 3) / 2,   y in [-1, 1],

i.e. (Y + 1) / 2 ~ Beta((d-1)/2, (d-1)/2).  The codebook for (d, b) is the MSE
Lloyd-Max fixed point with 2^b cells: every centroid is the conditional mean of
its cell, every threshold is the midpoint of its two neighbouring centroids.

Closed forms used:
  CDF      F(t) = I_{(1+t)/2}(k+1, k+1)          (regularised incomplete beta)
  moment   int_a^b y f(y) dy = [(1-a^2)^(k+1) - (1-b^2)^(k+1)] / (2 (k+1) Z)
  Z        = B(1/2, k+1)
"""
import functools
import math

import numpy as np
import scipy.special as sps


def _log_z(d):
    k = (d - 3) / 2.0
    return sps.betaln(0.5, k + 1.0)


def cdf(t, d):
    """P(Y <= t) for one coordinate of a uniform unit vector in R^d."""
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    a = (d - 1) / 2.0
    return sps.betainc(a, a, (1.0 + t) / 2.0)


def partial_moment(a, b, d):
    """int_a^b y f_d(y) dy, from the antiderivative -(1-y^2)^(k+1) / (2 (k+1) Z)."""
    k = (d - 3) / 2.0
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)

    def g(y):
        # (1 - y^2)^(k+1) / (2 (k+1) Z), evaluated in log space.
        with np.errstate(divide="ignore"):
            lg = (k + 1.0) * np.log1p(-y * y) - math.log(2.0 * (k + 1.0)) - _log_z(d)
        return np.exp(lg)

    return g(a) - g(b)


def centroids_from_thresholds(thr, d):
    """Conditional mean of every cell delimited by the inner thresholds thr."""
    edges = np.concatenate([[-1.0], np.asarray(thr, dtype=np.float64), [1.0]])
    mass = cdf(edges[1:], d) - cdf(edges[:-1], d)
    mom = partial_moment(edges[:-1], edges[1:], d)
    return mom / mass


def thresholds_from_centroids(c):
    """Lloyd's nearest-neighbour condition: midpoints of neighbouring centroids."""
    c = np.asarray(c, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


def lloyd_max(d, bits, tol=5e-14, max_iter=20000):
    """Lloyd-Max fixed point for f_d with 2^bits cells.

    Returns (centroids[2^bits], thresholds[2^bits - 1]) ascending, in fp64.
    Starts from the equal-mass partition and alternates the two Lloyd
    conditions until the centroids move by less than tol (relative to the
    largest centroid).  fp64 evaluation of the cell masses has a noise floor
    near 1e-14 relative, so tol sits just above it.
    """
    if d < 3:
        raise ValueError("d must be >= 3 for the Beta marginal")
    levels = 1 << bits
    a = (d - 1) / 2.0
    q = np.arange(1, levels) / levels
    thr = 2.0 * sps.betaincinv(a, a, q) - 1.0
    c = centroids_from_thresholds(thr, d)
    for _ in range(max_iter):
        thr = thresholds_from_centroids(c)
        c_new = centroids_from_thresholds(thr, d)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta <= tol * np.max(np.abs(c)):
            break
    # The density is even, so the fixed point is odd-symmetric; remove the
    # last-ulp asymmetry so the middle threshold is exactly 0 and a zero
    # coordinate always takes the lower cell.
    c = 0.5 * (c - c[::-1])
    thr = thresholds_from_centroids(c)
    return c, thr


def distortion(c, thr, d):
    """Per-coordinate MSE E[(Y - Q(Y))^2] of the quantiser (c, thr) under f_d.

    Uses E[Y^2] = 1/d (a unit vector's coordinates have mean square 1/d) and
    the cell identity E[(Y-c_j)^2; cell j] = E[Y^2; cell j] - 2 c_j M_j + c_j^2 P_j,
    where M_j, P_j are the cell's first moment and mass.  With c_j the
    conditional means this reduces to 1/d - sum_j c_j^2 P_j, but the general
    form is kept so a non-fixed-point codebook is also priced correctly.
    """
    edges = np.concatenate([[-1.0], np.asarray(thr, dtype=np.float64), [1.0]])
    mass = cdf(edges[1:], d) - cdf(edges[:-1], d)
    mom = partial_moment(edges[:-1], edges[1:], d)
    c = np.asarray(c, dtype=np.float64)
    return 1.0 / d - np.sum(2.0 * c * mom) + np.sum(c * c * mass)


@functools.lru_cache(maxsize=None)
def codebook_f32(d, bits):
    """The stored codebook the codec consumes, as fp32 arrays.

    The pages fix the codebook (the Beta Lloyd-Max fixed point) but not its
    storage precision; both tables are the fixed point's own values rounded
    to the nearest fp32: centroids c_j, and thresholds (c_j + c_{j+1}) / 2
    formed in fp64 before the rounding.  The stored tables therefore satisfy
    both Lloyd conditions to fp32 rounding.  Exact odd symmetry survives the
    rounding, so the middle threshold is exactly 0.
    """
    c, t = lloyd_max(d, bits)
    c32 = c.astype(np.float32)
    t32 = t.astype(np.float32)
    c32.setflags(write=False)
    t32.setflags(write=False)
    return c32, t32
