"""Pins of the oracle's TQ-QKV key path (oracle/qjl.py).

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression" summary, "Experimental setup" and "Key contributions" 1-2; the
estimator is the published QJL one (Zandieh, Daliri and Han, 2024).  The pins
are what the estimator's definition fixes: unbiasedness and its closed-form
variance over draws of S, convergence as m grows, the residual's norm, the
Jensen inflation the page describes, and the bit layout.
"""
import math

import numpy as np

from oracle import codebook as cb
from oracle import codec, qjl

D = 64


def setup(seed=0, d=D):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, d))
    q = rng.standard_normal((1, d)) * 0.7
    signs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    c4 = cb.codebook_f32(d, 4)
    return rng, x, q, signs, c4


def residual_estimate(q, enc, signs, c4, S):
    """QJL estimate of <q, e> (the correction term alone, scale 1)."""
    full = qjl.logits_qjl(q, enc["codes"], enc["norms"], enc["bits"], enc["gamma"], signs, c4[0],
                          S, 1.0)
    return float(full[0, 0] - qjl.logits_tq(q, enc["codes"], enc["norms"], signs, c4[0], 1.0)[0, 0])


def exact_residual_product(x, q, enc, signs, c4):
    xh = codec.decode(enc["codes"], enc["norms"], signs, c4[0])
    return float(q[0] @ (x[0] - xh[0])), float(np.linalg.norm(x[0] - xh[0]))


def test_gamma_is_the_norm_of_the_key_error():
    rng, x, q, signs, c4 = setup(1)
    S = rng.standard_normal((D, D))
    enc = qjl.encode(x, signs, c4[1], c4[0], S)
    _, enorm = exact_residual_product(x, q, enc, signs, c4)
    assert abs(float(enc["gamma"][0]) - enorm) <= 1e-6 * enorm


def test_estimate_is_unbiased_with_the_closed_form_variance():
    rng, x, q, signs, c4 = setup(2)
    S0 = rng.standard_normal((D, D))
    enc0 = qjl.encode(x, signs, c4[1], c4[0], S0)
    qe, enorm = exact_residual_product(x, q, enc0, signs, c4)
    n = 3000
    est = np.empty(n)
    for i in range(n):
        S = rng.standard_normal((D, D))
        enc = qjl.encode(x, signs, c4[1], c4[0], S)
        est[i] = residual_estimate(q, enc, signs, c4, S)
    # one row: Var[sqrt(pi/2) ||e|| <g,q> sign<g,e>] = pi/2 ||e||^2 ||q||^2 - <q,e>^2
    var = (math.pi / 2 * enorm ** 2 * float(q[0] @ q[0]) - qe ** 2) / D
    assert abs(est.mean() - qe) < 4 * math.sqrt(var / n)
    assert abs(est.var() / var - 1) < 0.1


def test_estimate_converges_as_the_sketch_grows():
    rng, x, q, signs, c4 = setup(3)
    m = 40000
    S = rng.standard_normal((m, D))
    enc = qjl.encode(x, signs, c4[1], c4[0], S)
    qe, enorm = exact_residual_product(x, q, enc, signs, c4)
    var = (math.pi / 2 * enorm ** 2 * float(q[0] @ q[0]) - qe ** 2) / m
    assert abs(residual_estimate(q, enc, signs, c4, S) - qe) < 5 * math.sqrt(var)


def test_jensen_inflation_of_softmax_weights():
    # a zero-mean correction of variance sigma^2 inflates E[exp(s)] by about
    # exp(sigma^2 / 2) (the page's Jensen mechanism for the key path)
    rng, x, q, signs, c4 = setup(5)
    q = q * 0.6  # correction variance about 0.5
    n = 3000
    s = np.empty(n)
    for i in range(n):
        S = rng.standard_normal((D, D))
        enc = qjl.encode(x, signs, c4[1], c4[0], S)
        s[i] = qjl.logits_qjl(q, enc["codes"], enc["norms"], enc["bits"], enc["gamma"], signs,
                              c4[0], S, 1.0)[0, 0]
    exact = float(q[0] @ x[0])
    ratio = np.exp(s - exact).mean()
    assert 0.2 < s.var() < 1.0
    assert ratio > 1.0
    assert abs(ratio / math.exp(s.var() / 2) - 1) < 0.05


def test_sketch_bit_layout():
    bits = np.zeros((1, 16), dtype=bool)
    bits[0, [0, 9, 15]] = True
    np.testing.assert_array_equal(qjl.pack_bits(bits), np.array([[0x01, 0x82]], np.uint8))
    np.testing.assert_array_equal(qjl.unpack_bits(qjl.pack_bits(bits), 16), bits)
