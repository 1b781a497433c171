"""Pins of the oracle's pre-RoPE fetch path (oracle/rope.py).

Page: "Tamarin (HSQ)" summary, section 2, "Decode process", fetching step;
RoPE as defined by Su et al. (RoFormer, 2021), half-split pairing.  The pins
are what that definition fixes: a worked case computed by hand (pairing,
sign and frequencies), the identity at position 0, norm preservation, the
relative-position property of the inner product, composition of positions,
and that the fetch path is the codec's dequantisation followed by RoPE.
"""
import math

import numpy as np

from oracle import codebook as cb
from oracle import codec, rope


def test_worked_case_d4():
    # d = 4, base = 1e4: theta = (1, 0.01); pairs (x0, x2) and (x1, x3)
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = rope.rope(x, [2], 1e4)[0]
    c0, s0 = math.cos(2.0), math.sin(2.0)
    c1, s1 = math.cos(0.02), math.sin(0.02)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_unit_vector_traces_the_circle():
    # e_0 at position p goes to cos(p) e_0 + sin(p) e_{d/2}, whatever d and base
    d = 128
    x = np.zeros((3, d))
    x[:, 0] = 1
    got = rope.rope(x, [0, 1, 1000], 1e6)
    for k, p in enumerate([0, 1, 1000]):
        want = np.zeros(d)
        want[0], want[d // 2] = math.cos(p), math.sin(p)
        np.testing.assert_allclose(got[k], want, rtol=0, atol=1e-12)


def test_highest_pair_frequency():
    # the last pair turns by base^(-(d-2)/d) per position
    d, base = 64, 1e6
    x = np.zeros((1, d))
    x[0, d // 2 - 1] = 1
    p = 12345
    a = p * base ** (-(d - 2) / d)
    got = rope.rope(x, [p], base)[0]
    assert abs(got[d // 2 - 1] - math.cos(a)) < 1e-12
    assert abs(got[d - 1] - math.sin(a)) < 1e-12


def test_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128))
    np.testing.assert_array_equal(rope.rope(x, np.zeros(50, int), 1e6), x)
    y = rope.rope(x, rng.integers(-10 ** 6, 10 ** 6, 50), 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_inner_product_depends_on_the_offset_only():
    rng = np.random.default_rng(1)
    d = 64
    q, k = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    ref = float(rope.rope(q, [7], 1e4)[0] @ k[0])
    for m in [7, 100, 5000, 32767]:
        n = m - 7
        v = float(rope.rope(q, [m], 1e4)[0] @ rope.rope(k, [n], 1e4)[0])
        assert abs(v - ref) < 1e-10
    # and a different offset gives a different value
    assert abs(float(rope.rope(q, [8], 1e4)[0] @ k[0]) - ref) > 1e-3


def test_positions_compose_and_invert():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((20, 128))
    a = rng.integers(0, 40000, 20)
    b = rng.integers(-40000, 40000, 20)
    np.testing.assert_allclose(rope.rope(rope.rope(x, a, 1e6), b, 1e6), rope.rope(x, a + b, 1e6),
                               rtol=0, atol=1e-9)
    np.testing.assert_allclose(rope.rope(rope.rope(x, a, 1e6), -a, 1e6), x, rtol=0, atol=1e-9)


def test_fetch_is_dequantise_then_rope():
    rng = np.random.default_rng(3)
    d = 64
    x = rng.standard_normal((30, d))
    signs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    c, t = cb.codebook_f32(d, 4)
    codes, norms, _ = codec.encode(x, signs, t)
    pos = rng.integers(0, 16384, 30)
    got = rope.decode_rope(codes, norms, signs, c, pos, 1e6)
    # RoPE keeps norms, so the fetched row has the dequantised row's norm
    xh = codec.decode(codes, norms, signs, c)
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(xh, axis=1), rtol=1e-12)
    # and rotating back to position 0 recovers the dequantised row
    np.testing.assert_allclose(rope.rope(got, -pos, 1e6), xh, rtol=0, atol=1e-9)
