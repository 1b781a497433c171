"""Pins of the oracle's codec variants: 2-bit packing and codebook, and
Plain-KV (the rotation off).

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", technical summary: "Key contributions" item 1 (the three
non-dominated methods, among them Plain-KV, scalar quantisation without a
rotation, effective on isotropic data) and "Results and recommendations"
(at a 2-bit budget no method dominates; TQ-KV wins on heavy tails because the
Walsh-Hadamard transform spreads the outliers).
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import codebook as cb
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack2_golden():
    with open(os.path.join(GOLDEN, "pack_patterns.json")) as f:
        g = json.load(f)
    c2 = np.array([g["codes2"]], dtype=np.uint8)
    assert codec.pack(c2, 2).tolist()[0] == g["bytes2"]


@pytest.mark.parametrize("d", [64, 128])
def test_pack2_is_the_lsb_first_stream(d):
    # the stream written out bit by bit: bit j of the row is bit (j % 2) of
    # code j // 2, bit j lands in byte j // 8 at position j % 8
    rng = np.random.default_rng(d)
    codes = rng.integers(0, 4, size=(40, d)).astype(np.uint8)
    stream = np.zeros((40, 2 * d), dtype=np.uint8)
    for j in range(2 * d):
        stream[:, j] = (codes[:, j // 2] >> (j % 2)) & 1
    want = np.zeros((40, d // 4), dtype=np.uint8)
    for j in range(2 * d):
        want[:, j // 8] |= (stream[:, j] << (j % 8)).astype(np.uint8)
    packed = codec.pack(codes, 2)
    np.testing.assert_array_equal(packed, want)
    np.testing.assert_array_equal(codec.unpack(packed, 2, d), codes)


@pytest.mark.parametrize("d", [64, 128])
def test_two_bit_codebook_cells(d):
    # four cells, symmetric, threshold 0 in the middle, and every stored
    # threshold the midpoint of its stored neighbours to fp32 rounding
    c32, t32 = cb.codebook_f32(d, 2)
    assert c32.shape == (4,) and t32.shape == (3,)
    np.testing.assert_array_equal(c32, -c32[::-1])
    assert t32[1] == 0.0
    mid = 0.5 * (c32[:-1].astype(np.float64) + c32[1:].astype(np.float64))
    assert np.all(np.abs(t32.astype(np.float64) - mid) <= np.spacing(np.abs(t32)).astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_plain_basis_vector(bits):
    # R = I: a scaled basis vector s e_k has y = sign(s) e_k, so coordinate k
    # takes the top (or bottom) cell and every other coordinate is exactly 0,
    # which lies on the middle threshold and goes to the lower cell L/2 - 1
    d, L = 64, 1 << bits
    c32, t32 = cb.codebook_f32(d, bits)
    x = np.zeros((2, d))
    x[0, 5] = 3.5
    x[1, 40] = -0.25
    codes, norms, y = codec.encode(x, None, t32)
    np.testing.assert_array_equal(norms, np.array([3.5, 0.25], dtype=np.float32))
    want = np.full((2, d), L // 2 - 1, dtype=np.uint8)
    want[0, 5] = L - 1
    want[1, 40] = 0
    np.testing.assert_array_equal(codes, want)
    xh = codec.decode(codes, norms, None, c32)
    np.testing.assert_allclose(xh[0, 5], 3.5 * float(c32[-1]), rtol=1e-15)
    np.testing.assert_allclose(xh[1, 0], 0.25 * float(c32[L // 2 - 1]), rtol=1e-15)


@pytest.mark.parametrize("bits", [2, 4])
def test_rotated_equals_plain_of_rotated_input(bits):
    # TQ-KV of x is Plain-KV of R x (R orthonormal keeps the norm), with R
    # built here from scipy's Sylvester Hadamard matrix and the sign diagonal
    d = 128
    rng = np.random.default_rng(17 + bits)
    words = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    bit = (words[np.arange(d) // 32] >> (np.arange(d) % 32).astype(np.uint32)) & 1
    R = scipy.linalg.hadamard(d) * np.where(bit == 1, -1.0, 1.0)[None, :] / np.sqrt(d)
    x = rng.standard_normal((300, d))
    _, t32 = cb.codebook_f32(d, bits)
    c_rot, n_rot, y_rot = codec.encode(x, words, t32)
    c_pl, n_pl, y_pl = codec.encode(x @ R.T, None, t32)
    np.testing.assert_allclose(y_pl, y_rot, atol=1e-13)
    np.testing.assert_allclose(n_pl, n_rot, rtol=1e-6)
    near = np.min(np.abs(y_rot[:, :, None] - t32[None, None, :].astype(np.float64)), axis=2) < 1e-9
    assert np.array_equal(c_rot[~near], c_pl[~near])


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 2), (128, 3)])
def test_plain_on_isotropic_data_meets_the_codebook(d, bits):
    # isotropic Gaussian rows: x / r is a uniform unit vector, so with the
    # rotation off every coordinate already follows the Beta marginal; the
    # cell frequencies and the MSE are those the codebook predicts
    rng = np.random.default_rng(100 + d + bits)
    n = 40000
    x = rng.standard_normal((n, d))
    c32, t32 = cb.codebook_f32(d, bits)
    codes, norms, y = codec.encode(x, None, t32)
    edges = np.concatenate([[-1.0], t32.astype(np.float64), [1.0]])
    mass = cb.cdf(edges[1:], d) - cb.cdf(edges[:-1], d)
    counts = np.bincount(codes.reshape(-1), minlength=1 << bits)
    expected = mass * codes.size
    assert np.all(np.abs(counts - expected) < 6 * np.sqrt(2 * expected) + 1)
    emp = np.mean((y - c32.astype(np.float64)[codes]) ** 2)
    pred = cb.distortion(c32.astype(np.float64), t32.astype(np.float64), d)
    assert abs(emp - pred) / pred < 0.02


@pytest.mark.parametrize("bits", [2, 4])
def test_rotation_wins_on_heavy_tails_and_ties_on_isotropic_data(bits):
    # the ablation's finding in the two regimes: with a few large-scale
    # channels (heavy tails) the rotated codec has the lower relative MSE;
    # on isotropic data the two agree to sampling error
    d, n = 128, 4000
    rng = np.random.default_rng(7 + bits)
    words = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    c32, t32 = cb.codebook_f32(d, bits)

    def relmse(x, signs):
        codes, norms, _ = codec.encode(x, signs, t32)
        xh = codec.decode(codes, norms, signs, c32)
        return np.sum((xh - x) ** 2) / np.sum(x * x)

    z = rng.standard_normal((n, d)) / np.sqrt(rng.chisquare(3, size=(n, d)) / 3)
    z[:, rng.choice(d, size=4, replace=False)] *= 20.0
    assert relmse(z, words) < 0.8 * relmse(z, None)
    g = rng.standard_normal((n, d))
    a, b = relmse(g, words), relmse(g, None)
    assert abs(a - b) / b < 0.03
