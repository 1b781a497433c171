"""Pins of the oracle's TurboQuant codec: rotation, quantiser, packing, round trip.

Pages: "Tamarin (HSQ)" summary, section 2, "Key technical components"
(rotation + scalar quantisation, 4-bit L1/L3, 3-bit L2); "Ablation,
Statistical Inference, and Validation for KV-Cache Compression", technical
summary, "Experimental setup" (random Walsh-Hadamard transform, Beta Lloyd-Max).
"""
import json
import os

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sylvester(d):
    """Hadamard matrix by Sylvester's doubling H_2n = [[H, H], [H, -H]]."""
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_popcount_equals_sylvester(d):
    np.testing.assert_array_equal(codec.hadamard(d), sylvester(d))
    h = codec.hadamard(d)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthonormal(d):
    rng = np.random.default_rng(5)
    words = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    r = codec.rotation_matrix(words, d)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-12)
    x = rng.standard_normal(d)
    np.testing.assert_allclose(np.linalg.norm(r @ x), np.linalg.norm(x), rtol=1e-13)
    np.testing.assert_allclose(r.T @ (r @ x), x, atol=1e-12)
    # the first basis vector maps to s_0 * (1, ..., 1) / sqrt(d)
    s = codec.sign_vector(words, d)
    np.testing.assert_allclose(r[:, 0], s[0] * np.ones(d) / np.sqrt(d), atol=0)


def test_sign_mask_bit_order():
    # bit i of word i // 32 negates coordinate i
    words = np.zeros(2, dtype=np.uint32)
    words[0] = 1 << 3
    words[1] = 1 << 31
    s = codec.sign_vector(words, 64)
    neg = np.nonzero(s < 0)[0].tolist()
    assert neg == [3, 63]


@pytest.mark.parametrize("bits", [3, 4])
def test_threshold_count_equals_nearest_centroid(bits):
    # brute force: argmin_j |y - c_j| against the fp64 fixed-point centroids,
    # first index on ties.  The stored thresholds are the fp32 roundings of
    # those centroids' midpoints, so the threshold count agrees with the brute
    # force everywhere except between a midpoint and its fp32 rounding (half
    # an fp32 ulp wide); a value exactly on a stored threshold goes to the
    # lower cell.
    d = 128
    c64, m64 = cb.lloyd_max(d, bits)
    c32, t32 = cb.codebook_f32(d, bits)
    rng = np.random.default_rng(7)
    y = rng.standard_normal(10 ** 6) / np.sqrt(d)
    j = rng.integers(0, len(t32), 1000)
    y[:1000] = t32[j]                                   # values exactly on thresholds
    y[1000:2000] = np.nextafter(t32[j].astype(np.float64), np.inf)  # just above
    brute = np.argmin(np.abs(y[:, None] - c64[None, :]), axis=1)
    count = np.sum(y[:, None] > t32.astype(np.float64)[None, :], axis=1)
    np.testing.assert_array_equal(count[:1000], j)
    np.testing.assert_array_equal(count[1000:2000], j + 1)
    t = t32.astype(np.float64)
    lo = np.minimum(t, m64)
    hi = np.maximum(t, m64)
    between = np.any((y[:, None] >= lo[None, :]) & (y[:, None] <= hi[None, :]), axis=1)
    assert np.all(np.abs(t - m64) <= 0.5 * np.spacing(np.abs(t32)).astype(np.float64))
    # the generic draws (all but the planted ones, which sit closer to a
    # threshold than fp64 can resolve against the centroids) agree except
    # inside the half-ulp bands, where they essentially never fall
    gen = ~between
    gen[:2000] = False
    np.testing.assert_array_equal(brute[gen], count[gen])
    assert between[2000:].sum() <= 2


def test_pack_fixed_patterns():
    with open(os.path.join(GOLDEN, "pack_patterns.json")) as f:
        g = json.load(f)
    c4 = np.array([g["codes4"]], dtype=np.uint8)
    assert codec.pack(c4, 4).tolist()[0] == g["bytes4"]
    c3 = np.array([g["codes3"]], dtype=np.uint8)
    assert codec.pack(c3, 3).tolist()[0] == g["bytes3"]


@pytest.mark.parametrize("bits,d", [(3, 64), (3, 128), (4, 64), (4, 128)])
def test_pack_roundtrip(bits, d):
    rng = np.random.default_rng(bits * d)
    codes = rng.integers(0, 1 << bits, size=(50, d)).astype(np.uint8)
    packed = codec.pack(codes, bits)
    assert packed.shape == (50, bits * d // 8)
    np.testing.assert_array_equal(codec.unpack(packed, bits, d), codes)


def test_pack3_bit_positions():
    # one code set at a time: code i with value v sets bits 3i.. of the stream
    d = 64
    for i in (0, 1, 2, 10, 21, 42, 63):
        for v in (1, 2, 4, 7):
            codes = np.zeros((1, d), dtype=np.uint8)
            codes[0, i] = v
            p = codec.pack(codes, 3)[0]
            stream_bits = [(int(p[j // 8]) >> (j % 8)) & 1 for j in range(3 * d)]
            want = [0] * (3 * d)
            for b in range(3):
                want[3 * i + b] = (v >> b) & 1
            assert stream_bits == want


@pytest.mark.parametrize("bits", [3, 4])
def test_zero_vector_takes_lower_middle_cell(bits):
    c32, t32 = cb.codebook_f32(64, bits)
    words = np.zeros(2, dtype=np.uint32)
    codes, norms, _ = codec.encode(np.zeros((1, 64)), words, t32)
    assert norms[0] == 0
    assert np.all(codes == (1 << (bits - 1)) - 1)
    np.testing.assert_array_equal(codec.decode(codes, norms, words, c32), np.zeros((1, 64)))


@pytest.mark.parametrize("d,bits", [(64, 4), (128, 4), (128, 3)])
def test_round_trip_error_matches_distortion(d, bits):
    # E ||x - x_hat||^2 / ||x||^2 = d * D(d, b) for isotropic x, any rotation
    c32, t32 = cb.codebook_f32(d, bits)
    c64, thr64 = cb.lloyd_max(d, bits)
    rng = np.random.default_rng(11)
    words = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    x = rng.standard_normal((4000, d)) * 3.0
    codes, norms, _ = codec.encode(x, words, t32)
    xh = codec.decode(codes, norms, words, c32)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    pred = d * cb.distortion(c64, thr64, d)
    assert abs(rel.mean() - pred) / pred < 0.03


def test_rotation_spreads_an_outlier_channel():
    # a one-hot vector has all its energy in one coordinate; after H D / sqrt(d)
    # every coordinate carries 1/d of it (the page's energy-spreading claim).
    d = 128
    words = np.arange(4, dtype=np.uint32) * 0x9E3779B9
    x = np.zeros((1, d))
    x[0, 17] = 5.0
    _, _, y = codec.encode(x, words, cb.codebook_f32(d, 4)[1])
    np.testing.assert_allclose(np.abs(y), 1 / np.sqrt(d), atol=1e-15)


def test_encode_is_scale_invariant_and_rotation_consistent():
    d = 64
    c32, t32 = cb.codebook_f32(d, 4)
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 32, size=2, dtype=np.uint64).astype(np.uint32)
    x = rng.standard_normal((20, d))
    c1, n1, y1 = codec.encode(x, words, t32)
    c2, n2, y2 = codec.encode(x * 4.0, words, t32)  # power of two: exact scaling
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_allclose(n2, 4.0 * n1, rtol=0)
    # y is R (x / r) computed by an explicit matrix; check one row by FWHT-free
    # direct sum over the popcount definition
    s = codec.sign_vector(words, d)
    u = x[0] / np.linalg.norm(x[0])
    direct = np.array([sum(((-1) ** bin(i & j).count("1")) * s[j] * u[j] for j in range(d))
                       for i in range(d)]) / np.sqrt(d)
    np.testing.assert_allclose(y1[0], direct, atol=1e-14)


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4)])
def test_exact_zero_coordinate_takes_lower_cell(d, bits):
    # x = e_0 + e_1 with no sign flips: (H x)_i = 1 + (-1)^(i & 1), exactly 0
    # for every odd i.  A coordinate equal to the middle threshold (0) belongs
    # to the lower cell, so odd coordinates get code 2^(b-1) - 1.
    c32, t32 = cb.codebook_f32(d, bits)
    x = np.zeros((1, d))
    x[0, 0] = x[0, 1] = 1.0
    codes, _, y = codec.encode(x, np.zeros(d // 32, dtype=np.uint32), t32)
    assert np.all(y[0, 1::2] == 0.0)
    assert np.all(codes[0, 1::2] == (1 << (bits - 1)) - 1)
    assert np.all(y[0, 0::2] > 0)
