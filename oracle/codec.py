"""TurboQuant codec (oracle, fp64).  TEST INFRASTRUCTURE ONLY.

Sources:
* "Tamarin (HSQ)" summary, section 2, "Key technical components",
  quantisation item: randomised scalar quantisation after a fixed random
  orthonormal rotation that decorrelates coordinates; L1 and L3 at 4 bits,
  L2 at 3 bits.
* "Ablation, Statistical Inference, and Validation for KV-Cache Compression",
  technical summary, "Experimental setup": the rotation is a random
  Walsh-Hadamard transform, the quantiser a data-oblivious Beta Lloyd-Max
  codebook.

Readings taken where the pages are silent:
* Rotation R = H_d D / sqrt(d): D = diag(s) with s_i = -1 where bit i of the
  sign mask is set, applied first; H_d the Sylvester-ordered Hadamard matrix
  H_ij = (-1)^popcount(i & j).  One D per (layer, kv-head, K|V), shared by
  every tier.  Sign masks are input data: uint32 words, bit i of word i // 32.
* Norm: r = ||x||_2 of the input vector, stored as fp32.  The unit vector
  x / r is rotated and quantised; r = 0 stores 0 and quantises the zero vector.
  Dequantisation is x_hat = r * R^T c[code] (no re-normalisation).
* Quantisation is deterministic: code_i = #{j : t_j < y_i} against the fp32
  thresholds, i.e. a value equal to a threshold goes to the lower cell, which
  equals nearest-centroid with ties to the lower index.
* Packing: 4-bit, byte k = code[2k] | code[2k+1] << 4.  3-bit, an LSB-first
  bit stream, code i in bits [3i, 3i+3), bit j in byte j // 8 at position j % 8.
  2-bit, the same stream: byte k = code[4k] | code[4k+1] << 2 | code[4k+2] << 4
  | code[4k+3] << 6.

Variants from the same page's ablation (its list of non-dominated methods and
its results at a 2-bit budget):
* Plain-KV, scalar quantisation with the rotation off.  Reading: R = I, every
  other step unchanged (norm, the same Beta Lloyd-Max codebook for (d, b),
  threshold count, packing); sign_words=None selects it.  On isotropic data
  x / r is already a uniform unit vector, so the codebook fits it exactly.
* b = 2: a four-cell codebook of the same family.
"""
import numpy as np


def hadamard(d):
    """Sylvester-ordered Hadamard matrix, entries (-1)^popcount(i & j)."""
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    andm = i[:, None] & i[None, :]
    pop = np.zeros_like(andm)
    x = andm.copy()
    while np.any(x):
        pop += x & 1
        x >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def sign_vector(sign_words, d):
    """+-1 diagonal of D from a uint32 sign mask (bit set means -1)."""
    w = np.asarray(sign_words, dtype=np.uint32).reshape(-1)
    if w.size * 32 < d:
        raise ValueError("sign mask too short")
    bits = (w[np.arange(d) // 32] >> (np.arange(d) % 32).astype(np.uint32)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def rotation_matrix(sign_words, d):
    """R = H_d D / sqrt(d), explicit d x d matrix."""
    return hadamard(d) * sign_vector(sign_words, d)[None, :] / np.sqrt(d)


def to_f64(x):
    """Exact widening of fp32 / bf16 (given as torch or numpy) to fp64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def encode(x, sign_words, thresholds):
    """Encode rows of x (n x d): returns (codes uint8 [n, d], norms fp32 [n], y fp64 [n, d]).

    y is the rotated unit vector, returned so tests can measure the distance of
    each coordinate to its nearest threshold.
    """
    x = to_f64(x)
    n, d = x.shape
    r = np.sqrt(np.sum(x * x, axis=1))
    y = np.zeros_like(x)
    nz = r > 0
    if sign_words is None:  # Plain-KV: no rotation, y = x / r
        y[nz] = x[nz] / r[nz, None]
    else:
        # y = R (x / r) = H (D x) / (sqrt(d) r).  The +-1 sums H (D x) are
        # formed first: for fp32 / bf16 inputs they are exact in fp64, so a
        # coordinate whose exact value sits on a threshold (0 is one) is
        # decided exactly.
        hx = (x * sign_vector(sign_words, d)[None, :]) @ hadamard(d).T
        y[nz] = hx[nz] / (np.sqrt(d) * r[nz, None])
    t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)
    if np.any(np.diff(t) <= 0):
        raise ValueError("thresholds must be strictly ascending")
    # code = #{j : t_j < y}: for ascending t, the left insertion point of y
    codes = np.searchsorted(t, y, side="left").astype(np.uint8)
    return codes, r.astype(np.float32), y


def decode(codes, norms, sign_words, centroids):
    """x_hat = r * R^T c[code] for every row (R = I when sign_words is None);
    fp64 [n, d]."""
    codes = np.asarray(codes)
    n, d = codes.shape
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    unit_rot = c[codes.astype(np.int64)]
    x_unit = unit_rot if sign_words is None else unit_rot @ rotation_matrix(sign_words, d)
    return x_unit * np.asarray(norms, dtype=np.float32).astype(np.float64)[:, None]


def pack(codes, bits):
    """Pack code rows (n x d, values < 2^bits) into bytes (n x bits*d/8)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, d = codes.shape
    if bits == 4:
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    if bits == 2:
        return (codes[:, 0::4] | (codes[:, 1::4] << 2) | (codes[:, 2::4] << 4)
                | (codes[:, 3::4] << 6)).astype(np.uint8)
    if bits == 3:
        # bit stream: bit j of row = bit (j % 3) of code j // 3
        stream = np.zeros((n, 3 * d), dtype=np.uint8)
        for b in range(3):
            stream[:, b::3] = (codes >> b) & 1
        return np.packbits(stream, axis=1, bitorder="little")
    raise ValueError("bits must be 2, 3 or 4")


def unpack(packed, bits, d):
    """Inverse of pack."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    if bits == 4:
        out = np.empty((n, d), dtype=np.uint8)
        out[:, 0::2] = packed & 0x0F
        out[:, 1::2] = packed >> 4
        return out
    if bits == 2:
        out = np.empty((n, d), dtype=np.uint8)
        for k in range(4):
            out[:, k::4] = (packed >> (2 * k)) & 0x03
        return out
    if bits == 3:
        stream = np.unpackbits(packed, axis=1, bitorder="little")[:, : 3 * d]
        out = np.zeros((n, d), dtype=np.uint8)
        for b in range(3):
            out |= (stream[:, b::3] << b).astype(np.uint8)
        return out
    raise ValueError("bits must be 2, 3 or 4")


def code_bytes(d, bits):
    return d * bits // 8
