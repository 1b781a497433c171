"""TQ-QKV: the 1-bit QJL residual sketch on the key path (oracle, fp64).
TEST INFRASTRUCTURE ONLY.

Source: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression" technical summary, "Experimental setup" (TurboQuant may add a
1-bit Johnson-Lindenstrauss (QJL) residual sketch on the K or V path) and
"Key contributions" 1 (TQ-QKV = TQ-KV plus a 1-bit QJL residual sketch on the
key path, the only QJL variant kept) and 2 (a zero-mean score correction with
variance sigma^2 inflates softmax weights by about exp(sigma^2 / 2), Jensen).

The page names the sketch but not its formulas; the estimator is the
published QJL one (Zandieh, Daliri and Han, "QJL: 1-Bit Quantized JL
Transform for KV Cache Quantization with Zero Overhead", 2024): for a vector
e and a matrix S of i.i.d. N(0, 1) entries with m rows, store sign(S e) and
||e||; then for any q, sqrt(pi / 2) / m * ||e|| * <S q, sign(S e)> is an
unbiased estimate of <q, e>, because for g ~ N(0, I),
E[<g, q> sign(<g, e>)] = sqrt(2 / pi) <q, e> / ||e||.

Readings taken:
* The residual is the TurboQuant error of the key in the rotated unit domain,
  u = y - c[code] with y = R x / r (codec module); e = x - x_hat = r R^T u,
  so <q, e> = r <R q, u> and ||e|| = r ||u||.  The sketch is taken of u
  (S R is again an i.i.d. Gaussian matrix, so this is the same estimator
  applied to e).
* m = d rows; one S per (layer, kv-head), shared by every key of that head,
  given as data (like the rotation signs).
* Stored per key: the TurboQuant codes and norm r, the m sketch bits (bit j
  set when (S u)_j < 0; LSB-first, bit j in byte j // 8 at position j % 8) and
  gamma = r ||u|| as fp32.
* Corrected logit: scale * (r <R q, c[code]> + sqrt(pi/2) / m * gamma *
  sum_j (S R q)_j * (1 - 2 bit_j)).
"""
import numpy as np

from . import codec


def pack_bits(bits):
    """bool [n, m] -> uint8 [n, m/8], bit j of a row at byte j // 8, position j % 8."""
    return np.packbits(np.asarray(bits, dtype=np.uint8), axis=1, bitorder="little")


def unpack_bits(packed, m):
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=1, bitorder="little")[:, :m]


def encode(x, sign_words, thresholds, centroids, S):
    """TQ codes of the rows of x plus their residual sketch.

    Returns dict: codes uint8 [n, d], norms fp32 [n], y fp64 [n, d],
    u fp64 [n, d] (unit-domain residual), proj fp64 [n, m] (S u),
    bits bool [n, m], gamma fp32 [n].
    """
    codes, norms, y = codec.encode(x, sign_words, thresholds)
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    u = y - c[codes.astype(np.int64)]
    # a zero vector has y = 0 and norm 0: its residual carries no weight
    u[np.asarray(norms) == 0] = 0.0
    proj = u @ np.asarray(S, dtype=np.float64).T
    bits = proj < 0
    gamma = (norms.astype(np.float64) * np.sqrt(np.sum(u * u, axis=1))).astype(np.float32)
    return {"codes": codes, "norms": norms, "y": y, "u": u, "proj": proj, "bits": bits,
            "gamma": gamma}


def logits_tq(q, codes, norms, sign_words, centroids, scale):
    """TQ-KV logits scale * q . x_hat for query rows q [G, d] and keys: [G, n]."""
    xh = codec.decode(codes, norms, sign_words, centroids)
    return scale * (np.asarray(q, dtype=np.float64) @ xh.T)


def correction(q, bits, gamma, sign_words, S):
    """QJL estimate of the residual's share of q . x for query rows q [G, d]
    and sketched keys (bits bool [n, m], gamma [n]):
    sqrt(pi/2) / m * gamma * <S R q, 1 - 2 bits>, unscaled.  Returns [G, n]."""
    q = np.asarray(q, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    m, d = S.shape
    rq = q @ codec.rotation_matrix(sign_words, d).T        # R q, [G, d]
    sq = rq @ S.T                                          # S R q, [G, m]
    sgn = 1.0 - 2.0 * np.asarray(bits, dtype=np.float64)    # [n, m]
    return np.sqrt(np.pi / 2) / m * (sq @ sgn.T) * np.asarray(gamma, dtype=np.float64)[None, :]


def logits_qjl(q, codes, norms, bits, gamma, sign_words, centroids, S, scale):
    """TQ-QKV logits: the TQ-KV logit plus the QJL estimate of the residual's
    inner product.  q [G, d]; bits bool [n, m].  Returns [G, n]."""
    return (logits_tq(q, codes, norms, sign_words, centroids, scale)
            + scale * correction(q, bits, gamma, sign_words, S))


def unit_sketches(k_raw, l1_pos, groups, sign_words, thresholds, centroids, S):
    """Sketches of one unit's token keys, as the TQ-QKV decode step reads
    them: the L1 keys (rows l1_pos) and every grouped token (groups [ng, N]),
    each encoded on its own exactly as the 4-bit tiers encode it.
    Returns dict: l1_bits bool [n1, m], l1_gamma fp32 [n1],
    l3_bits bool [ng, N, m], l3_gamma fp32 [ng, N]."""
    x = codec.to_f64(k_raw)
    groups = np.asarray(groups, dtype=np.int64)
    ng, gn = groups.shape
    m = np.asarray(S).shape[0]
    a = encode(x[np.asarray(l1_pos, dtype=np.int64)], sign_words, thresholds, centroids, S)
    b = encode(x[groups.reshape(-1)], sign_words, thresholds, centroids, S)
    return {"l1_bits": a["bits"], "l1_gamma": a["gamma"],
            "l3_bits": b["bits"].reshape(ng, gn, m), "l3_gamma": b["gamma"].reshape(ng, gn)}
