"""Pre-RoPE archive: dequantise, then rotate to the token's position (oracle,
fp64).  TEST INFRASTRUCTURE ONLY.

Source: "Tamarin (HSQ)" summary (Korean and Dutch versions), section 2,
"Decode process", fetching step: the selected groups' original tokens are
brought from the archive, dequantised on the GPU and rotated to their
semantic positions.  The other reading of that step (the inverse TurboQuant
rotation alone, archive holding post-RoPE keys) is the decode step's; this
module is the variant whose archive holds the keys before the rotary position
embedding, so the embedding is applied at fetch.

The pages give no RoPE parameters.  Readings taken:
* RoPE as defined by Su et al., "RoFormer: Enhanced Transformer with Rotary
  Position Embedding" (2021): coordinate pairs are rotated by the angle
  p * theta_i, theta_i = base^(-2 i / d), i = 0 .. d/2 - 1.
* Pairing: coordinate i with coordinate i + d/2 (the half-split layout of the
  Qwen3 models the workloads are named after); the rotated pair is
  (x_i cos a - x_{i+d/2} sin a, x_{i+d/2} cos a + x_i sin a).
* base is an argument; the workloads use 1e6, the Qwen3 models' published
  rotary base.
* A position is any integer (a negative one rotates backwards).
"""
import numpy as np

from . import codec


def frequencies(d, base):
    """theta_i = base^(-2 i / d) for i = 0 .. d/2 - 1, fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope(x, positions, base):
    """Rotate each row x[n] [d] to position positions[n]; fp64 [n, d]."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    h = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * frequencies(d, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[:, :h], x[:, h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=1)


def decode_rope(codes, norms, sign_words, centroids, positions, base):
    """Dequantised archive rows (codec.decode) rotated to their positions."""
    return rope(codec.decode(codes, norms, sign_words, centroids), positions, base)
