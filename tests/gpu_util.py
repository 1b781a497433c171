"""Helpers for GPU parity tests (comparison rules from the HSQ north-star
tolerances: packed codes bit-exact except coordinates within 1e-6 of a
threshold, fewer than 1e-5 of the total; norms within 1e-6 relative;
selected sets exact except near-ties within 1e-5; attention within 2e-3
relative L2)."""
import numpy as np
import torch

from oracle import codec

CODE_BAND = 1e-6
CODE_FRACTION = 1e-5
NORM_RTOL = 1e-6
TIE_BAND = 1e-5
ATTN_REL_L2 = 2e-3


def gpu_available():
    return torch.cuda.is_available()


def signs_to_dev(words, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


def compare_codes(gpu_packed, ora_codes, ora_y, thresholds, bits, d, label="", fraction=True):
    """Assert the GPU's packed codes equal the oracle's except near thresholds.
    fraction=False leaves the "fewer than 1e-5 of the total" part to the
    caller, which applies it to a whole workload.  Returns (mismatches, total)."""
    g = codec.unpack(np.asarray(gpu_packed).reshape(-1, bits * d // 8), bits, d)
    o = np.asarray(ora_codes).reshape(-1, d)
    y = np.asarray(ora_y).reshape(-1, d)
    bad = g != o
    n_bad = int(bad.sum())
    if n_bad:
        t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)
        dist = np.min(np.abs(y[bad][:, None] - t[None, :]), axis=1)
        assert np.all(dist < CODE_BAND), (
            f"{label}: {n_bad} code mismatches, max threshold distance {dist.max():.3e}")
        assert not fraction or n_bad < CODE_FRACTION * o.size, (
            f"{label}: {n_bad} near-threshold mismatches of {o.size}")
    return n_bad, o.size


def compare_norms(gpu, ora, label=""):
    g = np.asarray(gpu, dtype=np.float64).reshape(-1)
    o = np.asarray(ora, dtype=np.float64).reshape(-1)
    np.testing.assert_allclose(g, o, rtol=NORM_RTOL, atol=1e-30, err_msg=label)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
