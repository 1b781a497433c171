"""GPU parity of the pre-RoPE archive fetch (hsq_decode_rope) against the
oracle (oracle/rope.py).

Page: "Tamarin (HSQ)" summary, section 2, "Decode process", fetching step
(dequantise, then rotate to the semantic positions); RoPE as in Su et al.
(RoFormer, 2021), half-split pairing.  Codes and norms are drawn on the host,
so both sides read the same stored archive rows.  Tolerance: the decode's
(1e-6 of the largest output) plus the rotation's fp32 sine, cosine and the fp32
fraction of a turn (a few 1e-7 relative), 4e-6 of the largest output in all.
"""
import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb
from oracle import codec, rope
from tests.gpu_util import signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
BASE = 1e6
EDGE_POS = [0, 1, -1, 2 ** 31 - 1, -2 ** 31, 32767, 1 << 20]


def archive(rng, n, d, bits, n_rot):
    signs = rng.integers(0, 1 << 32, size=(n_rot, d // 32), dtype=np.uint64).astype(np.uint32)
    codes = rng.integers(0, 1 << bits, size=(n, d)).astype(np.uint8)
    norms = (rng.random(n) * 10).astype(np.float32)
    if n > 2:
        norms[2] = 0.0
    return signs, codes, norms


def gpu(codes, norms, bits, d, signs, c32, pos, per_rot, n_rot, out, base=BASE):
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    return hsq.decode_rope(f(codec.pack(codes, bits)), f(norms), bits, d,
                           None if signs is None else signs_to_dev(signs), f(c32),
                           f(pos.astype(np.int32)), base, vecs_per_rot=per_rot, n_rot=n_rot,
                           out_dtype=out).float().cpu().numpy().astype(np.float64)


def check(g, want, out):
    atol = 4e-6 * max(np.abs(want).max(), 1e-30)
    if out == torch.float32:
        np.testing.assert_allclose(g, want, rtol=0, atol=atol)
    else:
        w = torch.from_numpy(want).to(torch.bfloat16).double().numpy()
        np.testing.assert_allclose(g, w, rtol=2 ** -7, atol=atol)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rot", [True, False])
def test_decode_rope_parity(d, bits, out, rot):
    print(f"[rope] d={d} bits={bits} out={out} rot={rot}", flush=True)
    rng = np.random.default_rng(d * 10 + bits + rot)
    n = 1003  # several work-groups and a ragged tail
    signs, codes, norms = archive(rng, n, d, bits, 2)
    c32, _ = ocb.codebook_f32(d, bits)
    pos = rng.integers(0, 1 << 20, size=n)
    pos[:len(EDGE_POS)] = EDGE_POS
    half = 502  # rows 0..501 take mask 0, rows 502..1002 mask 1
    if rot:
        want = np.concatenate([
            rope.decode_rope(codes[:half], norms[:half], signs[0], c32, pos[:half], BASE),
            rope.decode_rope(codes[half:], norms[half:], signs[1], c32, pos[half:], BASE)])
        g = gpu(codes, norms, bits, d, signs, c32, pos, half, 2, out)
    else:
        want = rope.decode_rope(codes, norms, None, c32, pos, BASE)
        g = gpu(codes, norms, bits, d, None, c32, pos, half, 2, out)
    check(g, want, out)


@pytest.mark.parametrize("base", [1e4, 5e5, 1e6])
def test_other_bases(base):
    rng = np.random.default_rng(int(base))
    d, bits, n = 128, 4, 300
    signs, codes, norms = archive(rng, n, d, bits, 1)
    c32, _ = ocb.codebook_f32(d, bits)
    pos = rng.integers(-40000, 40000, size=n)
    want = rope.decode_rope(codes, norms, signs[0], c32, pos, base)
    check(gpu(codes, norms, bits, d, signs, c32, pos, n, 1, torch.float32, base), want,
          torch.float32)


@pytest.mark.parametrize("d", [64, 128])
def test_position_zero_is_the_plain_decode(d):
    rng = np.random.default_rng(5)
    signs, codes, norms = archive(rng, 777, d, 4, 1)
    c32, _ = ocb.codebook_f32(d, 4)
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    for out in (torch.float32, torch.bfloat16):
        a = hsq.decode(f(codec.pack(codes, 4)), f(norms), 4, d, signs_to_dev(signs), f(c32),
                       out_dtype=out)
        b = hsq.decode_rope(f(codec.pack(codes, 4)), f(norms), 4, d, signs_to_dev(signs), f(c32),
                            torch.zeros(777, dtype=torch.int32, device=DEV), BASE, out_dtype=out)
        # equal to fp32 rounding: RoPE at position 0 is the identity, and the
        # fetch kernel's FWHT runs over a relabelling of the coordinate bits
        # (each rotary pair in one lane), which changes only the order of
        # its additions
        ad, bd = a.double().cpu().numpy(), b.double().cpu().numpy()
        tol = 4e-6 * np.abs(ad).max()
        if out == torch.float32:
            np.testing.assert_allclose(bd, ad, rtol=0, atol=tol)
        else:
            np.testing.assert_allclose(bd, ad, rtol=2 ** -7, atol=tol)


def test_one_vector_and_empty():
    rng = np.random.default_rng(9)
    signs, codes, norms = archive(rng, 1, 128, 4, 1)
    c32, _ = ocb.codebook_f32(128, 4)
    pos = np.array([12345])
    check(gpu(codes, norms, 4, 128, signs, c32, pos, 1, 1, torch.float32),
          rope.decode_rope(codes, norms, signs[0], c32, pos, BASE), torch.float32)
    e = hsq.decode_rope(torch.zeros((0, 64), dtype=torch.uint8, device=DEV),
                        torch.zeros(0, device=DEV), 4, 128, signs_to_dev(signs),
                        torch.from_numpy(np.array(c32)).to(DEV), torch.zeros(0, dtype=torch.int32,
                                                                    device=DEV), BASE)
    assert e.shape == (0, 128)


def test_codec_workload_fetch():
    # the codec workload's size (32768 tokens x 8 heads, d = 128, 4 bits, bf16
    # out), every head's tokens at positions 0 .. 32767, in the launch the
    # benchmark times; 2000 sampled rows against the oracle
    c = W.CODEC
    n = c.heads * c.tokens
    rng = np.random.default_rng(21)
    signs, codes, norms = archive(rng, n, c.d, 4, c.heads)
    c32, _ = ocb.codebook_f32(c.d, 4)
    pos = np.tile(np.arange(c.tokens), c.heads)
    g = gpu(codes, norms, 4, c.d, signs, c32, pos, c.tokens, c.heads, torch.bfloat16)
    rows = np.sort(rng.choice(n, size=2000, replace=False))
    rows[-1] = n - 1
    want = np.concatenate([rope.decode_rope(codes[r:r + 1], norms[r:r + 1], signs[r // c.tokens],
                                            c32, pos[r:r + 1], BASE) for r in rows])
    check(g[rows], want, torch.bfloat16)
