"""GPU parity of the codec variants (hsq_encode, hsq_decode) against the fp64
oracle: the 2-bit budget and Plain-KV (signs = NULL, the rotation off).

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", technical summary, "Key contributions" item 1 (Plain-KV among
the non-dominated methods) and "Results and recommendations" (2-bit budget).
"""
import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from oracle import codebook as ocb
from oracle import codec
from tests.gpu_util import compare_codes, compare_norms, signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
VARIANTS = [(2, True), (2, False), (3, False), (4, False)]  # (bits, rotation on)


def _inputs(n, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, d), generator=g) * torch.exp(torch.randn((n, 1), generator=g))
    if n > 3:
        x[1] = 0.0                      # zero vector
        x[2, 5] += 1e4                  # one huge outlier coordinate
        x[3] = 0.0
        x[3, 7] = -2.5                  # a basis vector: exact zeros elsewhere
    return x.to(torch.bfloat16) if dtype == "bf16" else x


@pytest.mark.parametrize("bits,rot", VARIANTS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 37, 5000])
def test_encode_variant_parity(bits, rot, d, dtype, n):
    print(f"encode variant bits={bits} rot={rot} d={d} dtype={dtype} n={n}", flush=True)
    rng = np.random.default_rng(d * 11 + bits + n + rot)
    signs = rng.integers(0, 1 << 32, size=(1, d // 32), dtype=np.uint64).astype(np.uint32)
    x = _inputs(n, d, dtype, seed=n + d + bits + 2 * rot)
    _, t32 = ocb.codebook_f32(d, bits)
    codes, norms = hsq.encode(x.to(DEV), bits, signs_to_dev(signs) if rot else None,
                              torch.from_numpy(np.array(t32)).to(DEV))
    torch.cuda.synchronize()
    assert codes.shape == (n, bits * d // 8)
    oc, on, oy = codec.encode(x, signs[0] if rot else None, t32)
    compare_codes(codes.cpu().numpy(), oc, oy, t32, bits, d, f"bits {bits} rot {rot}")
    compare_norms(norms.cpu().numpy(), on, f"bits {bits} rot {rot}")


@pytest.mark.parametrize("bits,rot", VARIANTS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_decode_variant_parity(bits, rot, d, out):
    print(f"decode variant bits={bits} rot={rot} d={d} out={out}", flush=True)
    rng = np.random.default_rng(5 + d + bits + rot)
    n = 777
    signs = rng.integers(0, 1 << 32, size=(1, d // 32), dtype=np.uint64).astype(np.uint32)
    codes = rng.integers(0, 1 << bits, size=(n, d)).astype(np.uint8)
    norms = (rng.random(n) * 10).astype(np.float32)
    norms[0] = 0.0
    c32, _ = ocb.codebook_f32(d, bits)
    od = codec.decode(codes, norms, signs[0] if rot else None, c32)
    g = hsq.decode(torch.from_numpy(codec.pack(codes, bits)).to(DEV),
                   torch.from_numpy(norms).to(DEV), bits, d,
                   signs_to_dev(signs) if rot else None, torch.from_numpy(np.array(c32)).to(DEV),
                   out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    g = g.float().cpu().numpy().astype(np.float64)
    if out == "f32":
        # rotation off: one fp32 product per value; on: the fp32 transform
        np.testing.assert_allclose(g, od, rtol=2e-6, atol=1e-6 * np.abs(od).max())
    else:
        want = torch.from_numpy(od).to(torch.bfloat16).double().numpy()
        np.testing.assert_allclose(g, want, rtol=2 ** -7, atol=1e-6 * np.abs(od).max())


@pytest.mark.parametrize("bits", [2, 4])
def test_plain_round_trip_on_codec_workload_shape(bits):
    # a codec-shaped batch (Student-t rows with outlier channels) through
    # encode and decode with the rotation off: the GPU round trip equals the
    # oracle's, and its relative MSE is the oracle's
    d, n = 128, 4096
    print(f"plain round trip bits={bits}", flush=True)
    g = torch.Generator().manual_seed(40 + bits)
    chi2 = sum(torch.randn((n, d), generator=g) ** 2 for _ in range(3))
    z = torch.randn((n, d), generator=g) / torch.sqrt(chi2 / 3.0)
    z[:, :4] *= 20.0
    x = z.to(torch.bfloat16)
    c32, t32 = ocb.codebook_f32(d, bits)
    codes, norms = hsq.encode(x.to(DEV), bits, None, torch.from_numpy(np.array(t32)).to(DEV))
    xh = hsq.decode(codes, norms, bits, d, None, torch.from_numpy(np.array(c32)).to(DEV))
    torch.cuda.synchronize()
    oc, on, oy = codec.encode(x, None, t32)
    compare_codes(codes.cpu().numpy(), oc, oy, t32, bits, d, "plain round trip")
    ox = codec.decode(oc, on, None, c32)
    xf = codec.to_f64(x)
    g_rel = np.sum((xh.cpu().double().numpy() - xf) ** 2) / np.sum(xf * xf)
    o_rel = np.sum((ox - xf) ** 2) / np.sum(xf * xf)
    assert abs(g_rel - o_rel) <= 1e-4 * o_rel


@pytest.mark.parametrize("vpr,n_rot", [(1, 7), (2, 3), (64, 5), (999, 2), (4999, 3), (5000, 1),
                                       (1 << 20, 4)])
def test_rotation_index_for_many_divisors(vpr, n_rot):
    # vector i uses mask (i / vecs_per_rot) % n_rot, for divisors of every
    # kind (1, powers of two, odd, near the count, beyond it), in encode and
    # in decode
    d, bits, n = 64, 4, 5000
    print(f"rotation index vpr={vpr} n_rot={n_rot}", flush=True)
    rng = np.random.default_rng(vpr * 31 + n_rot)
    signs = rng.integers(0, 1 << 32, size=(n_rot, d // 32), dtype=np.uint64).astype(np.uint32)
    x = _inputs(n, d, "f32", seed=vpr + n_rot)
    c32, t32 = ocb.codebook_f32(d, bits)
    codes, norms = hsq.encode(x.to(DEV), bits, signs_to_dev(signs), torch.from_numpy(np.array(t32)).to(DEV),
                              vecs_per_rot=vpr, n_rot=n_rot)
    xh = hsq.decode(codes, norms, bits, d, signs_to_dev(signs), torch.from_numpy(np.array(c32)).to(DEV),
                    vecs_per_rot=vpr, n_rot=n_rot)
    torch.cuda.synchronize()
    rot = (np.arange(n) // vpr) % n_rot
    gc, gn, gx = codes.cpu().numpy(), norms.cpu().numpy(), xh.cpu().double().numpy()
    for r in range(n_rot):
        sel = np.nonzero(rot == r)[0]
        if sel.size == 0:
            continue
        oc, on, oy = codec.encode(x[sel], signs[r], t32)
        compare_codes(gc[sel], oc, oy, t32, bits, d, f"rot {r}")
        compare_norms(gn[sel], on, f"rot {r}")
        od = codec.decode(codec.unpack(gc[sel], bits, d), gn[sel], signs[r], c32)
        np.testing.assert_allclose(gx[sel], od, rtol=2e-6, atol=1e-6 * np.abs(od).max())


@pytest.mark.parametrize("close", [False, True])
def test_encode_4bit_any_symmetric_thresholds(close):
    # the 4-bit encoder counts thresholds through a table of 64 bins of |y|
    # when no bin holds two of them, else by seven compares; both give the
    # oracle's codes (thresholds symmetric about 0, as the entry point asks)
    d, n = 128, 3000
    print(f"encode 4-bit custom thresholds close={close}", flush=True)
    pos = [0.005, 0.01, 0.0105, 0.05, 0.1, 0.2, 0.5] if close else \
          [0.02, 0.045, 0.07, 0.1, 0.13, 0.17, 0.99]
    t = np.array([-p for p in pos[::-1]] + [0.0] + pos, dtype=np.float32)
    rng = np.random.default_rng(8 + close)
    signs = rng.integers(0, 1 << 32, size=(1, d // 32), dtype=np.uint64).astype(np.uint32)
    x = _inputs(n, d, "f32", seed=77 + close)
    codes, norms = hsq.encode(x.to(DEV), 4, signs_to_dev(signs), torch.from_numpy(np.array(t)).to(DEV))
    torch.cuda.synchronize()
    oc, on, oy = codec.encode(x, signs[0], t)
    compare_codes(codes.cpu().numpy(), oc, oy, t, 4, d, f"close {close}")
    compare_norms(norms.cpu().numpy(), on, f"close {close}")
