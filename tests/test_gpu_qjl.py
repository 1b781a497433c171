"""GPU parity of the TQ-QKV key path (hsq_encode_qjl, hsq_qjl_logits) against
the oracle (oracle/qjl.py).

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression" summary, "Experimental setup" and "Key contributions" 1-2.
Tolerances: codes and norms as for the codec; a sketch bit may differ only
where the oracle's projection (S u)_j lies within 1e-5 of zero, in rows whose
codes all match (a code that takes the adjacent cell near a threshold changes
that row's residual), fewer than 1e-4 of those bits; gamma to 1e-5 relative;
logits, computed on both sides from the same key records (written by the
oracle's encoder), to 1e-5 of the largest term of the sum.
"""
import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb
from oracle import qjl
from tests.gpu_util import compare_codes, compare_norms, signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
PROJ_BAND = 1e-5


def inputs(n, d, dtype, seed, student=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(n, d)) if student else rng.standard_normal((n, d))
    xt = torch.from_numpy(x.astype(np.float32))
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    signs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    S = rng.standard_normal((d, d)).astype(np.float32)
    return xt, signs, S


def encode_both(xt, signs, S, bits):
    d = xt.shape[1]
    c, t = ocb.codebook_f32(d, bits)
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    g = hsq.encode_qjl(xt.to(DEV), bits, signs_to_dev(signs), f(t), f(c), f(S))
    o = qjl.encode(xt, signs, t, c, S)
    return [a.cpu().numpy() for a in g], o, (c, t)


def check_encode(g, o, ct, bits, d, label):
    codes, norms, sketch, gamma = g
    c, t = ct
    compare_codes(codes, o["codes"], o["y"], t, bits, d, label)
    compare_norms(norms, o["norms"], label)
    from oracle import codec
    same = np.all(codec.unpack(codes, bits, d) == o["codes"], axis=1)
    gb = qjl.unpack_bits(sketch, d)[same]
    ob = o["bits"][same]
    bad = gb != ob
    if bad.any():
        near = np.abs(o["proj"][same][bad]) < PROJ_BAND
        assert near.all(), f"{label}: sketch bits differ away from zero projections"
        assert bad.sum() < 1e-4 * ob.size or bad.sum() <= 1, f"{label}: {bad.sum()} sketch bits"
    np.testing.assert_allclose(gamma, o["gamma"], rtol=1e-5, atol=1e-30, err_msg=label)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 37, 3000])
def test_encode_qjl_parity(d, bits, dtype, n):
    print(f"[qjl encode] d={d} bits={bits} {dtype} n={n}", flush=True)
    xt, signs, S = inputs(n, d, dtype, seed=n + d + bits)
    g, o, ct = encode_both(xt, signs, S, bits)
    check_encode(g, o, ct, bits, d, f"d={d} b={bits} {dtype} n={n}")
    # the codes and norms are the codec's, bit for bit
    c, t = ct
    codes, norms = hsq.encode(xt.to(DEV), bits, signs_to_dev(signs), torch.from_numpy(np.array(t)).to(DEV))
    assert np.array_equal(codes.cpu().numpy(), g[0])
    assert np.array_equal(norms.cpu().numpy(), g[1])


def test_zero_vectors_have_no_residual():
    xt, signs, S = inputs(40, 128, "f32", seed=3)
    xt[5] = 0
    xt[17] = 0
    g, o, ct = encode_both(xt, signs, S, 4)
    assert g[3][5] == 0 and g[3][17] == 0 and g[1][5] == 0
    assert not qjl.unpack_bits(g[2][5:6], 128).any()  # S 0 = 0 is not negative


@pytest.mark.parametrize("d,bits,n_q", [(64, 4, 3), (128, 4, 5), (128, 3, 8), (128, 4, 1)])
def test_qjl_logits_parity(d, bits, n_q):
    print(f"[qjl logits] d={d} bits={bits} n_q={n_q}", flush=True)
    n = 777
    xt, signs, S = inputs(n, d, "bf16", seed=d * bits + n_q, student=True)
    c, t = ocb.codebook_f32(d, bits)
    # the stored keys come from the oracle's encoder (the GPU encoder has its
    # own parity test), so both sides read the same records
    from oracle import codec
    o = qjl.encode(xt, signs, t, c, S)
    codes, norms, gamma = codec.pack(o["codes"], bits), o["norms"], o["gamma"]
    sketch = qjl.pack_bits(o["bits"])
    rng = np.random.default_rng(n_q)
    q = rng.standard_normal((n_q, d)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    got = hsq.qjl_logits(f(q), bits, f(codes), f(norms), f(sketch), f(gamma), signs_to_dev(signs),
                         f(c), f(S), float(scale)).cpu().numpy()
    want = qjl.logits_qjl(q, o["codes"], norms, o["bits"], gamma, signs, c, S, scale)
    # largest term: the norm times |R q| . |c| plus the correction's magnitude
    bound = scale * (np.abs(norms)[None, :] * np.abs(q).sum(1, keepdims=True) * np.abs(c).max()
                     + np.sqrt(np.pi / 2) / d * gamma[None, :] * np.abs(q @ S.T).sum(1, keepdims=True))
    err = np.abs(got - want)
    assert np.all(err <= 1e-5 * bound + 1e-6), float(np.max(err / (bound + 1e-30)))
    # and the correction moves the TQ-KV logit towards the exact one on average
    exact = scale * (q.astype(np.float64) @ xt.double().numpy().T)
    tq = qjl.logits_tq(q, o["codes"], norms, signs, c, scale)
    assert abs(float(np.mean(got - exact))) <= abs(float(np.mean(tq - exact))) + 3 * float(
        np.std(got - exact)) / np.sqrt(got.size)


def test_codec_workload_head():
    # one head of the codec workload (32768 tokens, d = 128, bf16 Student-t with
    # outlier channels): encode at 4 bits with the sketch; sampled rows checked
    c = W.CODEC
    k, _ = W.codec_inputs(c, DEV)
    ks, _ = W.codec_signs(c)
    x = k.view(c.heads, c.tokens, c.d)[3].contiguous()
    rng = np.random.default_rng(11)
    S = rng.standard_normal((c.d, c.d)).astype(np.float32)
    cb, t = ocb.codebook_f32(c.d, 4)
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    g = [a.cpu().numpy() for a in hsq.encode_qjl(x, 4, signs_to_dev(ks[3]), f(t), f(cb), f(S))]
    rows = np.sort(rng.choice(c.tokens, size=2000, replace=False))
    o = qjl.encode(x[torch.from_numpy(rows).to(DEV)].cpu(), ks[3], t, cb, S)
    check_encode([g[0][rows], g[1][rows], g[2][rows], g[3][rows]], o, (cb, t), 4, c.d,
                 "codec workload head 3")
