"""GPU parity of the TurboQuant codec kernels (hsq_encode, hsq_decode,
hsq_build_tiers) against the fp64 oracle.

Pages: "Tamarin (HSQ)" summary, section 2 ("Key technical components",
quantisation; "Three-tier architecture"); "Ablation, Statistical Inference,
and Validation for KV-Cache Compression", "Experimental setup".
"""
import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb
from oracle import codec, tiers as otiers
from tests.gpu_util import compare_codes, compare_norms, signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand_signs(rng, n_rot, d):
    return rng.integers(0, 1 << 32, size=(n_rot, d // 32), dtype=np.uint64).astype(np.uint32)


def _inputs(n, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, d), generator=g) * torch.exp(torch.randn((n, 1), generator=g))
    if n > 3:
        x[1] = 0.0                      # zero vector
        x[2, 5] += 1e4                  # one huge outlier coordinate
    return x.to(torch.bfloat16) if dtype == "bf16" else x


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 37, 5000])
def test_encode_parity(d, bits, dtype, n):
    print(f"encode parity d={d} bits={bits} dtype={dtype} n={n}", flush=True)
    rng = np.random.default_rng(d * 7 + bits + n)
    n_rot, vpr = 3, max(1, (n + 2) // 3)
    signs = _rand_signs(rng, n_rot, d)
    x = _inputs(n, d, dtype, seed=n + d + bits)
    c32, t32 = ocb.codebook_f32(d, bits)
    codes, norms = hsq.encode(x.to(DEV), bits, signs_to_dev(signs), torch.from_numpy(np.array(t32)).to(DEV),
                              vecs_per_rot=vpr, n_rot=n_rot)
    torch.cuda.synchronize()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    for r in range(n_rot):
        lo, hi = r * vpr, min((r + 1) * vpr, n)
        if lo >= hi:
            continue
        oc, on, oy = codec.encode(x[lo:hi], signs[r], t32)
        compare_codes(gc[lo:hi], oc, oy, t32, bits, d, f"rot {r}")
        compare_norms(gn[lo:hi], on, f"rot {r}")


@pytest.mark.parametrize("d,bits,gn", [(128, 3, 16), (64, 3, 8), (128, 4, 8)])
def test_encode_group_mean_and_row_index(d, bits, gn):
    print(f"encode group mean d={d} bits={bits} N={gn}", flush=True)
    rng = np.random.default_rng(99)
    rows = 640
    x = torch.randn((rows, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    n_vec = 23
    idx = rng.choice(rows, size=n_vec * gn, replace=False).astype(np.int64)
    signs = _rand_signs(rng, 1, d)
    c32, t32 = ocb.codebook_f32(d, bits)
    codes, norms = hsq.encode(x.to(DEV), bits, signs_to_dev(signs), torch.from_numpy(np.array(t32)).to(DEV),
                              row_idx=torch.from_numpy(idx).to(DEV), group_n=gn)
    torch.cuda.synchronize()
    mean = codec.to_f64(x)[idx].reshape(n_vec, gn, d).mean(axis=1)
    oc, on, oy = codec.encode(mean, signs[0], t32)
    compare_codes(codes.cpu().numpy(), oc, oy, t32, bits, d, "group mean")
    compare_norms(norms.cpu().numpy(), on, "group mean")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_decode_parity(d, bits, out):
    print(f"decode parity d={d} bits={bits} out={out}", flush=True)
    rng = np.random.default_rng(3 + d + bits)
    n = 1000
    signs = _rand_signs(rng, 2, d)
    codes = rng.integers(0, 1 << bits, size=(n, d)).astype(np.uint8)
    norms = (rng.random(n) * 10).astype(np.float32)
    norms[0] = 0.0
    packed = codec.pack(codes, bits)
    c32, _ = ocb.codebook_f32(d, bits)
    od = np.concatenate([codec.decode(codes[:500], norms[:500], signs[0], c32),
                         codec.decode(codes[500:], norms[500:], signs[1], c32)])
    g = hsq.decode(torch.from_numpy(packed).to(DEV), torch.from_numpy(norms).to(DEV), bits, d,
                   signs_to_dev(signs), torch.from_numpy(np.array(c32)).to(DEV), vecs_per_rot=500, n_rot=2,
                   out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    g = g.float().cpu().numpy().astype(np.float64)
    if out == "f32":
        np.testing.assert_allclose(g, od, rtol=2e-6, atol=1e-6 * np.abs(od).max())
    else:
        want = torch.from_numpy(od).to(torch.bfloat16).double().numpy()
        # bf16 rounding of an fp32 value within 1e-6 of the fp64 one: equal or one bf16 ulp
        np.testing.assert_allclose(g, want, rtol=2 ** -7, atol=1e-6 * np.abs(od).max())


@pytest.mark.parametrize("wl,T,B", [(W.TINY, None, None), (W.QWEN3_8B_8K, 1200, 2),
                                     (W.QWEN3_14B_16K, 700, 2)])
def test_build_tiers_parity(wl, T, B):
    w = wl.smaller(T=T or wl.T, batch=B or wl.batch,
                   n_marked=min(wl.n_marked, max(1, (T or wl.T) // 50)))
    print(f"build tiers parity {w.name} T={w.T} B={w.batch}", flush=True)
    k, v = W.kv(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = torch.from_numpy(np.stack([p[0] for p in plans])).to(DEV)
    gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in plans])).to(DEV)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    t = hsq.build_tiers(k, v, l1, gp, w.group_n, signs_to_dev(ks), signs_to_dev(vs),
                        torch.from_numpy(np.array(c4[1])).to(DEV), torch.from_numpy(np.array(c3[1])).to(DEV))
    torch.cuda.synchronize()
    kc, vc = k.cpu(), v.cpu()
    host = {name: getattr(t, name).cpu().numpy() for name in
            ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n", "l3")}
    for b in range(w.batch):
        ol1, og = otiers.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
        for h in range(w.hkv):
            u = otiers.build_unit(kc[b, h], vc[b, h], ol1, og, ks[h], vs[h], c4, c3)
            lab = f"b{b} h{h}"
            for kv in ("k", "v"):
                compare_codes(host[f"l1{kv}"][b, h], u[f"l1{kv}_codes"], u[f"l1{kv}_y"], c4[1], 4,
                              w.d, lab + f" L1{kv}")
                compare_norms(host[f"l1{kv}_n"][b, h], u[f"l1{kv}_n"], lab)
                compare_codes(host[f"l2{kv}"][b, h], u[f"l2{kv}_codes"], u[f"l2{kv}_y"], c3[1], 3,
                              w.d, lab + f" L2{kv}")
                compare_norms(host[f"l2{kv}_n"][b, h], u[f"l2{kv}_n"], lab)
            kp, kn, vp, vn = otiers.split_l3_record(host["l3"][b, h], w.group_n, w.d)
            compare_codes(kp, u["l3k_codes"], u["l3k_y"], c4[1], 4, w.d, lab + " L3k")
            compare_codes(vp, u["l3v_codes"], u["l3v_y"], c4[1], 4, w.d, lab + " L3v")
            compare_norms(kn, u["l3k_n"], lab)
            compare_norms(vn, u["l3v_n"], lab)


@pytest.mark.parametrize("bits", [4, 3])
def test_codec_workload_all_heads(bits):
    # The codec workload at full size: 32768 tokens x 8 heads x d = 128, bf16
    # Student-t(3) K and V with 4 outlier channels x20 per head, one rotation
    # per head, encoded and decoded in one call each (as timed).  Every
    # head, 4096 sampled rows per head and K|V, against the oracle: codes
    # under the code rule, norms to 1e-6, the bf16 decode of the GPU's codes
    # against the oracle's dequantisation of the same codes.
    c = W.CODEC
    print(f"codec workload bits={bits}", flush=True)
    k, v = W.codec_inputs(c, DEV)
    ks, vs = W.codec_signs(c)
    c32, t32 = ocb.codebook_f32(c.d, bits)
    n = c.heads * c.tokens
    rng = np.random.default_rng(31 + bits)
    rows = np.sort(rng.choice(c.tokens, size=4096, replace=False))
    total_bad = total = 0
    for name, x, sg in (("K", k, ks), ("V", v, vs)):
        codes, norms = hsq.encode(x.view(n, c.d), bits, signs_to_dev(sg),
                                  torch.from_numpy(np.array(t32)).to(DEV), vecs_per_rot=c.tokens,
                                  n_rot=c.heads)
        dec = hsq.decode(codes, norms, bits, c.d, signs_to_dev(sg), torch.from_numpy(np.array(c32)).to(DEV),
                         vecs_per_rot=c.tokens, n_rot=c.heads, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        gc = codes.view(c.heads, c.tokens, -1).cpu().numpy()
        gn = norms.view(c.heads, c.tokens).cpu().numpy()
        gd = dec.view(c.heads, c.tokens, c.d).float().cpu().numpy().astype(np.float64)
        xh = x.cpu()
        for h in range(c.heads):
            oc, on, oy = codec.encode(xh[h, rows], sg[h], t32)
            nb, tot = compare_codes(gc[h, rows], oc, oy, t32, bits, c.d, f"{name} head {h}")
            total_bad += nb
            total += tot
            compare_norms(gn[h, rows], on, f"{name} head {h}")
            want = codec.decode(codec.unpack(gc[h, rows], bits, c.d), gn[h, rows], sg[h], c32)
            wb = torch.from_numpy(want).to(torch.bfloat16).double().numpy()
            np.testing.assert_allclose(gd[h, rows], wb, rtol=2 ** -7,
                                       atol=1e-6 * np.abs(want).max(), err_msg=f"{name} head {h}")
    assert total_bad < 1e-5 * total
    print(f"  {total_bad} near-threshold code differences of {total}", flush=True)
