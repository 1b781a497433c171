"""GPU parity of decode-time tier maintenance (hsq_cache_append) and the decode
step over a cache laid out with capacities (hsq_cache_decode_step).

Page: "Tamarin (HSQ)" summary, section 2, "Three-tier architecture"; the
reading (tiers after every append = the compress-time build of the longer
context) is the oracle's, oracle/cache.py, pinned in tests/test_oracle_cache.py.
"""
import math

import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import cache as ocache
from oracle import codebook as ocb
from oracle import codec as ocodec
from oracle import decode as odec
from oracle import tiers as otiers
from tests.gpu_util import (ATTN_REL_L2, compare_codes, compare_norms, rel_l2, signs_to_dev)

pytestmark = pytest.mark.gpu
DEV = "cuda"


class CacheCase:
    """Raw K/V of T0 + K tokens; a GPU cache built from the first T0."""

    def __init__(self, w, T0, K):
        self.w, self.T0, self.K = w, T0, K
        full = w.smaller(T=T0 + K)
        self.k, self.v = W.kv(full, 0, DEV)
        self.q = W.query(full, 0, DEV)
        pre = w.smaller(T=T0)
        self.marks = [W.marked(pre, b) for b in range(w.batch)]
        self.ks, self.vs = W.signs(w.seed, 0, w.hkv, w.d)
        self.dks, self.dvs = signs_to_dev(self.ks), signs_to_dev(self.vs)
        self.c4, self.c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
        f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
        self.cb4, self.thr4, self.cb3, self.thr3 = f(self.c4[0]), f(self.c4[1]), f(self.c3[0]), f(self.c3[1])
        self.ng_cap = (T0 + K) // w.group_n + 2
        self.cache = self.build(T0)

    def build(self, T):
        w = self.w
        return hsq.Cache.from_prefix(self.k[:, :, :T].contiguous(), self.v[:, :, :T].contiguous(),
                                     w.n_sink, w.n_recent, self.marks, w.group_n, self.dks,
                                     self.dvs, self.thr4, self.thr3, self.ng_cap)

    def append(self, t):
        self.cache.append(self.k[:, :, t].contiguous(), self.v[:, :, t].contiguous(), self.dks,
                          self.dvs, self.thr4, self.thr3)


def assert_caches_identical(a, b):
    assert (a.t, a.n_pending, a.n_groups, a.n1) == (b.t, b.n_pending, b.n_groups, b.n1)
    for bb in range(a.B):
        assert a.pos_l1(bb) == b.pos_l1(bb)
    n1, ng, nr = a.n1, a.n_groups, a.n_recent + a.n_pending
    for name in ("l1k", "l1k_n", "l1v", "l1v_n"):
        assert torch.equal(getattr(a, name)[:, :, :n1], getattr(b, name)[:, :, :n1]), name
    for name in ("l2k", "l2k_n", "l2v", "l2v_n", "l3"):
        assert torch.equal(getattr(a, name)[:, :, :ng], getattr(b, name)[:, :, :ng]), name
    for name in ("raw_k", "raw_v"):
        assert torch.equal(getattr(a, name)[:, :, :nr], getattr(b, name)[:, :, :nr]), name


SMALL = [
    ("tiny_f32_d64_n8", W.TINY.smaller(batch=2, hq=4, hkv=2, n_recent=16, n_marked=10), 200, 19),
    ("bf16_d128_n16", W.QWEN3_8B_8K.smaller(batch=2, hq=8, hkv=2, n_marked=7, beta=5), 300, 37),
]


@pytest.mark.parametrize("name,w,T0,K", SMALL, ids=[s[0] for s in SMALL])
def test_appends_match_the_oracle_cache(name, w, T0, K):
    print(f"[cache oracle parity] {name} T0={T0} K={K}", flush=True)
    c = CacheCase(w, T0, K)
    units = [(b, h) for b in range(w.batch) for h in range(w.hkv)]
    ora = {}
    for b, h in units:
        ora[b, h] = ocache.UnitCache(c.k[b, h, :T0].cpu(), c.v[b, h, :T0].cpu(), w.n_sink,
                                     w.n_recent, c.marks[b], w.group_n, c.ks[h], c.vs[h], c.c4,
                                     c.c3)
    kc, vc = c.k.cpu(), c.v.cpu()
    for t in range(T0, T0 + K):
        c.append(t)
        for b, h in units:
            ora[b, h].append(kc[b, h, t], vc[b, h, t])
    torch.cuda.synchronize()
    g = c.cache
    d, gn = w.d, w.group_n
    for b, h in units:
        o = ora[b, h]
        assert g.n_groups == o.n_groups and g.n_pending == len(o.pending)
        pos = np.array(g.pos_l1(b))
        assert sorted(pos.tolist()) == sorted(o.l1)
        for kv, raw, sg in (("k", kc, c.ks[h]), ("v", vc, c.vs[h])):
            x = raw[b, h].double().numpy()
            # L1 rows (each row's position from the host map)
            codes, norms, y = ocodec.encode(x[pos], sg, c.c4[1])
            compare_codes(getattr(g, f"l1{kv}")[b, h, :g.n1].cpu().numpy(), codes, y, c.c4[1], 4,
                          d, f"{name} L1 {kv} unit {b},{h}")
            compare_norms(getattr(g, f"l1{kv}_n")[b, h, :g.n1].cpu().numpy(), norms,
                          f"{name} L1 {kv} norms")
            # L2 summaries: 3-bit code of the mean of each group's raw rows
            grp = np.array([gg["pos"] for gg in o.groups])
            mean = x[grp.reshape(-1)].reshape(len(grp), gn, d).mean(axis=1)
            codes, norms, y = ocodec.encode(mean, sg, c.c3[1])
            compare_codes(getattr(g, f"l2{kv}")[b, h, :g.n_groups].cpu().numpy(), codes, y,
                          c.c3[1], 3, d, f"{name} L2 {kv} unit {b},{h}")
            compare_norms(getattr(g, f"l2{kv}_n")[b, h, :g.n_groups].cpu().numpy(), norms,
                          f"{name} L2 {kv} norms")
            # L3 records: the group's tokens at 4 bits, in position order
            kp, kn, vp, vn = otiers.split_l3_record(g.l3[b, h, :g.n_groups].cpu().numpy(), gn, d)
            packed, rn = (kp, kn) if kv == "k" else (vp, vn)
            codes, norms, y = ocodec.encode(x[grp.reshape(-1)], sg, c.c4[1])
            compare_codes(packed.reshape(-1, d // 2), codes, y, c.c4[1], 4, d,
                          f"{name} L3 {kv} unit {b},{h}")
            compare_norms(rn.reshape(-1), norms, f"{name} L3 {kv} norms")


@pytest.mark.parametrize("name,w,T0,K", SMALL, ids=[s[0] for s in SMALL])
def test_appends_equal_the_build_of_the_longer_context(name, w, T0, K):
    # bit for bit: the same encodes in the same order, so the incremental cache
    # and a compress-time build at every length agree exactly
    print(f"[cache vs build] {name}", flush=True)
    c = CacheCase(w, T0, K)
    for t in range(T0, T0 + K):
        c.append(t)
        if (t - T0) % 6 == 5 or t == T0 + K - 1:
            assert_caches_identical(c.cache, c.build(t + 1))


@pytest.mark.parametrize("name,w,T0,K", SMALL, ids=[s[0] for s in SMALL])
def test_cache_decode_step(name, w, T0, K):
    print(f"[cache decode] {name}", flush=True)
    c = CacheCase(w, T0, K)
    for t in range(T0, T0 + K):
        c.append(t)
    g = c.cache
    beta = min(w.beta, g.n_groups)
    out, idx = g.decode_step(c.q, w.beta, c.dks, c.dvs, c.cb4, c.cb3)
    # the same kernels over dense copies of the used rows: identical results
    dense = g.tiers()
    out2, idx2 = hsq.decode_step(c.q, dense, w.beta, c.dks, c.dvs, c.cb4, c.cb3)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)
    # against the oracle, fed the GPU's selection
    scale = 1 / math.sqrt(w.d)
    worst = 0.0
    kc, vc = c.k.cpu(), c.v.cpu()
    for b in range(w.batch):
        for h in range(w.hkv):
            o = ocache.UnitCache(kc[b, h, :T0], vc[b, h, :T0], w.n_sink, w.n_recent, c.marks[b],
                                 w.group_n, c.ks[h], c.vs[h], c.c4, c.c3)
            for t in range(T0, T0 + K):
                o.append(kc[b, h, t], vc[b, h, t])
            u = o.as_unit()
            deq = odec.dequant_unit(u, w.d, w.group_n, c.ks[h], c.vs[h], c.c4, c.c3)
            qh = c.q[b, h * w.G:(h + 1) * w.G].double().cpu().numpy()
            sel = idx[b, h].cpu().numpy() if beta > 0 else np.zeros(0, np.int64)
            want = odec.hsq_attention_unit(qh, deq, u["l3"], sel, w.group_n, w.d, c.ks[h],
                                           c.vs[h], c.c4, scale)
            worst = max(worst, rel_l2(out[b, h * w.G:(h + 1) * w.G].cpu().numpy(), want))
            # the selection is the oracle's top-beta up to near-ties
            scores, _ = odec.route_scores(qh, deq["l2k"], scale)
            want_sel = odec.top_beta(scores, beta)
            diff = set(sel.tolist()) ^ set(want_sel.tolist())
            if diff:
                sb = np.sort(scores)[::-1][beta - 1]
                assert all(abs(scores[gg] - sb) < 1e-5 for gg in diff), (b, h, diff)
    assert worst < ATTN_REL_L2, worst


def test_headline_shape_append_and_decode():
    # Qwen3-14B-shaped layer (batch 64, 8 kv heads, d = 128, N = 8) near 16K
    # context: nine appends cross one seal; the cache then equals the build of
    # the longer context bit for bit, and its decode step equals the dense one
    w = W.QWEN3_14B_16K
    T0, K = w.T - 5, 9
    print(f"[cache headline] T0={T0} K={K}", flush=True)
    c = CacheCase(w, T0, K)
    ng0 = c.cache.n_groups
    for t in range(T0, T0 + K):
        c.append(t)
    assert c.cache.n_groups == ng0 + 1
    assert_caches_identical(c.cache, c.build(T0 + K))
    out, idx = c.cache.decode_step(c.q, w.beta, c.dks, c.dvs, c.cb4, c.cb3)
    out2, idx2 = hsq.decode_step(c.q, c.cache.tiers(), w.beta, c.dks, c.dvs, c.cb4, c.cb3)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(out, out2)


@pytest.mark.parametrize("beta", [0, 1, 10000])
def test_cache_decode_beta_edges(beta):
    # nothing fetched, one group, every group: the strided step equals the
    # dense one bit for bit, and the oracle within the attention tolerance
    w = W.TINY.smaller(batch=2, hq=4, hkv=2, n_recent=16, n_marked=10, beta=beta)
    T0, K = 200, 11
    print(f"[cache decode beta={beta}]", flush=True)
    c = CacheCase(w, T0, K)
    for t in range(T0, T0 + K):
        c.append(t)
    g = c.cache
    out, idx = g.decode_step(c.q, beta, c.dks, c.dvs, c.cb4, c.cb3)
    out2, idx2 = hsq.decode_step(c.q, g.tiers(), beta, c.dks, c.dvs, c.cb4, c.cb3)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    b_eff = min(beta, g.n_groups)
    if b_eff > 0:
        assert torch.equal(idx, idx2) and idx.shape[-1] == b_eff
    kc, vc = c.k.cpu(), c.v.cpu()
    scale = 1 / math.sqrt(w.d)
    for b in range(w.batch):
        for h in range(w.hkv):
            o = ocache.UnitCache(kc[b, h, :T0], vc[b, h, :T0], w.n_sink, w.n_recent, c.marks[b],
                                 w.group_n, c.ks[h], c.vs[h], c.c4, c.c3)
            for t in range(T0, T0 + K):
                o.append(kc[b, h, t], vc[b, h, t])
            u = o.as_unit()
            deq = odec.dequant_unit(u, w.d, w.group_n, c.ks[h], c.vs[h], c.c4, c.c3)
            sel = idx[b, h].cpu().numpy() if b_eff > 0 else np.zeros(0, np.int64)
            qh = c.q[b, h * w.G:(h + 1) * w.G].double().cpu().numpy()
            want = odec.hsq_attention_unit(qh, deq, u["l3"], sel, w.group_n, w.d, c.ks[h],
                                           c.vs[h], c.c4, scale)
            assert rel_l2(out[b, h * w.G:(h + 1) * w.G].cpu().numpy(), want) < ATTN_REL_L2
