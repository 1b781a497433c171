"""GPU parity of the decode step over a pre-RoPE archive
(hsq_decode_step_prerope) against the fp64 oracle.

Page: "Tamarin (HSQ)" summary, section 2, "Decode process": the fetched
groups' originals are dequantised and rotated to their semantic positions
before attention (read as re-applying RoPE, Su et al., RoFormer 2021, with
the half-split pairing); L1 and the L2 summaries hold embedded keys.

Inputs: a workload's raw keys are the keys before the embedding (k_pre); the
embedded keys are k_post = RoPE(k_pre) at positions offset + t (oracle.rope).
The oracle builds every unit's records (L1 and L2 from k_post, L3 from
k_pre), the GPU step runs on those same bytes, so the comparison sees only
the step's arithmetic.  Rules as for the plain step: selections equal the
oracle's except groups within 1e-5 of the beta-th score, attention within
2e-3 relative L2 per unit (the oracle fed the GPU's selection).
"""
import math

import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb
from oracle import decode as odec
from oracle import rope as orope
from oracle import tiers as otiers
from tests.gpu_util import ATTN_REL_L2, TIE_BAND, rel_l2, signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n", "l3")


def run_case(w, beta, base=1e6, offset=0, agg="max", bias=0.0, units=None):
    """Oracle records for the units (all by default; the rest of the batch
    holds the records of unit (0, 0)), the GPU step on them, every checked
    unit against the oracle.  Returns the worst relative L2."""
    print(f"[prerope] T={w.T} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.group_n} "
          f"beta={beta} base={base} offset={offset} agg={agg}", flush=True)
    k_dev, v_dev = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    scale = 1.0 / math.sqrt(w.d)
    pos = offset + np.arange(w.T)
    plans = [otiers.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    all_u = [(b, h) for b in range(w.batch) for h in range(w.hkv)]
    units = all_u if units is None else units
    recs, deqs = {}, {}
    for (b, h) in sorted(set(units) | {(0, 0)}):
        l1, g = plans[b]
        kp = k_dev[b, h].double().cpu().numpy()
        vb = v_dev[b, h].cpu()
        post = otiers.build_unit(orope.rope(kp, pos, base), vb, l1, g, ks[h], vs[h], c4, c3)
        pre = otiers.build_unit(kp, vb, l1, g, ks[h], vs[h], c4, c3)
        u = {n: post[n] for n in NAMES}
        u["l3"] = pre["l3"]
        recs[(b, h)] = u
        deqs[(b, h)] = odec.dequant_unit(u, w.d, w.group_n, ks[h], vs[h], c4, c3)
    n1, ng = recs[(0, 0)]["l1k"].shape[0], recs[(0, 0)]["l2k"].shape[0]
    t = hsq.alloc_tiers(w.batch, w.hkv, w.d, n1, ng, w.group_n, DEV)
    for (b, h) in all_u:
        r = recs.get((b, h), recs[(0, 0)])
        for name in NAMES:
            getattr(t, name)[b, h].copy_(torch.from_numpy(np.ascontiguousarray(r[name])).to(DEV))
    del k_dev, v_dev
    # RoPE positions of the grouped tokens, [B][ng * N] group-major
    gpos = np.stack([offset + plans[b][1].reshape(-1) for b in range(w.batch)]).astype(np.int32)
    out, idx = hsq.decode_step_prerope(
        q, t, beta, signs_to_dev(ks), signs_to_dev(vs), torch.from_numpy(np.array(c4[0])).to(DEV),
        torch.from_numpy(np.array(c3[0])).to(DEV), torch.from_numpy(gpos).to(DEV), base,
        agg=hsq.HSQ_AGG_MEAN if agg == "mean" else hsq.HSQ_AGG_MAX, summary_bias=bias)
    torch.cuda.synchronize()
    go = out.double().cpu().numpy()
    gi = idx.cpu().numpy() if idx is not None else None
    b_eff = min(beta, ng)
    worst = 0.0
    G = w.G
    for (b, h) in units:
        deq = deqs[(b, h)]
        qh = q[b, h * G:(h + 1) * G].double().cpu().numpy()
        os_, _ = odec.route_scores(qh, deq["l2k"], scale, agg)
        if b_eff > 0:
            gsel = gi[b, h]
            assert gsel.shape[0] == b_eff and np.all(np.diff(gsel) > 0), f"unit {(b, h)}"
            kth = np.sort(os_)[::-1][b_eff - 1]
            osel = odec.top_beta(os_, beta)
            for g in sorted(set(gsel.tolist()) ^ set(osel.tolist())):
                assert abs(os_[g] - kth) < TIE_BAND, (
                    f"unit {(b, h)}: group {g} differs, score {os_[g]:.8f} vs beta-th {kth:.8f}")
            sel = gsel
        else:
            sel = np.zeros(0, dtype=np.int64)
        want = odec.hsq_attention_unit(qh, deq, recs[(b, h)]["l3"], sel, w.group_n, w.d, ks[h],
                                       vs[h], c4, scale, bias, group_pos=plans[b][1] + offset,
                                       rope_base=base)
        e = rel_l2(go[b, h * G:(h + 1) * G], want)
        worst = max(worst, e)
        assert e < ATTN_REL_L2, f"unit {(b, h)}: rel L2 {e:.3e}"
    print(f"  worst rel L2 {worst:.2e}", flush=True)
    return worst


CASES = {
    "tiny": (W.TINY, None),
    "q8_2k": (W.QWEN3_8B_8K.smaller(T=2048, batch=2, n_marked=41), None),
    "q14_1k_b4_n8": (W.QWEN3_14B_16K.smaller(T=1100, batch=4, n_marked=10, beta=9), None),
    "d64_g3_n8": (W.TINY.smaller(d=64, hq=6, hkv=2, group_n=8, T=700, beta=7), None),
    "d64_n16": (W.TINY.smaller(d=64, hq=8, hkv=2, group_n=16, T=900, beta=5), None),
}


@pytest.mark.parametrize("case", list(CASES))
def test_prerope_step_parity(case):
    w, units = CASES[case]
    run_case(w, w.beta, units=units)


@pytest.mark.parametrize("offset", [0, 1 << 20, 2 ** 31 - 70_000])
def test_prerope_step_positions(offset):
    # far positions: the angles' fraction of a turn from the 64-bit turns
    w = W.QWEN3_8B_8K.smaller(T=1024, batch=1, n_marked=12, beta=12)
    run_case(w, w.beta, offset=offset, base=1e4)


@pytest.mark.parametrize("beta", [0, 1, 10_000])
def test_prerope_step_beta_edges(beta):
    # nothing fetched (the dense rows are never read), one group, every group
    run_case(W.TINY, beta)


@pytest.mark.parametrize("case", ["no_l1", "no_groups"])
def test_prerope_step_empty_tiers(case):
    base = W.QWEN3_8B_8K.smaller(T=1024, batch=2, n_marked=12)
    if case == "no_l1":
        w = base.smaller(n_sink=0, n_recent=0, n_marked=0, T=1024)
    else:
        w = base.smaller(T=60, n_marked=0)
    run_case(w, w.beta)


def test_prerope_step_mean_and_bias():
    w = W.QWEN3_14B_16K.smaller(T=1500, batch=2, n_marked=15, beta=11)
    run_case(w, w.beta, agg="mean", bias=0.75)


def test_prerope_step_at_position_zero_matches_plain_step():
    # every RoPE position 0: the embedding is the identity, so the pre-RoPE
    # step on an archive equals the plain step on the same bytes up to the
    # fp16 rounding of the re-rotated keys
    w = W.QWEN3_8B_8K.smaller(T=2048, batch=2, n_marked=30, beta=16)
    k, v = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = torch.from_numpy(np.stack([p[0] for p in plans])).to(DEV)
    gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in plans])).to(DEV)
    dks, dvs = signs_to_dev(ks), signs_to_dev(vs)
    f = lambda a: torch.from_numpy(np.array(a)).to(DEV)
    t = hsq.build_tiers(k, v, l1, gp, w.group_n, dks, dvs, f(c4[1]), f(c3[1]))
    a, ia = hsq.decode_step(q, t, w.beta, dks, dvs, f(c4[0]), f(c3[0]))
    b, ib = hsq.decode_step_prerope(q, t, w.beta, dks, dvs, f(c4[0]), f(c3[0]),
                                    torch.zeros_like(gp), 1e6)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib)
    e = rel_l2(b.double().cpu().numpy(), a.double().cpu().numpy())
    print(f"  pre-RoPE at position 0 vs plain step: rel L2 {e:.2e}", flush=True)
    assert e < 1e-3


def test_prerope_step_full_size_sampled_units():
    # the Qwen3-14B-shaped layer at full size (batch 64, T = 16384, N = 8,
    # beta = 128) through the pre-RoPE entry point; eight sampled units
    # against the oracle
    w = W.QWEN3_14B_16K
    rng = np.random.default_rng(5)
    units = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.batch, 8),
                                              rng.integers(0, w.hkv, 8))]
    run_case(w, w.beta, units=sorted(set(units)))


def test_prerope_step_beyond_on_chip_router_logits():
    # G * n_groups = 5 * 3051 > 12288: the split route, the RoPE pass over
    # its selection, and the split attend with the dense key rows
    w = W.QWEN3_14B_16K.smaller(T=24576, batch=1, n_marked=100)
    run_case(w, w.beta)
