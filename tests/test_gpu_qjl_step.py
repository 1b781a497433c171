"""GPU parity of the decode step over TQ-QKV token keys
(hsq_decode_step_qjl) against the fp64 oracle.

Page: "Ablation, Statistical Inference, and Validation for KV-Cache
Compression" technical summary, "Key contributions" 1 (TQ-QKV: the 1-bit QJL
residual sketch on the key path), inside the "Tamarin (HSQ)" decode step
(section 2, "Decode process").  Read for the step: every 4-bit token key (L1
and the archive) carries its sketch and gamma; the summaries do not.

The oracle builds every checked unit's records and sketches; the GPU step
runs on those same bytes, so the comparison sees only the step's arithmetic.
Rules as for the plain step: selections equal the oracle's except groups
within 1e-5 of the beta-th score, attention within 2e-3 relative L2 per unit
(the oracle fed the GPU's selection).
"""
import math

import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb
from oracle import decode as odec
from oracle import qjl as oqjl
from oracle import tiers as otiers
from tests.gpu_util import ATTN_REL_L2, CODE_BAND, TIE_BAND, rel_l2, signs_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n", "l3")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.array(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def run_case(w, beta, agg="max", bias=0.0, units=None, zero_gamma=False):
    """Oracle records and sketches for the units (all by default; the rest of
    the batch holds unit (0, 0)'s), the GPU step on them, every checked unit
    against the oracle.  Returns (out, idx, tiers, sketches, inputs)."""
    print(f"[qjl-step] T={w.T} B={w.batch} Hq={w.hq} Hkv={w.hkv} d={w.d} N={w.group_n} "
          f"beta={beta} agg={agg} bias={bias}", flush=True)
    k_dev, v_dev = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    S = W.sketch_matrices(w.seed, 0, w.hkv, w.d)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    scale = 1.0 / math.sqrt(w.d)
    plans = [otiers.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    all_u = [(b, h) for b in range(w.batch) for h in range(w.hkv)]
    units = all_u if units is None else units
    recs, sks, deqs = {}, {}, {}
    for (b, h) in sorted(set(units) | {(0, 0)}):
        l1, g = plans[b]
        kb, vb = k_dev[b, h].cpu(), v_dev[b, h].cpu()
        recs[(b, h)] = otiers.build_unit(kb, vb, l1, g, ks[h], vs[h], c4, c3)
        sk = oqjl.unit_sketches(kb, l1, g, ks[h], c4[1], c4[0], S[h])
        if zero_gamma:
            sk["l1_gamma"] = np.zeros_like(sk["l1_gamma"])
            sk["l3_gamma"] = np.zeros_like(sk["l3_gamma"])
        sks[(b, h)] = dict(sk, S=S[h])
        deqs[(b, h)] = odec.dequant_unit(recs[(b, h)], w.d, w.group_n, ks[h], vs[h], c4, c3)
    del k_dev, v_dev
    u0 = recs[(0, 0)]
    n1, ng = u0["l1k"].shape[0], u0["l2k"].shape[0]
    m, N = w.d, w.group_n
    t = hsq.alloc_tiers(w.batch, w.hkv, w.d, n1, ng, N, DEV)
    l1_sk = torch.zeros((w.batch, w.hkv, n1, m // 8), dtype=torch.uint8, device=DEV)
    l1_gm = torch.zeros((w.batch, w.hkv, n1), dtype=torch.float32, device=DEV)
    l3_sk = torch.zeros((w.batch, w.hkv, ng, N, m // 8), dtype=torch.uint8, device=DEV)
    l3_gm = torch.zeros((w.batch, w.hkv, ng, N), dtype=torch.float32, device=DEV)
    for (b, h) in all_u:
        r = recs.get((b, h), u0)
        sk = sks.get((b, h), sks[(0, 0)])
        for name in NAMES:
            getattr(t, name)[b, h].copy_(to_dev(r[name]))
        if n1:
            l1_sk[b, h].copy_(to_dev(oqjl.pack_bits(sk["l1_bits"])))
            l1_gm[b, h].copy_(to_dev(sk["l1_gamma"]))
        if ng:
            l3_sk[b, h].copy_(to_dev(oqjl.pack_bits(sk["l3_bits"].reshape(-1, m))
                                     .reshape(ng, N, m // 8)))
            l3_gm[b, h].copy_(to_dev(sk["l3_gamma"]))
    dks, dvs = signs_to_dev(ks), signs_to_dev(vs)
    cb4, cb3 = to_dev(np.array(c4[0])), to_dev(np.array(c3[0]))
    out, idx = hsq.decode_step_qjl(q, t, beta, dks, dvs, cb4, cb3, l1_sk, l1_gm, l3_sk, l3_gm,
                                   to_dev(S), agg=hsq.HSQ_AGG_MEAN if agg == "mean"
                                   else hsq.HSQ_AGG_MAX, summary_bias=bias)
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
                                       vs[h], c4, scale, bias, qjl=sks[(b, h)])
        e = rel_l2(go[b, h * G:(h + 1) * G], want)
        worst = max(worst, e)
        assert e < ATTN_REL_L2, f"unit {(b, h)}: rel L2 {e:.3e}"
    print(f"  worst rel L2 {worst:.2e}", flush=True)
    return out, idx, t, (dks, dvs, cb4, cb3), q


CASES = {
    "tiny": W.TINY,
    "q8_2k": W.QWEN3_8B_8K.smaller(T=2048, batch=2, n_marked=41),
    "q14_1k_b4_n8": W.QWEN3_14B_16K.smaller(T=1100, batch=4, n_marked=10, beta=9),
    "d64_g3_n8": W.TINY.smaller(d=64, hq=6, hkv=2, group_n=8, T=700, beta=7),
    "d64_n16": W.TINY.smaller(d=64, hq=8, hkv=2, group_n=16, T=900, beta=5),
}


@pytest.mark.parametrize("case", list(CASES))
def test_qjl_step_parity(case):
    w = CASES[case]
    run_case(w, w.beta)


@pytest.mark.parametrize("beta", [0, 1, 10_000])
def test_qjl_step_beta_edges(beta):
    run_case(W.TINY, beta)


@pytest.mark.parametrize("case", ["no_l1", "no_groups"])
def test_qjl_step_empty_tiers(case):
    # a tier without entries passes null sketches: every position grouped
    # (the archive's corrections alone), or everything in L1
    base = W.QWEN3_8B_8K.smaller(T=1024, batch=2, n_marked=12)
    if case == "no_l1":
        w = base.smaller(n_sink=0, n_recent=0, n_marked=0, T=1024)
    else:
        w = base.smaller(T=60, n_marked=0)
    run_case(w, w.beta)


def test_qjl_step_mean_and_bias():
    w = W.QWEN3_14B_16K.smaller(T=1500, batch=2, n_marked=15, beta=11)
    run_case(w, w.beta, agg="mean", bias=0.75)


def test_qjl_step_zero_gamma_is_the_two_launch_step_bit_for_bit():
    # gamma = 0 everywhere: every correction is an exact zero, so the step is
    # the plain two-launch step (the same route and token tiles) bit for bit
    w = W.QWEN3_8B_8K.smaller(T=2048, batch=2, n_marked=30, beta=16)
    out, idx, t, (dks, dvs, cb4, cb3), q = run_case(w, w.beta, zero_gamma=True)
    ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, min(w.beta, t.ng), w.group_n,
                            DEV)
    hsq.step_route(q, t, w.beta, dks, cb3, ws)
    plain = torch.empty_like(out)
    hsq.step_attend(q, t, w.beta, dks, dvs, cb4, ws, plain)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)


def test_qjl_step_full_size_sampled_units():
    # the Qwen3-14B-shaped layer at full size (batch 64, T = 16384, N = 8,
    # beta = 128) with TQ-QKV token keys; eight sampled units against the
    # oracle
    w = W.QWEN3_14B_16K
    rng = np.random.default_rng(9)
    units = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.batch, 8),
                                              rng.integers(0, w.hkv, 8))]
    run_case(w, w.beta, units=sorted(set(units)))


PROJ_BAND = 1e-5  # |(S u)_j| below which fp32 and fp64 may take other signs


@pytest.mark.parametrize("case", ["q8_2k", "d64_g3_n8"])
def test_build_sketches_parity(case):
    # hsq_build_sketches straight from the raw keys at the tier plan's rows
    # against the oracle's per-key encode: on every key with no coordinate
    # within the code band of a threshold (so its codes are the oracle's),
    # the sketch bits match except at projections within 1e-5 of zero and
    # gamma matches to 1e-5 relative.  About 1% of the keys have such a
    # coordinate (128 coordinates, 15 thresholds); they are left out
    w = CASES[case]
    print(f"[build sketches] {case}", flush=True)
    k, _ = W.kv(w, 0, DEV)
    ks, _ = W.signs(w.seed, 0, w.hkv, w.d)
    S = W.sketch_matrices(w.seed, 0, w.hkv, w.d)
    c4 = ocb.codebook_f32(w.d, 4)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = to_dev(np.stack([p[0] for p in plans]))
    gp = to_dev(np.stack([p[1].reshape(-1) for p in plans]))
    g = [a.cpu().numpy() for a in hsq.build_sketches(
        k, l1, gp, w.group_n, signs_to_dev(ks), to_dev(np.array(c4[1])), to_dev(np.array(c4[0])),
        to_dev(S))]
    m = w.d
    n_rows = n_near = 0
    for b in range(w.batch):
        for h in range(w.hkv):
            rows = np.concatenate([plans[b][0], plans[b][1].reshape(-1)])
            o = oqjl.encode(k[b, h].cpu()[torch.from_numpy(rows)], ks[h], c4[1], c4[0], S[h])
            gb = np.concatenate([oqjl.unpack_bits(g[0][b, h], m),
                                 oqjl.unpack_bits(g[2][b, h].reshape(-1, m // 8), m)])
            gg = np.concatenate([g[1][b, h], g[3][b, h].reshape(-1)])
            # the oracle's codes of the same keys, against the GPU tier build's
            # rule: a key whose coordinates all sit away from the thresholds
            # has the same codes on both sides
            yd = np.abs(o["y"][:, :, None] - np.asarray(c4[1], np.float64)[None, None, :]).min(2)
            same = np.all(yd > CODE_BAND, axis=1)
            n_rows += len(rows)
            n_near += int((~same).sum())
            bad = gb[same] != o["bits"][same]
            if bad.any():
                assert np.all(np.abs(o["proj"][same][bad]) < PROJ_BAND), f"unit {(b, h)}"
            np.testing.assert_allclose(gg[same], o["gamma"][same], rtol=1e-5, atol=1e-30,
                                       err_msg=f"unit {(b, h)}")
    print(f"  {n_near} of {n_rows} keys near a threshold, left out", flush=True)
    assert n_near < 0.05 * n_rows


def test_qjl_step_from_raw_keys():
    # the whole TQ-QKV path on the GPU from raw keys: hsq_build_tiers,
    # hsq_build_sketches, hsq_decode_step_qjl; every unit against the
    # oracle's own build, fed the GPU's selection
    w = W.QWEN3_8B_8K.smaller(T=1500, batch=2, n_marked=20, beta=24)
    k, v = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    S = W.sketch_matrices(w.seed, 0, w.hkv, w.d)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = to_dev(np.stack([p[0] for p in plans]))
    gp = to_dev(np.stack([p[1].reshape(-1) for p in plans]))
    dks, dvs = signs_to_dev(ks), signs_to_dev(vs)
    t = hsq.build_tiers(k, v, l1, gp, w.group_n, dks, dvs, to_dev(np.array(c4[1])),
                        to_dev(np.array(c3[1])))
    sk = hsq.build_sketches(k, l1, gp, w.group_n, dks, to_dev(np.array(c4[1])),
                            to_dev(np.array(c4[0])), to_dev(S))
    out, idx = hsq.decode_step_qjl(q, t, w.beta, dks, dvs, to_dev(np.array(c4[0])),
                                   to_dev(np.array(c3[0])), *sk, to_dev(S))
    torch.cuda.synchronize()
    go, gi = out.double().cpu().numpy(), idx.cpu().numpy()
    scale = 1.0 / math.sqrt(w.d)
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.hkv):
            l1p, g = plans[b]
            kb, vb = k[b, h].cpu(), v[b, h].cpu()
            u = otiers.build_unit(kb, vb, l1p, g, ks[h], vs[h], c4, c3)
            osk = dict(oqjl.unit_sketches(kb, l1p, g, ks[h], c4[1], c4[0], S[h]), S=S[h])
            deq = odec.dequant_unit(u, w.d, w.group_n, ks[h], vs[h], c4, c3)
            qh = q[b, h * w.G:(h + 1) * w.G].double().cpu().numpy()
            want = odec.hsq_attention_unit(qh, deq, u["l3"], gi[b, h], w.group_n, w.d, ks[h],
                                           vs[h], c4, scale, qjl=osk)
            e = rel_l2(go[b, h * w.G:(h + 1) * w.G], want)
            worst = max(worst, e)
            assert e < ATTN_REL_L2, f"unit {(b, h)}: rel L2 {e:.3e}"
    print(f"  worst rel L2 {worst:.2e}", flush=True)


@pytest.mark.parametrize("variant", ["qjl", "prerope"])
def test_variant_steps_graph_replays_match_eager(variant):
    # the TQ-QKV step (two launches) and the pre-RoPE step (three launches,
    # the fetched-key rows handed over in the workspace) captured in a graph:
    # three replays with eager work and a scrambled workspace between them
    # equal the eager call bit for bit
    w = W.QWEN3_14B_16K.smaller(T=2048, batch=4, n_marked=20)
    print(f"graph replays: {variant}", flush=True)
    k, v = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = to_dev(np.stack([p[0] for p in plans]))
    gp = to_dev(np.stack([p[1].reshape(-1) for p in plans]))
    dks, dvs = signs_to_dev(ks), signs_to_dev(vs)
    cb4, cb3 = to_dev(np.array(c4[0])), to_dev(np.array(c3[0]))
    t = hsq.build_tiers(k, v, l1, gp, w.group_n, dks, dvs, to_dev(np.array(c4[1])),
                        to_dev(np.array(c3[1])))
    beta = min(w.beta, t.ng)
    out = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.batch, w.hkv, beta), dtype=torch.int32, device=DEV)
    if variant == "qjl":
        S = to_dev(W.sketch_matrices(w.seed, 0, w.hkv, w.d))
        sk = hsq.build_sketches(k, l1, gp, w.group_n, dks, to_dev(np.array(c4[1])), cb4, S)
        ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)

        def step():
            hsq.decode_step_qjl(q, t, w.beta, dks, dvs, cb4, cb3, *sk, S, ws=ws, out=out, idx=idx)
    else:
        ws = hsq.Workspace(hsq.prerope_workspace_bytes(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng,
                                                       beta, w.group_n), DEV)

        def step():
            hsq.decode_step_prerope(q, t, w.beta, dks, dvs, cb4, cb3, gp, 1e6, ws=ws, out=out,
                                    idx=idx)

    step()
    torch.cuda.synchronize()
    out0, idx0 = out.clone(), idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    for r in range(3):
        out.fill_(float("nan"))
        idx.fill_(-1)
        ws.buf.fill_(0x5A)  # the workspace's contents must not matter
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx0), f"replay {r}: selection differs"
        assert torch.equal(out, out0), f"replay {r}: output differs"
        del junk


def test_qjl_step_beyond_on_chip_router_logits():
    # G * n_groups = 5 * 3051 > 12288: the split route and the split attend
    # with the sketch correction
    w = W.QWEN3_14B_16K.smaller(T=24576, batch=1, n_marked=100)
    run_case(w, w.beta)
