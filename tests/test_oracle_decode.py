"""Pins of the oracle's tier plan, router, top-beta and union-set attention.

Page: "Tamarin (HSQ)" summary, section 2, "Three-tier architecture" and
"Decode process" (route the L2 summary keys, fetch the top-beta groups from
L3, attend over L1 + unfetched summaries + fetched originals, masking the
fetched groups' summaries).
"""
import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import codec, decode, qjl, rope, tiers


def make_unit(T=200, d=64, n_sink=4, n_recent=16, n_marked=10, gn=8, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    pool = np.arange(n_sink, T - n_recent)
    marked = np.sort(rng.choice(pool, size=n_marked, replace=False))
    l1, groups = tiers.tier_plan(T, n_sink, n_recent, marked, gn)
    ks = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    vs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    cb4, cb3 = cb.codebook_f32(d, 4), cb.codebook_f32(d, 3)
    unit = tiers.build_unit(k, v, l1, groups, ks, vs, cb4, cb3)
    return dict(k=k, v=v, l1=l1, groups=groups, ks=ks, vs=vs, cb4=cb4, cb3=cb3, unit=unit,
                marked=marked, T=T, d=d, gn=gn)


def test_tier_plan_tiny_counts():
    # T = 512, 4 sinks, 32 recent, 16 marked: 460 remaining = 57 groups of 8 + 4
    rng = np.random.default_rng(0)
    marked = np.sort(rng.choice(np.arange(4, 512 - 32), size=16, replace=False))
    l1, groups = tiers.tier_plan(512, 4, 32, marked, 8)
    assert groups.shape == (57, 8)
    assert l1.size == 56


@pytest.mark.parametrize("T,ns,nr,nm,gn", [(512, 4, 32, 16, 8), (300, 4, 64, 7, 16), (50, 4, 64, 0, 8),
                                           (1000, 0, 0, 0, 8), (129, 1, 0, 3, 16)])
def test_tier_plan_partition(T, ns, nr, nm, gn):
    rng = np.random.default_rng(T)
    lo, hi = ns, max(T - nr, ns)
    marked = np.sort(rng.choice(np.arange(lo, hi), size=min(nm, hi - lo), replace=False))
    l1, groups = tiers.tier_plan(T, ns, nr, marked, gn)
    allpos = np.concatenate([l1, groups.reshape(-1)])
    np.testing.assert_array_equal(np.sort(allpos), np.arange(T))  # each position exactly once
    assert np.all(np.diff(l1) > 0)
    assert np.all(np.diff(groups.reshape(-1)) > 0)
    must = set(range(min(ns, T))) | set(range(max(T - nr, 0), T)) | set(marked.tolist())
    assert must <= set(l1.tolist())
    assert l1.size - len(must) < gn  # only a short remainder is promoted
    # the promoted remainder are the last non-L1 positions
    rest = sorted(set(range(T)) - must)
    assert set(l1.tolist()) - must == set(rest[len(rest) - (len(rest) % gn):])


def test_l3_records_reverse_to_single_token_encodes():
    # reversibility: every archived token decodes exactly as if encoded alone
    u = make_unit()
    d, gn = u["d"], u["gn"]
    kp, kn, vp, vn = tiers.split_l3_record(u["unit"]["l3"], gn, d)
    for g in (0, 5, u["groups"].shape[0] - 1):
        for j in range(gn):
            pos = u["groups"][g, j]
            c, n, _ = codec.encode(u["k"][pos:pos + 1], u["ks"], u["cb4"][1])
            np.testing.assert_array_equal(kp[g, j], codec.pack(c, 4)[0])
            assert kn[g, j] == n[0]
            c, n, _ = codec.encode(u["v"][pos:pos + 1], u["vs"], u["cb4"][1])
            np.testing.assert_array_equal(vp[g, j], codec.pack(c, 4)[0])
            assert vn[g, j] == n[0]


def test_summary_is_3bit_encode_of_group_mean():
    u = make_unit()
    d = u["d"]
    g = 3
    mean = u["k"][u["groups"][g]].mean(axis=0, keepdims=True)
    c, n, _ = codec.encode(mean, u["ks"], u["cb3"][1])
    np.testing.assert_array_equal(u["unit"]["l2k"][g], codec.pack(c, 3)[0])
    assert u["unit"]["l2k_n"][g] == n[0]
    deq = codec.decode(codec.unpack(u["unit"]["l2k"][g:g + 1], 3, d), u["unit"]["l2k_n"][g:g + 1],
                       u["ks"], u["cb3"][0])
    # 3-bit relative error of a summary is about sqrt(d * D(d, 3)) ~ 0.18
    assert np.linalg.norm(deq - mean) / np.linalg.norm(mean) < 0.3


@pytest.mark.parametrize("seed", range(5))
def test_top_beta_matches_stable_sort(seed):
    rng = np.random.default_rng(seed)
    s = np.round(rng.standard_normal(300), 1)  # many exact ties
    for beta in (0, 1, 7, 50, 299, 300, 400):
        want = np.sort(np.argsort(-s, kind="stable")[: min(beta, 300)])
        np.testing.assert_array_equal(decode.top_beta(s, beta), want)


def _full_dense(u, q_heads, scale):
    """Dense attention over all T tokens, each encoded on its own at 4 bits."""
    ck, nk, _ = codec.encode(u["k"], u["ks"], u["cb4"][1])
    cv, nv, _ = codec.encode(u["v"], u["vs"], u["cb4"][1])
    kh = codec.decode(ck, nk, u["ks"], u["cb4"][0])
    vh = codec.decode(cv, nv, u["vs"], u["cb4"][0])
    return np.stack([decode.softmax_attention(q, kh, vh, scale) for q in q_heads])


def test_beta_all_equals_dense_attention():
    u = make_unit(T=300, seed=4)
    d = u["d"]
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, d)) * 2
    ng = u["groups"].shape[0]
    out, sel, _ = decode.decode_step_unit(q, u["unit"], u["gn"], d, u["ks"], u["vs"], u["cb4"],
                                          u["cb3"], ng, 1 / math.sqrt(d))
    assert sel.tolist() == list(range(ng))
    np.testing.assert_allclose(out, _full_dense(u, q, 1 / math.sqrt(d)), rtol=1e-12, atol=1e-12)


def test_beta_zero_equals_l1_plus_all_summaries():
    u = make_unit(T=300, seed=5)
    d, gn = u["d"], u["gn"]
    rng = np.random.default_rng(10)
    q = rng.standard_normal((2, d))
    scale = 1 / math.sqrt(d)
    out, sel, _ = decode.decode_step_unit(q, u["unit"], gn, d, u["ks"], u["vs"], u["cb4"], u["cb3"],
                                          0, scale)
    assert sel.size == 0
    # independent construction: encode L1 tokens and group means directly
    ck, nk, _ = codec.encode(u["k"][u["l1"]], u["ks"], u["cb4"][1])
    cv, nv, _ = codec.encode(u["v"][u["l1"]], u["vs"], u["cb4"][1])
    mk = u["k"][u["groups"]].mean(axis=1)
    mv = u["v"][u["groups"]].mean(axis=1)
    sk, snk, _ = codec.encode(mk, u["ks"], u["cb3"][1])
    sv, snv, _ = codec.encode(mv, u["vs"], u["cb3"][1])
    keys = np.concatenate([codec.decode(ck, nk, u["ks"], u["cb4"][0]),
                           codec.decode(sk, snk, u["ks"], u["cb3"][0])])
    vals = np.concatenate([codec.decode(cv, nv, u["vs"], u["cb4"][0]),
                           codec.decode(sv, snv, u["vs"], u["cb3"][0])])
    want = np.stack([decode.softmax_attention(qh, keys, vals, scale) for qh in q])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_single_token_and_dominant_logit():
    d = 64
    c4, c3 = cb.codebook_f32(d, 4), cb.codebook_f32(d, 3)
    rng = np.random.default_rng(2)
    ks = rng.integers(0, 1 << 32, size=2, dtype=np.uint64).astype(np.uint32)
    vs = rng.integers(0, 1 << 32, size=2, dtype=np.uint64).astype(np.uint32)
    # T = 1: the output is the one dequantised value
    k = rng.standard_normal((1, d))
    v = rng.standard_normal((1, d))
    l1, groups = tiers.tier_plan(1, 4, 0, [], 8)
    unit = tiers.build_unit(k, v, l1, groups, ks, vs, c4, c3)
    out, _, _ = decode.decode_step_unit(rng.standard_normal((1, d)), unit, 8, d, ks, vs, c4, c3, 4,
                                        0.125)
    cv, nv, _ = codec.encode(v, vs, c4[1])
    np.testing.assert_allclose(out[0], codec.decode(cv, nv, vs, c4[0])[0], rtol=1e-13)
    # one key aligned with q by a large margin: output -> that token's value
    T = 64
    k = rng.standard_normal((T, d)) * 0.01
    v = rng.standard_normal((T, d))
    k[0] = 10.0 * np.ones(d)
    l1, groups = tiers.tier_plan(T, 1, 0, [], 8)
    unit = tiers.build_unit(k, v, l1, groups, ks, vs, c4, c3)
    q = np.ones((1, d))
    out, _, _ = decode.decode_step_unit(q, unit, 8, d, ks, vs, c4, c3, 2, 1 / math.sqrt(d))
    cv, nv, _ = codec.encode(v[:1], vs, c4[1])
    v0 = codec.decode(cv, nv, vs, c4[0])[0]
    np.testing.assert_allclose(out[0], v0, atol=1e-6 * np.abs(v0).max())


def test_l1_order_invariance():
    u = make_unit(seed=8)
    d, gn = u["d"], u["gn"]
    q = np.random.default_rng(1).standard_normal((2, d))
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    sel = np.array([1, 4, 6])
    a = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"], 0.1)
    perm = np.random.default_rng(2).permutation(deq["l1k"].shape[0])
    deq2 = dict(deq, l1k=deq["l1k"][perm], l1v=deq["l1v"][perm])
    b = decode.hsq_attention_unit(q, deq2, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"], 0.1)
    np.testing.assert_allclose(a, b, rtol=1e-12)


@pytest.mark.parametrize("agg,bias,given", [("max", 0.0, None), ("mean", -0.4, None),
                                             ("max", 0.9, [0, 3, 11])])
def test_decode_from_raw_equals_full_build(agg, bias, given):
    # encoding only what the step reads gives the full build's result
    u = make_unit(T=260, seed=12)
    d, gn = u["d"], u["gn"]
    q = np.random.default_rng(4).standard_normal((3, d))
    scale = 1 / math.sqrt(d)
    want, wsel, wsc = decode.decode_step_unit(q, u["unit"], gn, d, u["ks"], u["vs"], u["cb4"],
                                             u["cb3"], 5, scale, agg, bias)
    if given is not None:
        deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
        want = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], given, gn, d, u["ks"], u["vs"],
                                         u["cb4"], scale, bias)
    got, osel, sc, l2 = decode.decode_step_from_raw(
        q, u["k"], u["v"], u["l1"], u["groups"], u["ks"], u["vs"], u["cb4"], u["cb3"], 5, scale,
        agg, bias, sel=given)
    np.testing.assert_array_equal(osel, wsel)
    np.testing.assert_array_equal(sc, wsc)
    np.testing.assert_array_equal(l2["codes"], u["unit"]["l2k_codes"])
    np.testing.assert_array_equal(l2["y"], u["unit"]["l2k_y"])
    np.testing.assert_array_equal(l2["n"], u["unit"]["l2k_n"])
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_planted_needle_is_routed():
    # one group's keys aligned with the query must be selected
    u = make_unit(T=400, seed=6)
    d, gn = u["d"], u["gn"]
    g = 17
    k = u["k"].copy()
    q = np.random.default_rng(3).standard_normal((2, d))
    k[u["groups"][g]] = 3.0 * q[0] / np.linalg.norm(q[0]) * np.sqrt(d) + 0.1 * k[u["groups"][g]]
    unit = tiers.build_unit(k, u["v"], u["l1"], u["groups"], u["ks"], u["vs"], u["cb4"], u["cb3"])
    _, sel, scores = decode.decode_step_unit(q, unit, gn, d, u["ks"], u["vs"], u["cb4"], u["cb3"], 1,
                                             1 / math.sqrt(d))
    assert sel.tolist() == [g]


# ---------------------------------------------------------------------------
# Independent brute force on a tiny case: pure-Python loops, Sylvester
# Hadamard, nearest-centroid quantisation, explicit union of entries.

def _bf_rotate(x, signs_pm, H):
    d = len(x)
    return [sum(H[i][j] * signs_pm[j] * x[j] for j in range(d)) / math.sqrt(d) for i in range(d)]


def _bf_unrotate(y, signs_pm, H):
    d = len(y)
    return [signs_pm[i] * sum(H[j][i] * y[j] for j in range(d)) / math.sqrt(d) for i in range(d)]


def _bf_quant_dequant(x, signs_pm, H, cent):
    r = math.sqrt(sum(a * a for a in x))
    r32 = float(np.float32(r))
    if r == 0:
        u = [0.0] * len(x)
    else:
        u = [a / r for a in x]
    y = _bf_rotate(u, signs_pm, H)
    idx = []
    for yi in y:
        best, bj = None, 0
        for j, c in enumerate(cent):
            dd = abs(yi - c)
            if best is None or dd < best:
                best, bj = dd, j
        idx.append(bj)
    yq = [cent[j] for j in idx]
    return [r32 * a for a in _bf_unrotate(yq, signs_pm, H)], y


def test_route_scores_hand_worked_max_and_mean():
    # two query heads against three summary keys, scale 1/2:
    #   head 0: q = (1, 0): logits 0.5, 1.0, 0.0
    #   head 1: q = (0, 2): logits 1.0, -1.0, 0.0
    q = np.array([[1.0, 0.0], [0.0, 2.0]])
    khat = np.array([[1.0, 1.0], [2.0, -1.0], [0.0, 0.0]])
    s_max, lg = decode.route_scores(q, khat, 0.5, "max")
    s_mean, _ = decode.route_scores(q, khat, 0.5, "mean")
    np.testing.assert_array_equal(lg, [[0.5, 1.0, 0.0], [1.0, -1.0, 0.0]])
    np.testing.assert_array_equal(s_max, [1.0, 1.0, 0.0])
    np.testing.assert_array_equal(s_mean, [0.75, 0.0, 0.0])
    # max: groups 0 and 1 tie, the lower index wins; mean: group 0 alone
    assert decode.top_beta(s_max, 1).tolist() == [0]
    assert decode.top_beta(s_mean, 1).tolist() == [0]
    # mean, beta 2: groups 1 and 2 tie at 0, the lower index wins
    assert decode.top_beta(s_mean, 2).tolist() == [0, 1]
    with pytest.raises(ValueError):
        decode.route_scores(q, khat, 0.5, "median")


@pytest.mark.parametrize("bias", [0.0, -0.7, 1.3])
def test_summary_bias_hand_worked(bias):
    # one L1 token and one unfetched summary, both with key 0 (logit 0):
    # the softmax weights are 1 and e^bias, so
    #   out = (v_L1 + e^bias v_summary) / (1 + e^bias)
    d, gn = 4, 8
    deq = {"l1k": np.zeros((1, d)), "l1v": np.array([[1.0, 0.0, 0.0, 0.0]]),
           "l2k": np.zeros((1, d)), "l2v": np.array([[0.0, 2.0, 0.0, 0.0]])}
    l3 = np.zeros((1, gn * (d + 8)), dtype=np.uint8)
    signs = np.zeros(1, dtype=np.uint32)
    c4 = cb.codebook_f32(d, 4)
    q = np.array([[0.3, -0.2, 0.5, 0.1]])
    out = decode.hsq_attention_unit(q, deq, l3, [], gn, d, signs, signs, c4, 0.5, bias)
    e = math.exp(bias)
    np.testing.assert_allclose(out[0], [1.0 / (1 + e), 2.0 * e / (1 + e), 0.0, 0.0], rtol=1e-15)
    # a fetched summary takes no bias: with the group fetched the summary is
    # gone and the group's tokens enter unbiased
    out_f = decode.hsq_attention_unit(q, deq, l3, [0], gn, d, signs, signs, c4, 0.5, bias)
    # the fetched record is all-zero codes with zero norms: gn tokens with
    # key 0 and value 0 next to the L1 token
    np.testing.assert_allclose(out_f[0], [1.0 / (1 + gn), 0.0, 0.0, 0.0], rtol=1e-15)


@pytest.mark.parametrize("agg,bias", [("max", 0.0), ("mean", 0.0), ("max", -0.7), ("mean", 1.3)])
def test_brute_force_tiny_end_to_end(agg, bias):
    d, T, gn, beta = 8, 40, 4, 2
    rng = np.random.default_rng(21)
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    q = rng.standard_normal((2, d))
    ks = np.array([0b10110010], dtype=np.uint32)
    vs = np.array([0b01001101], dtype=np.uint32)
    c4, c3 = cb.codebook_f32(d, 4), cb.codebook_f32(d, 3)
    marked = [9, 22]
    l1, groups = tiers.tier_plan(T, 2, 5, marked, gn)
    unit = tiers.build_unit(k, v, l1, groups, ks, vs, c4, c3)
    scale = 1 / math.sqrt(d)
    out, sel, scores = decode.decode_step_unit(q, unit, gn, d, ks, vs, c4, c3, beta, scale,
                                               agg=agg, summary_bias=bias)

    # --- brute force ---
    H = [[1]]
    while len(H) < d:
        H = [row + row for row in H] + [row + [-a for a in row] for row in H]
    spm_k = [(-1.0 if (int(ks[0]) >> i) & 1 else 1.0) for i in range(d)]
    spm_v = [(-1.0 if (int(vs[0]) >> i) & 1 else 1.0) for i in range(d)]
    cent4 = [float(c) for c in c4[0]]
    cent3 = [float(c) for c in c3[0]]
    l1set = set(range(2)) | set(range(T - 5, T)) | set(marked)
    rest = [p for p in range(T) if p not in l1set]
    ngb = len(rest) // gn
    for p in rest[ngb * gn:]:
        l1set.add(p)
    grp = [rest[i * gn:(i + 1) * gn] for i in range(ngb)]
    near_thr = False
    kh4, vh4, sk, sv = {}, {}, [], []
    for p in range(T):
        kh4[p], yk = _bf_quant_dequant(list(k[p]), spm_k, H, cent4)
        vh4[p], yv = _bf_quant_dequant(list(v[p]), spm_v, H, cent4)
        near_thr |= min(abs(a - t) for a in yk + yv for t in c4[1]) < 1e-9
    for gpos in grp:
        mk = [sum(k[p][i] for p in gpos) / gn for i in range(d)]
        mv = [sum(v[p][i] for p in gpos) / gn for i in range(d)]
        a, _ = _bf_quant_dequant(mk, spm_k, H, cent3)
        b, _ = _bf_quant_dequant(mv, spm_v, H, cent3)
        sk.append(a)
        sv.append(b)
    assert not near_thr
    dot = lambda a, b: sum(x * y for x, y in zip(a, b))
    if agg == "max":
        bf_scores = [max(scale * dot(qh, sk[g]) for qh in q) for g in range(ngb)]
    else:
        bf_scores = [sum(scale * dot(qh, sk[g]) for qh in q) / len(q) for g in range(ngb)]
    np.testing.assert_allclose(scores, bf_scores, rtol=1e-12, atol=1e-12)
    ranked = sorted(range(ngb), key=lambda g: (-bf_scores[g], g))[:beta]
    assert sorted(ranked) == sel.tolist()
    for h, qh in enumerate(q):
        ents = [(scale * dot(qh, kh4[p]), vh4[p]) for p in sorted(l1set)]
        ents += [(scale * dot(qh, sk[g]) + bias, sv[g]) for g in range(ngb) if g not in ranked]
        ents += [(scale * dot(qh, kh4[p]), vh4[p]) for g in ranked for p in grp[g]]
        m = max(e[0] for e in ents)
        w = [math.exp(e[0] - m) for e in ents]
        o = [sum(wi * e[1][i] for wi, e in zip(w, ents)) / sum(w) for i in range(d)]
        np.testing.assert_allclose(out[h], o, rtol=1e-11, atol=1e-12)


# ---- pre-RoPE archive: the fetched keys are rotated to their positions ----

def _prerope_unit(T=240, d=64, gn=8, seed=21, base=1e4):
    """A unit whose L1 and L2 come from embedded keys and whose L3 archive
    holds the keys before the rotary embedding (k_pre); k_post = RoPE(k_pre)
    at positions 0 .. T-1 (oracle.rope)."""
    u = make_unit(T=T, d=d, gn=gn, seed=seed)
    k_pre = u["k"]
    k_post = rope.rope(k_pre, np.arange(T), base)
    post = tiers.build_unit(k_post, u["v"], u["l1"], u["groups"], u["ks"], u["vs"], u["cb4"],
                            u["cb3"])
    pre = tiers.build_unit(k_pre, u["v"], u["l1"], u["groups"], u["ks"], u["vs"], u["cb4"],
                           u["cb3"])
    unit = dict(post)
    unit["l3"] = pre["l3"]
    return dict(u, unit=unit, k_pre=k_pre, k_post=k_post, base=base)


def test_prerope_positions_zero_is_the_plain_step():
    # RoPE at position 0 is the identity: with every group at position 0 the
    # pre-RoPE attention is the plain one on the same archive
    u = _prerope_unit()
    d, gn = u["d"], u["gn"]
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, d))
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    sel = np.array([0, 3, 7, 11])
    zero = np.zeros_like(u["groups"])
    a = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d), group_pos=zero, rope_base=u["base"])
    b = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d))
    np.testing.assert_array_equal(a, b)


def test_prerope_all_fetched_equals_dense_attention():
    # beta = ng: the L1 tokens (embedded keys, each encoded at 4 bits) and every
    # grouped token (its pre-embedding key encoded at 4 bits, decoded, then
    # rotated to its position with the textbook pair rotation written out
    # here) in one dense softmax
    u = _prerope_unit()
    d, gn, base = u["d"], u["gn"], u["base"]
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, d)) * 2
    scale = 1 / math.sqrt(d)
    ng = u["groups"].shape[0]
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    got = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], np.arange(ng), gn, d, u["ks"],
                                    u["vs"], u["cb4"], scale, group_pos=u["groups"],
                                    rope_base=base)

    def enc_dec(x, signs):
        c, n, _ = codec.encode(x, signs, u["cb4"][1])
        return codec.decode(c, n, signs, u["cb4"][0])

    gpos = u["groups"].reshape(-1)
    kg = enc_dec(u["k_pre"][gpos], u["ks"])
    half = d // 2
    out = np.empty_like(kg)
    for r, p in enumerate(gpos):
        for i in range(half):
            a = p * base ** (-2.0 * i / d)
            out[r, i] = kg[r, i] * math.cos(a) - kg[r, i + half] * math.sin(a)
            out[r, i + half] = kg[r, i + half] * math.cos(a) + kg[r, i] * math.sin(a)
    keys = np.concatenate([enc_dec(u["k_post"][u["l1"]], u["ks"]), out])
    vals = np.concatenate([enc_dec(u["v"][u["l1"]], u["vs"]), enc_dec(u["v"][gpos], u["vs"])])
    want = np.stack([decode.softmax_attention(qh, keys, vals, scale) for qh in q])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_prerope_rotation_matters():
    # the embedding is not a no-op: at real positions the fetched keys, and so
    # the output, differ from the plain step on the same archive
    u = _prerope_unit()
    d, gn = u["d"], u["gn"]
    q = np.random.default_rng(5).standard_normal((1, d)) * 3
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    sel = np.arange(u["groups"].shape[0])
    a = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d), group_pos=u["groups"], rope_base=u["base"])
    b = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d))
    assert np.linalg.norm(a - b) > 1e-3 * np.linalg.norm(b)


# ---- TQ-QKV token keys in the decode step ----------------------------------
# Ablation page, "Key contributions" 1: TQ-QKV = TQ-KV plus a 1-bit QJL sketch
# of the key residual.  Read for the step: every 4-bit token key (L1 and the
# archive) carries its sketch and gamma; the summaries do not.

def _qjl_unit(T=220, d=64, gn=8, seed=31):
    u = make_unit(T=T, d=d, gn=gn, seed=seed)
    S = np.random.default_rng(seed + 1).standard_normal((d, d))
    sk = qjl.unit_sketches(u["k"], u["l1"], u["groups"], u["ks"], u["cb4"][1], u["cb4"][0], S)
    return dict(u, S=S, sk=dict(sk, S=S))


def _enc_dec(x, signs, c4):
    c, n, _ = codec.encode(x, signs, c4[1])
    return codec.decode(c, n, signs, c4[0])


def test_qjl_zero_gamma_is_the_plain_step():
    # gamma = 0 on every key: the correction vanishes and the step is TQ-KV
    u = _qjl_unit()
    d, gn = u["d"], u["gn"]
    q = np.random.default_rng(2).standard_normal((3, d))
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    sel = np.array([1, 4, 9])
    sk = dict(u["sk"], l1_gamma=np.zeros_like(u["sk"]["l1_gamma"]),
              l3_gamma=np.zeros_like(u["sk"]["l3_gamma"]))
    a = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d), 0.3, qjl=sk)
    b = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], sel, gn, d, u["ks"], u["vs"], u["cb4"],
                                  1 / math.sqrt(d), 0.3)
    np.testing.assert_array_equal(a, b)


def _dense(q, logits, vals):
    s = logits - logits.max()
    w = np.exp(s)
    return (w[:, None] * vals).sum(axis=0) / w.sum()


def test_qjl_all_fetched_equals_dense_attention_over_tq_qkv_logits():
    # beta = ng: one softmax over the L1 tokens and every grouped token, each
    # logit the codec-level TQ-QKV logit of its key (qjl.logits_qjl over the
    # key's own encode and sketch), values dequantised at 4 bits
    u = _qjl_unit()
    d, gn, S = u["d"], u["gn"], u["S"]
    q = np.random.default_rng(4).standard_normal((2, d)) * 2
    scale = 1 / math.sqrt(d)
    ng = u["groups"].shape[0]
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    got = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], np.arange(ng), gn, d, u["ks"],
                                    u["vs"], u["cb4"], scale, qjl=u["sk"])
    rows = np.concatenate([u["l1"], u["groups"].reshape(-1)])
    e = qjl.encode(u["k"][rows], u["ks"], u["cb4"][1], u["cb4"][0], S)
    lg = qjl.logits_qjl(q, e["codes"], e["norms"], e["bits"], e["gamma"], u["ks"], u["cb4"][0], S,
                        scale)
    vals = _enc_dec(u["v"][rows], u["vs"], u["cb4"])
    want = np.stack([_dense(q[h], lg[h], vals) for h in range(q.shape[0])])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_qjl_correction_enters_token_logits_only():
    # nothing fetched: the L1 tokens take the TQ-QKV logit, every summary its
    # plain logit plus the bias; and the correction is not a no-op
    u = _qjl_unit(seed=37)
    d, gn, S = u["d"], u["gn"], u["S"]
    q = np.random.default_rng(6).standard_normal((1, d)) * 3
    scale, bias = 1 / math.sqrt(d), -0.4
    deq = decode.dequant_unit(u["unit"], d, gn, u["ks"], u["vs"], u["cb4"], u["cb3"])
    none = np.zeros(0, dtype=np.int64)
    got = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], none, gn, d, u["ks"], u["vs"],
                                    u["cb4"], scale, bias, qjl=u["sk"])
    e = qjl.encode(u["k"][u["l1"]], u["ks"], u["cb4"][1], u["cb4"][0], S)
    l1 = qjl.logits_qjl(q, e["codes"], e["norms"], e["bits"], e["gamma"], u["ks"], u["cb4"][0], S,
                        scale)[0]
    l2 = scale * (deq["l2k"] @ q[0]) + bias
    vals = np.concatenate([_enc_dec(u["v"][u["l1"]], u["vs"], u["cb4"]), deq["l2v"]])
    want = _dense(q[0], np.concatenate([l1, l2]), vals)
    np.testing.assert_allclose(got[0], want, rtol=1e-12, atol=1e-12)
    plain = decode.hsq_attention_unit(q, deq, u["unit"]["l3"], none, gn, d, u["ks"], u["vs"],
                                      u["cb4"], scale, bias)
    assert np.abs(got - plain).max() > 1e-4
