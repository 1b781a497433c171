"""Pins of the oracle's decode-time tier maintenance (oracle/cache.py).

Page: "Tamarin (HSQ)" summary, section 2, "Three-tier architecture" (L1 =
sinks + recent window + reader-marked tokens; the rest in groups of N with a
3-bit summary in L2 and the 4-bit originals in L3).  The incremental cache is
checked against the compress-time build of the longer context, which the
tier-plan and tier-build pins cover on their own.
"""
import math

import numpy as np
import pytest

from oracle import cache, codec, decode, tiers
from oracle import codebook as cb


def make(T0, K, d, ns, nr, nm, gn, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T0 + K, d))
    v = rng.standard_normal((T0 + K, d))
    marked = np.sort(rng.choice(np.arange(ns, T0 - nr), size=nm, replace=False))
    ks = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    vs = rng.integers(0, 1 << 32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    cb4, cb3 = cb.codebook_f32(d, 4), cb.codebook_f32(d, 3)
    c = cache.UnitCache(k[:T0], v[:T0], ns, nr, marked, gn, ks, vs, cb4, cb3)
    return c, k, v, marked, ks, vs, cb4, cb3


def assert_same_as_build(c, k, v, marked, ks, vs, cb4, cb3):
    T = c.T
    l1, groups = tiers.tier_plan(T, c.n_sink, c.n_recent, marked, c.gn)
    want = tiers.build_unit(k[:T], v[:T], l1, groups, ks, vs, cb4, cb3)
    got = c.as_unit()
    np.testing.assert_array_equal(got["l1_pos"], l1)
    np.testing.assert_array_equal(got["groups"], groups)
    for key in ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n", "l3"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=f"{key} at T={T}")


@pytest.mark.parametrize("T0,d,ns,nr,nm,gn", [(200, 64, 4, 16, 10, 8), (203, 64, 4, 32, 16, 8),
                                              (300, 128, 4, 64, 7, 16)])
def test_appends_equal_the_build_of_the_longer_context(T0, d, ns, nr, nm, gn):
    K = 3 * gn + 3  # crosses three seals and ends with pending tokens
    c, k, v, marked, ks, vs, cb4, cb3 = make(T0, K, d, ns, nr, nm, gn, seed=T0 + d)
    assert_same_as_build(c, k, v, marked, ks, vs, cb4, cb3)
    for t in range(T0, T0 + K):
        c.append(k[t], v[t])
        if d == 64 or (t - T0) % 5 == 4 or len(c.pending) == 0:
            assert_same_as_build(c, k, v, marked, ks, vs, cb4, cb3)
    assert c.T == T0 + K


def test_group_count_and_l1_size_cycle_with_period_n():
    gn, ns, nr, nm = 8, 4, 16, 10
    c, k, v, *_ = make(200, 40, 64, ns, nr, nm, gn, seed=3)
    seen = []
    for t in range(200, 240):
        ng0 = c.n_groups
        c.append(k[t], v[t])
        seen.append(c.n_groups - ng0)
        # L1 = sinks + marks + window + pending (fewer than N)
        assert len(c.l1) == ns + nm + nr + len(c.pending)
        assert 0 <= len(c.pending) < gn
    # one seal every N appends
    assert sum(seen) == 40 // gn
    s = np.nonzero(seen)[0]
    assert np.all(np.diff(s) == gn)


def test_seal_uses_the_raw_mean_not_the_dequantised_tokens():
    # the summary of a sealed group is the 3-bit code of the mean of its raw
    # vectors (reading of the compressor), computed here independently
    gn = 8
    c, k, v, marked, ks, vs, cb4, cb3 = make(200, 16, 64, 4, 16, 10, gn, seed=11)
    ng0 = c.n_groups
    t = 200
    while c.n_groups == ng0:
        c.append(k[t], v[t])
        t += 1
    g = c.groups[-1]
    mk = k[np.array(g["pos"])].mean(axis=0, keepdims=True)
    code, norm, _ = codec.encode(mk, ks, cb3[1])
    np.testing.assert_array_equal(g["l2k"], code[0])
    assert g["l2k_n"] == norm[0]
    # the group is the N oldest positions outside sinks, marks and the window
    assert g["pos"] == sorted(g["pos"]) and len(g["pos"]) == gn
    assert max(g["pos"]) < c.T - c.n_recent


def test_decode_on_appended_cache_with_all_groups_is_dense_attention():
    d, gn = 64, 8
    c, k, v, marked, ks, vs, cb4, cb3 = make(160, 21, d, 4, 16, 6, gn, seed=5)
    for t in range(160, 181):
        c.append(k[t], v[t])
    u = c.as_unit()
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, d)) * 2
    scale = 1 / math.sqrt(d)
    out, sel, _ = decode.decode_step_unit(q, u, gn, d, ks, vs, cb4, cb3, c.n_groups, scale)
    ck, nk, _ = codec.encode(k[:c.T], ks, cb4[1])
    cv, nv, _ = codec.encode(v[:c.T], vs, cb4[1])
    kh, vh = codec.decode(ck, nk, ks, cb4[0]), codec.decode(cv, nv, vs, cb4[0])
    want = np.stack([decode.softmax_attention(qh, kh, vh, scale) for qh in q])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


def test_prefix_must_hold_a_full_window_past_the_sinks():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((30, 64))
    cb4, cb3 = cb.codebook_f32(64, 4), cb.codebook_f32(64, 3)
    s = np.zeros(2, np.uint32)
    with pytest.raises(ValueError):
        cache.UnitCache(k, k, 4, 32, [], 8, s, s, cb4, cb3)
    with pytest.raises(ValueError):  # a mark inside the window
        cache.UnitCache(k, k, 4, 16, [20], 8, s, s, cb4, cb3)
