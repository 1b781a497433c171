"""Host-side tests of libhsq: it loads, exports every declared symbol, its host
functions agree with the oracle, and argument errors are reported before any
launch (none of these calls touches a GPU)."""
import ctypes
import re
import os

import numpy as np
import pytest

from compressed_decode_attention_turboquant_amd import hsq
from oracle import codebook as ocb
from oracle import tiers as otiers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    src = open(os.path.join(ROOT, "include", "hsq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hsq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = hsq.lib()
    declared = header_symbols()
    assert declared == hsq.exported_symbols()
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.hsq_version().decode().startswith("hsq")


@pytest.mark.parametrize("d,bits", [(64, 3), (64, 4), (128, 3), (128, 4), (16, 2), (3, 3), (256, 4)])
def test_codebook_matches_oracle(d, bits):
    c, t = hsq.codebook(d, bits)
    oc, ot = ocb.codebook_f32(d, bits)
    # two independent double-precision generators, rounded to fp32: equal up to
    # one fp32 ulp (a value sitting on a rounding boundary may round either way)
    np.testing.assert_array_max_ulp(c, oc, maxulp=1)
    np.testing.assert_array_max_ulp(t, ot, maxulp=1)
    assert t[len(t) // 2] == 0.0
    np.testing.assert_array_equal(c, -c[::-1])


def test_codebook_tables_for_the_codec_are_identical():
    for d in (64, 128):
        for bits in (3, 4):
            c, t = hsq.codebook(d, bits)
            oc, ot = ocb.codebook_f32(d, bits)
            np.testing.assert_array_equal(c, oc)
            np.testing.assert_array_equal(t, ot)


@pytest.mark.parametrize("T,ns,nr,nm,gn", [(512, 4, 32, 16, 8), (8192, 4, 64, 164, 16),
                                           (300, 4, 64, 7, 16), (50, 4, 64, 0, 8), (1, 4, 0, 0, 8),
                                           (1000, 0, 0, 0, 8)])
def test_tier_plan_matches_oracle(T, ns, nr, nm, gn):
    rng = np.random.default_rng(T + nm)
    lo, hi = ns, max(T - nr, ns)
    marked = np.sort(rng.choice(np.arange(lo, hi), size=min(nm, max(hi - lo, 0)), replace=False))
    l1, groups = hsq.tier_plan(T, ns, nr, marked, gn)
    ol1, og = otiers.tier_plan(T, ns, nr, marked, gn)
    np.testing.assert_array_equal(l1, ol1)
    np.testing.assert_array_equal(groups, og)


def test_argument_errors_are_reported_without_launch():
    lib = hsq.lib()
    c = np.zeros(16, np.float32)
    assert lib.hsq_codebook(2, 4, c.ctypes.data, c.ctypes.data) == -1
    assert lib.hsq_codebook(64, 5, c.ctypes.data, c.ctypes.data) == -1
    assert lib.hsq_codebook(64, 4, None, c.ctypes.data) == -1
    assert "null" in lib.hsq_last_error().decode()
    # encode: unsupported d / bits / dtype, null pointers, bad sizes
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert lib.hsq_encode(p, 0, 10, 96, 4, None, 1, p, 1, 1, p, p, p, None) == -2
    assert lib.hsq_encode(p, 0, 10, 128, 1, None, 1, p, 1, 1, p, p, p, None) == -2
    assert lib.hsq_encode(p, 0, 10, 128, 5, None, 1, p, 1, 1, p, p, p, None) == -2
    assert lib.hsq_decode(p, p, 10, 128, 1, None, 1, 1, p, p, 0, None) == -2
    assert lib.hsq_decode(p, p, 10, 128, 5, None, 1, 1, p, p, 0, None) == -2
    # vector counts of 2^32 and more are refused before any launch
    assert lib.hsq_encode(p, 0, 1 << 32, 128, 4, None, 1, p, 1, 1, p, p, p, None) == -2
    assert lib.hsq_decode(p, p, 1 << 32, 128, 4, p, 1, 1, p, p, 0, None) == -2
    assert lib.hsq_build_tiers(p, p, 0, 1 << 16, 1 << 8, 1 << 8, 128, p, 16, p, 4, 8, p, p, p, p,
                               p, p, p, p, p, p, p, p, p, None) == -2
    # signs may be null (rotation off); the other pointers may not
    assert lib.hsq_encode(p, 0, 10, 128, 2, None, 1, None, 1, 1, None, p, p, None) == -1
    assert lib.hsq_decode(p, p, 10, 128, 2, None, 1, 1, None, p, 0, None) == -1
    assert lib.hsq_encode(p, 7, 10, 128, 4, None, 1, p, 1, 1, p, p, p, None) == -2
    assert lib.hsq_encode(None, 0, 10, 128, 4, None, 1, p, 1, 1, p, p, p, None) == -1
    assert lib.hsq_encode(p, 0, -1, 128, 4, None, 1, p, 1, 1, p, p, p, None) == -1
    assert lib.hsq_encode(p, 0, 10, 128, 4, None, 0, p, 1, 1, p, p, p, None) == -1
    assert lib.hsq_encode(None, 0, 0, 128, 4, None, 1, None, 1, 1, None, None, None, None) == 0
    # decode-step shapes: Hq % Hkv, G > 8, group size, beta < 0, workspace
    assert lib.hsq_workspace_bytes(1, 10, 4, 128, 10, 10, 2, 16) == 0
    assert lib.hsq_workspace_bytes(1, 36, 4, 128, 10, 10, 2, 16) == 0
    assert lib.hsq_workspace_bytes(1, 32, 8, 128, 10, 10, 2, 12) == 0
    assert lib.hsq_workspace_bytes(1, 32, 8, 128, 10, 10, -1, 16) == 0
    assert lib.hsq_workspace_bytes(1, 32, 8, 128, 10, 10, 2, 16) > 0
    assert lib.hsq_route_topk(p, 1, 32, 8, 128, p, p, 10, p, p, ctypes.c_float(0.1), 0, 2, p,
                              None, None, 0, None) == -4
    assert lib.hsq_route_topk(p, 1, 32, 8, 128, p, p, 10, p, p, ctypes.c_float(0.1), 9, 2, p,
                              None, None, 0, None) == -1
    assert lib.hsq_gather_l3(p, 100, 1, 1, 4, p, 2, p, None) == -1
    assert lib.hsq_gather_l3(p, 1088, 1, 1, 4, p, 5, p, None) == -1
    assert lib.hsq_gather_l3(p, (1 << 20) + 16, 1, 1, 4, p, 2, p, None) == -2
    # pre-RoPE step: workspace size (the plain one plus the fetched rows),
    # null positions, bad rotary base, workspace of only the plain size
    plain = lib.hsq_workspace_bytes(2, 32, 8, 128, 10, 10, 4, 16)
    pre = lib.hsq_prerope_workspace_bytes(2, 32, 8, 128, 10, 10, 4, 16)
    assert pre >= plain + 2 * 8 * 4 * 16 * 128 * 2
    assert lib.hsq_prerope_workspace_bytes(1, 36, 4, 128, 10, 10, 2, 16) == 0

    def pre_step(pos=p, base=1e6, ws_bytes=pre, ws=ctypes.c_void_p(256)):
        f = ctypes.c_float(0.1)
        return lib.hsq_decode_step_prerope(p, 2, 32, 8, 128, p, p, p, p, 10, p, p, p, p, 10, p,
                                           16, 4, 0, p, p, p, p, f, f, pos, base, None, ws,
                                           ws_bytes, p, None)

    assert pre_step(pos=None) == -1
    assert "group_pos" in lib.hsq_last_error().decode()
    assert pre_step(base=0.0) == -1
    assert pre_step(base=float("inf")) == -1
    assert pre_step(ws_bytes=plain) == -4
    assert pre_step(ws=None) == -4
    # TQ-QKV step: null S, null sketches of a tier that has entries
    def qjl_step(l1s=p, l1g=p, l3s=p, l3g=p, S=p, n_l1=10, ng=10):
        f = ctypes.c_float(0.1)
        return lib.hsq_decode_step_qjl(p, 2, 32, 8, 128, p, p, p, p, n_l1, p, p, p, p, ng, p, 16,
                                       4, 0, p, p, p, p, f, f, l1s, l1g, l3s, l3g, S, None,
                                       ctypes.c_void_p(256), plain, p, None)

    assert qjl_step(S=None) == -1
    assert "S" in lib.hsq_last_error().decode()
    assert qjl_step(l1s=None) == -1
    assert qjl_step(l3g=None) == -1
    assert qjl_step(S=ctypes.c_void_p(20)) == -1
    assert "aligned" in lib.hsq_last_error().decode()
    assert qjl_step(l1s=ctypes.c_void_p(18)) == -1
    assert lib.hsq_gather_l3_ordered(p, 1088, 1, 1, 4, p, 2, p, None, 0, None) == -1
    assert "turn" in lib.hsq_last_error().decode()
    assert lib.hsq_gather_l3_ordered(p, 1088, 1, 1, 4, p, 2, p, ctypes.c_void_p(18), 0, None) == -1
    assert lib.hsq_gather_l3_ordered(p, 1088, 1, 1, 4, p, 5, p, p, 0, None) == -1
    assert lib.hsq_tier_plan(10, 1, 1, None, 3, 8, None, None, None, None) == -1


def test_cache_argument_errors_are_reported_without_launch():
    lib = hsq.lib()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    P = [p] * 16

    def app(dtype=0, B=1, Hkv=1, d=128, N=8, n_fix=4, W=16, t=100, pend=0, ng=3, l1_cap=28,
            ng_cap=10, ptrs=None):
        return lib.hsq_cache_append(p, p, dtype, B, Hkv, d, N, n_fix, W, t, pend, ng, l1_cap,
                                    ng_cap, *(ptrs or P)[:4], *(ptrs or P)[4:15], None)

    assert app(d=96) == -2
    assert app(N=12) == -2
    assert app(dtype=5) == -2
    assert app(t=15) == -1                 # window not full
    assert app(pend=8) == -1               # pending must be < N
    assert app(l1_cap=27) == -1            # no room for the pending tokens
    assert app(pend=7, ng=10) == -1        # a seal with the group capacity full
    assert app(ng=11) == -1
    assert app(ptrs=[p] * 10 + [None] + [p] * 5) == -1
    assert "null" in lib.hsq_last_error().decode()
    f = ctypes.c_float(0.1)

    def step(n_l1=20, l1_cap=28, ng=3, ng_cap=10, G=4):
        return lib.hsq_cache_decode_step(p, 1, 8 * G, 8, 128, p, p, p, p, n_l1, l1_cap, p, p, p,
                                         p, ng, ng_cap, p, 8, 2, 0, p, p, p, p, f, f, None, None,
                                         0, p, None)

    assert step(l1_cap=19) == -1           # capacity below the count
    assert step(ng_cap=2) == -1
    assert step(G=9) == -2
    assert step() == -4                    # no workspace


def test_qjl_argument_errors_are_reported_without_launch():
    lib = hsq.lib()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    P = [p] * 9
    enc = lambda d=128, bits=4, dtype=0, n=10, ptrs=P: lib.hsq_encode_qjl(p, dtype, n, d, bits,
                                                                          *ptrs[:8], None)
    assert enc(d=96) == -2
    assert enc(bits=2) == -2
    assert enc(dtype=3) == -2
    assert enc(n=-1) == -1
    assert enc(ptrs=[p] * 4 + [None] + [p] * 4) == -1
    assert "null" in lib.hsq_last_error().decode()
    assert enc(n=0, ptrs=[None] * 9) == 0  # nothing to do
    f = ctypes.c_float(0.1)
    lg = lambda n_q=4, d=128, bits=4, n=10: lib.hsq_qjl_logits(p, n_q, d, bits, p, p, p, p, n, p,
                                                                p, p, f, p, None)
    assert lg(n_q=0) == -1
    assert lg(n_q=9) == -1
    assert lg(d=32) == -2
    assert lg(bits=5) == -2
    assert lg(n=-1) == -1


def test_decode_rope_argument_errors_are_reported_without_launch():
    lib = hsq.lib()
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first

    def call(n=10, d=128, bits=4, base=1e6, pos=p, out_dtype=0, signs=p):
        return lib.hsq_decode_rope(p, p, n, d, bits, signs, 1, 1, p, pos, ctypes.c_double(base),
                                   p, out_dtype, None)

    assert call(d=96) == -2 and call(bits=5) == -2 and call(out_dtype=3) == -2
    assert call(n=1 << 32) == -2
    assert call(n=-1) == -1
    assert call(pos=None) == -1 and "null" in lib.hsq_last_error().decode()
    for base in (0.0, -2.0, float("inf"), float("nan")):
        assert call(base=base) == -1
        assert "rope_base" in lib.hsq_last_error().decode()
    assert call(n=0, pos=None) == 0  # empty: no-op before the pointer checks
