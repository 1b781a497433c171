"""hsq_decode_step_static (the decode step with the library's static device
scratch as its workspace) against hsq_decode_step with a caller workspace,
through the C ABI: two calls in a row on one stream, the second with a
smaller input.  Both shapes take the split step (fewer than 128 units),
whose kernels keep their logits, keys, selection and partials in the
workspace; the results must be identical bit for bit (the same kernels)."""
import math

import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from oracle import codebook as ocb

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(w):
    k, v = W.kv(w, 0, DEV)
    q = W.query(w, 0, DEV)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    dks = torch.from_numpy(ks.view(np.int32)).to(DEV)
    dvs = torch.from_numpy(vs.view(np.int32)).to(DEV)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = torch.from_numpy(np.stack([p[0] for p in plans])).to(DEV)
    gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in plans])).to(DEV)
    c4, c3 = ocb.codebook_f32(w.d, 4), ocb.codebook_f32(w.d, 3)
    cb4, cb3 = (torch.from_numpy(np.array(c[0])).to(DEV) for c in (c4, c3))
    t4, t3 = (torch.from_numpy(np.array(c[1])).to(DEV) for c in (c4, c3))
    tiers = hsq.build_tiers(k, v, l1, gp, w.group_n, dks, dvs, t4, t3)
    return q, tiers, dks, dvs, cb4, cb3


def test_static_scratch_matches_workspace():
    big = W.QWEN3_8B_8K.smaller(T=4096, batch=2, n_marked=80)
    small = W.QWEN3_14B_16K.smaller(T=1500, batch=1, hkv=4, hq=20, n_marked=15)
    for w in (big, small):  # the second call is the smaller one
        print(f"static scratch: {w.name} B={w.batch} Hkv={w.hkv} T={w.T}", flush=True)
        q, t, dks, dvs, cb4, cb3 = _layer(w)
        assert w.batch * w.hkv < 128  # the split step, which uses the workspace
        o_s, i_s = hsq.decode_step_static(q, t, w.beta, dks, dvs, cb4, cb3)
        torch.cuda.synchronize()
        o_w, i_w = hsq.decode_step(q, t, w.beta, dks, dvs, cb4, cb3)
        torch.cuda.synchronize()
        assert torch.equal(i_s, i_w)
        assert torch.equal(o_s, o_w)
        assert torch.isfinite(o_s).all()


def test_static_scratch_rejects_oversized():
    # a shape whose workspace exceeds the 8 MiB static scratch is refused
    # before any launch (sizes only; no device data is read)
    lib = hsq.lib()
    need = hsq.workspace_bytes(64, 256, 64, 128, 736, 16000, 64, 8)
    assert need > 8 << 20
    rc = lib.hsq_decode_step_static(1, 64, 256, 64, 128, 1, 1, 1, 1, 736, 1, 1, 1, 1, 16000, 1, 8,
                                    64, 0, 1, 1, 1, 1, 1.0 / math.sqrt(128), 0.0, None, 1, None)
    assert rc == -2, rc
    assert b"static scratch holds" in lib.hsq_last_error()
