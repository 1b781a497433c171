"""GPU parity of the pinned-host archive path: hsq_gather_l3 on a side stream
between hsq_step_route and hsq_step_attend (l3_staged = 1).

Page: "Tamarin (HSQ)" summary, section 2, "Decode process" step 2 (the
originals of the chosen groups are fetched from the CPU archive) and section 4
"Results" (that fetch is the long-context bottleneck).  Workload: the
Qwen3-8B-shaped layer at 32K context, batch 8, N = 16, beta = 64, one layer of
the 36 the bench runs.
"""
import numpy as np
import pytest
import torch

from compressed_decode_attention_turboquant_amd import hsq
from compressed_decode_attention_turboquant_amd import workloads as W
from tests.test_gpu_step import Scenario, check_attn, check_route

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("where", ["host", "device"])
def test_gather_copies_the_selected_records(where):
    print(f"[gather] source in {where} memory", flush=True)
    B, Hkv, ng, beta, rec = 3, 2, 50, 7, 16 * (128 + 8)
    g = torch.Generator().manual_seed(5)
    src = torch.randint(0, 256, (B, Hkv, ng, rec), dtype=torch.uint8, generator=g)
    idx = torch.stack([torch.sort(torch.randperm(ng, generator=g)[:beta])[0]
                       for _ in range(B * Hkv)]).reshape(B, Hkv, beta).to(torch.int32)
    if where == "host":
        arch = hsq.HostArchive(src.numel())
        arch.host.copy_(src.reshape(-1))
        ptr = arch.dev_ptr
    else:
        dsrc = src.to(DEV)
        ptr = dsrc.data_ptr()
    staging = torch.zeros((B, Hkv, beta, rec), dtype=torch.uint8, device=DEV)
    hsq.gather_l3(ptr, rec, B, Hkv, ng, idx.to(DEV), staging)
    torch.cuda.synchronize()
    want = torch.stack([src[b, h, idx[b, h].long()] for b in range(B) for h in range(Hkv)])
    assert torch.equal(staging.cpu().reshape(B * Hkv, beta, rec), want)


def test_host_archive_step_matches_the_device_archive_step():
    w = W.QWEN3_8B_32K.smaller(layers=1)
    print(f"[host archive] {w.name} T={w.T} B={w.batch} beta={w.beta}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    rec, beta = t.rec_bytes, min(w.beta, t.ng)
    arch = hsq.HostArchive(t.l3.numel())  # pinned host copy of the archive
    arch.host.copy_(t.l3.reshape(-1).cpu())
    ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    idx = torch.empty((w.batch, w.hkv, beta), dtype=torch.int32, device=DEV)
    staging = torch.empty((w.batch, w.hkv, beta, rec), dtype=torch.uint8, device=DEV)
    out_host = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=DEV)
    out_dev = torch.empty_like(out_host)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    # as the bench runs it: route, the gather on a side stream, attend
    with torch.cuda.stream(main):
        hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws, idx=idx)
        ev = torch.cuda.Event()
        ev.record(main)
    with torch.cuda.stream(side):
        side.wait_event(ev)
        hsq.gather_l3(arch.dev_ptr, rec, w.batch, w.hkv, t.ng, idx, staging)
        ev2 = torch.cuda.Event()
        ev2.record(side)
    with torch.cuda.stream(main):
        main.wait_event(ev2)
        hsq.step_attend(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, ws, out_host,
                        l3=staging.data_ptr(), l3_staged=True)
        # the same two launches reading the archive in device memory in place
        hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws)
        hsq.step_attend(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, ws, out_dev)
    torch.cuda.synchronize()
    # staged records are the selected ones, byte for byte
    l3 = t.l3.reshape(w.batch * w.hkv, t.ng, rec)
    ix = idx.reshape(w.batch * w.hkv, beta).long()
    assert torch.equal(staging.reshape(w.batch * w.hkv, beta, rec),
                       torch.stack([l3[u, ix[u]] for u in range(w.batch * w.hkv)]))
    # the same kernels over the same record bytes: identical outputs
    assert torch.equal(out_host, out_dev)
    units = [(0, 0), (3, 5), (7, 7)]
    check_route(sc, idx, None, units, w.beta)
    worst = check_attn(sc, out_host, idx, units)
    print(f"  worst rel L2 vs oracle on {units}: {worst:.2e}", flush=True)
