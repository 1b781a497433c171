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


def test_gather_leaves_invalid_slots_untouched():
    # 20 units x 13 slots = 260 slots: two full work-groups of 128 records
    # and a partial one of 4; some slots name no record (negative or past
    # n_groups), in full work-groups and in the partial one
    print("[gather] invalid slots, ragged last work-group", flush=True)
    B, Hkv, ng, beta, rec = 5, 4, 40, 13, 8 * (64 + 8)
    g = torch.Generator().manual_seed(11)
    src = torch.randint(0, 256, (B, Hkv, ng, rec), dtype=torch.uint8, generator=g).to(DEV)
    idx = torch.randint(0, ng, (B, Hkv, beta), dtype=torch.int32, generator=g)
    idx[0, 0, 3] = -1
    idx[2, 1, 8] = ng
    idx[4, 3, 12] = -7   # slot 259, in the partial work-group
    idx[4, 3, 9] = ng + 5
    staging = torch.full((B, Hkv, beta, rec), 0xAB, dtype=torch.uint8, device=DEV)
    hsq.gather_l3(src.data_ptr(), rec, B, Hkv, ng, idx.to(DEV), staging)
    torch.cuda.synchronize()
    s, x = staging.cpu(), src.cpu()
    for b in range(B):
        for h in range(Hkv):
            for i in range(beta):
                gi = int(idx[b, h, i])
                if 0 <= gi < ng:
                    assert torch.equal(s[b, h, i], x[b, h, gi]), (b, h, i)
                else:
                    assert bool((s[b, h, i] == 0xAB).all()), (b, h, i)


def _gather_case(seed, B=4, Hkv=8, ng=300, beta=64, rec=16 * (128 + 8)):
    g = torch.Generator().manual_seed(seed)
    src = torch.randint(0, 256, (B, Hkv, ng, rec), dtype=torch.uint8, generator=g)
    idx = torch.stack([torch.sort(torch.randperm(ng, generator=g)[:beta])[0]
                       for _ in range(B * Hkv)]).reshape(B, Hkv, beta).to(torch.int32)
    want = torch.stack([src[b, h, idx[b, h].long()] for b in range(B) for h in range(Hkv)])
    return src, idx, want.reshape(B, Hkv, beta, rec)


def test_ordered_gathers_on_two_streams():
    # a chain of four ordered gathers over two streams, issued in turn order
    # (as the pinned-host step issues them): every staging buffer holds its
    # records, and the turn counter ends at the total record count
    print("[gather ordered] 4 gathers, 2 streams", flush=True)
    cases = [_gather_case(20 + k) for k in range(4)]
    arch = hsq.HostArchive(sum(c[0].numel() for c in cases))
    ptrs, off = [], 0
    for src, _, _ in cases:
        arch.host[off:off + src.numel()].copy_(src.reshape(-1))
        ptrs.append(arch.dev_ptr + off)
        off += src.numel()
    turn = torch.zeros(1, dtype=torch.int32, device=DEV)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    stg = [torch.zeros_like(c[2], device=DEV) for c in cases]
    idx = [c[1].to(DEV) for c in cases]
    torch.cuda.synchronize()
    after = 0
    for k, (src, ix, want) in enumerate(cases):
        B, Hkv, ng, rec = src.shape
        with torch.cuda.stream(streams[k % 2]):
            hsq.gather_l3_ordered(ptrs[k], rec, B, Hkv, ng, idx[k], stg[k], turn, after)
        after += B * Hkv * ix.shape[-1]
    torch.cuda.synchronize()
    for k, (_, _, want) in enumerate(cases):
        assert torch.equal(stg[k].cpu(), want), k
    assert int(turn.item()) == after


def test_ordered_gather_goes_ahead_when_its_turn_never_comes():
    # the host passes a turn that no gather will reach: the bounded wait on
    # the device ends (about 2 ms) and the records are copied regardless
    print("[gather ordered] turn never reached: bounded wait", flush=True)
    src, ix, want = _gather_case(31, B=2, Hkv=2, ng=50, beta=9, rec=8 * (64 + 8))
    B, Hkv, ng, rec = src.shape
    dsrc = src.to(DEV)
    turn = torch.zeros(1, dtype=torch.int32, device=DEV)
    staging = torch.zeros_like(want, device=DEV)
    hsq.gather_l3_ordered(dsrc.data_ptr(), rec, B, Hkv, ng, ix.to(DEV), staging, turn, 1 << 30)
    torch.cuda.synchronize()
    assert torch.equal(staging.cpu(), want)
    assert int(turn.item()) == B * Hkv * 9


def test_ordered_pipeline_graph_replays():
    # the pinned-host step as the bench runs it: two micro-batches on two
    # streams, route -> ordered gather -> attend per micro-batch and layer
    # pass, the turn counter zeroed by a fill kernel inside the graph.  Every
    # replay (with eager work between them) equals the eager run bit for
    # bit, and the staged outputs equal the two launches on the archive in
    # device memory.
    w = W.QWEN3_8B_32K.smaller(layers=1, T=8192, batch=4, n_marked=160)
    print(f"[ordered pipeline graph] {w.name} T={w.T} B={w.batch}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    rec, beta = t.rec_bytes, min(w.beta, t.ng)
    arch = hsq.HostArchive(t.l3.numel())
    arch.host.copy_(t.l3.reshape(-1).cpu())
    per_seq = w.hkv * t.ng * rec
    names = ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n")
    mb = []
    for b0, n in ((0, 2), (2, 2)):
        tv = hsq.Tiers(n, w.hkv, w.d, t.n1, t.ng, w.group_n,
                       *[getattr(t, f)[b0:b0 + n] for f in names], t.l3)
        ws = hsq.make_workspace(n, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
        stg = torch.empty((n, w.hkv, beta, rec), dtype=torch.uint8, device=DEV)
        outs = [torch.empty((n, w.hq, w.d), dtype=torch.float32, device=DEV) for _ in range(2)]
        mb.append((b0, n, tv, ws, stg, outs))
    turn = torch.zeros(1, dtype=torch.int32, device=DEV)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]

    def one_step():
        turn.zero_()
        streams[1].wait_stream(streams[0])
        after = 0
        for rep in range(2):  # two passes over the layer, as two layers
            for h, (b0, n, tv, ws, stg, outs) in enumerate(mb):
                with torch.cuda.stream(streams[h]):
                    q = sc.q[b0:b0 + n]
                    hsq.step_route(q, tv, w.beta, sc.dks, sc.cb3, ws)
                    idx = ws.buf[ws.ptr - ws.buf.data_ptr():][:4 * n * w.hkv * beta]
                    hsq.gather_l3_ordered(arch.dev_ptr + b0 * per_seq, rec, n, w.hkv, t.ng,
                                          idx.view(torch.int32).reshape(n, w.hkv, beta), stg,
                                          turn, after)
                    after += n * w.hkv * beta
                    hsq.step_attend(q, tv, w.beta, sc.dks, sc.dvs, sc.cb4, ws, outs[rep],
                                    l3=stg.data_ptr(), l3_staged=True)
        streams[0].wait_stream(streams[1])

    with torch.cuda.stream(streams[0]):
        one_step()
    torch.cuda.synchronize()
    eager = [o.clone() for (_, _, _, _, _, outs) in mb for o in outs]
    assert int(turn.item()) == 2 * w.batch * w.hkv * beta
    ref = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=DEV)
    wsd = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, wsd)
    hsq.step_attend(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, wsd, ref)
    torch.cuda.synchronize()
    for (b0, n, _, _, _, outs) in mb:
        for o in outs:
            assert torch.equal(o, ref[b0:b0 + n])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(streams[0]):
        with torch.cuda.graph(g, stream=streams[0]):
            one_step()
    for r in range(3):
        for (_, _, _, _, stg, outs) in mb:
            stg.zero_()
            for o in outs:
                o.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o for (_, _, _, _, _, outs) in mb for o in outs]
        for k, (a, e) in enumerate(zip(got, eager)):
            assert torch.equal(a, e), f"replay {r}, output {k}"
        assert int(turn.item()) == 2 * w.batch * w.hkv * beta
        del junk


def test_selection_is_left_at_the_start_of_the_workspace():
    w = W.QWEN3_8B_32K.smaller(T=4096, batch=2, n_marked=80)
    print(f"[workspace selection] {w.name} T={w.T} B={w.batch}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    beta = min(w.beta, t.ng)
    ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    idx = torch.empty((w.batch, w.hkv, beta), dtype=torch.int32, device=DEV)
    hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws, idx=idx)
    torch.cuda.synchronize()
    n = w.batch * w.hkv * beta
    head = ws.buf[ws.ptr - ws.buf.data_ptr():][:4 * n].view(torch.int32).reshape(idx.shape)
    assert torch.equal(head, idx)


def test_two_micro_batches_on_two_streams_match_one_batch():
    # as the bench runs the host archive: each half of the batch takes route,
    # gather (selection read in place) and attend on its own stream
    w = W.QWEN3_8B_32K.smaller(T=8192, batch=4, n_marked=160)
    print(f"[micro-batches] {w.name} T={w.T} B={w.batch}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    rec, beta = t.rec_bytes, min(w.beta, t.ng)
    arch = hsq.HostArchive(t.l3.numel())
    arch.host.copy_(t.l3.reshape(-1).cpu())
    lib = hsq.lib()
    # the same two launches over the whole batch, archive in device memory
    out_full = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=DEV)
    ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws)
    hsq.step_attend(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, ws, out_full)
    out = torch.empty_like(out_full)
    nb = w.batch // 2
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    per_seq = w.hkv * t.ng * rec
    keep = []
    torch.cuda.synchronize()
    for h, (b0, n) in enumerate([(0, nb), (nb, w.batch - nb)]):
        tv = hsq.Tiers(n, w.hkv, w.d, t.n1, t.ng, w.group_n,
                       *[getattr(t, f)[b0:b0 + n] for f in
                         ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n")], t.l3)
        wsh = hsq.make_workspace(n, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
        stg = torch.empty((n, w.hkv, beta, rec), dtype=torch.uint8, device=DEV)
        keep += [wsh, stg]
        with torch.cuda.stream(streams[h]):
            q = sc.q[b0:b0 + n]
            hsq.step_route(q, tv, w.beta, sc.dks, sc.cb3, wsh)
            hsq._check(lib.hsq_gather_l3(arch.dev_ptr + b0 * per_seq, rec, n, w.hkv, t.ng,
                                         wsh.ptr, beta, stg.data_ptr(),
                                         streams[h].cuda_stream))
            hsq.step_attend(q, tv, w.beta, sc.dks, sc.dvs, sc.cb4, wsh, out[b0:b0 + n],
                            l3=stg.data_ptr(), l3_staged=True)
    torch.cuda.synchronize()
    # one work-group per unit: a unit's result does not depend on the batch
    # it runs in, nor on where its records were read from
    assert torch.equal(out, out_full)


def test_two_launches_beyond_on_chip_logits_match_the_split_step():
    # G * n_groups above what the two-launch kernels hold on chip: hsq_step_route
    # and hsq_step_attend run as the split step's two halves, with the fetched
    # records staged by a gather in between (read by slot), and give the
    # one-call step's result exactly
    w = W.QWEN3_14B_16K.smaller(T=32768, batch=2, n_marked=328)
    print(f"[split halves] {w.name} T={w.T} B={w.batch}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    assert w.G * t.ng > 12288
    rec, beta = t.rec_bytes, min(w.beta, t.ng)
    ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    out_one, idx_one = hsq.decode_step(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, sc.cb3, ws=ws)
    ws2 = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta, w.group_n, DEV)
    idx = torch.empty((w.batch, w.hkv, beta), dtype=torch.int32, device=DEV)
    staging = torch.empty((w.batch, w.hkv, beta, rec), dtype=torch.uint8, device=DEV)
    out_two = torch.empty_like(out_one)
    hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws2, idx=idx)
    hsq.gather_l3(t.l3.data_ptr(), rec, w.batch, w.hkv, t.ng, idx, staging)
    hsq.step_attend(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, ws2, out_two,
                    l3=staging.data_ptr(), l3_staged=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_one)
    assert torch.equal(out_two, out_one)


def test_host_archive_prerope_step_matches_the_device_archive_prerope_step():
    # the pages' CPU-RAM archive with keys before RoPE: route, gather over
    # PCIe from pinned host memory, the fetched keys rotated to their
    # positions from the staged records, attend; against the pre-RoPE step
    # over the archive in device memory (the same kernels over the same
    # bytes: identical outputs), and sampled units against the oracle's
    # pre-RoPE reading
    from oracle import decode as odec
    w = W.QWEN3_8B_32K.smaller(layers=1, T=8192, batch=4, n_marked=80)
    print(f"[host archive, pre-RoPE] T={w.T} B={w.batch} beta={w.beta}", flush=True)
    sc = Scenario(w)
    t = sc.tiers
    rec, beta = t.rec_bytes, min(w.beta, t.ng)
    gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in sc.plans])).to(DEV)
    arch = hsq.HostArchive(t.l3.numel())
    arch.host.copy_(t.l3.reshape(-1).cpu())
    ws = hsq.Workspace(hsq.prerope_workspace_bytes(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, beta,
                                                   w.group_n), DEV)
    idx = torch.empty((w.batch, w.hkv, beta), dtype=torch.int32, device=DEV)
    staging = torch.empty((w.batch, w.hkv, beta, rec), dtype=torch.uint8, device=DEV)
    out_host = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=DEV)
    hsq.step_route(sc.q, t, w.beta, sc.dks, sc.cb3, ws, idx=idx)
    hsq.gather_l3(arch.dev_ptr, rec, w.batch, w.hkv, t.ng, idx, staging)
    hsq.step_attend_prerope(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, gp, 1e6, ws, out_host,
                            l3=staging.data_ptr(), l3_staged=True)
    out_dev, idx_dev = hsq.decode_step_prerope(sc.q, t, w.beta, sc.dks, sc.dvs, sc.cb4, sc.cb3,
                                               gp, 1e6)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_dev)
    assert torch.equal(out_host, out_dev)
    go = out_host.double().cpu().numpy()
    for (b, h) in [(0, 0), (3, 6)]:
        unit, deq = sc.oracle_unit(b, h)
        want = odec.hsq_attention_unit(sc.q_unit(b, h), deq, unit["l3"], idx[b, h].cpu().numpy(),
                                       w.group_n, w.d, sc.ks[h], sc.vs[h], sc.c4, sc.scale,
                                       group_pos=sc.plans[b][1], rope_base=1e6)
        e = float(np.linalg.norm(go[b, h * w.G:(h + 1) * w.G] - want) / np.linalg.norm(want))
        assert e < 2e-3, f"unit {(b, h)}: rel L2 {e:.3e}"
