#!/usr/bin/env python
"""Benchmark of the HSQ decode step and TurboQuant codec on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode step of one layer: router scores over the 3-bit L2
summary keys, top-beta selection, and fused attention over L1 + unfetched
summaries + the fetched 4-bit L3 groups, for every (sequence, kv-head) of the
batch.  The headline workload is the Qwen3-14B-shaped layer (40 query / 8 kv
heads, head dim 128, 16K context, batch 64, groups of 8, beta = 128) with the
archive resident in HBM.  The launches cycle through eight independent layer
instances (about 1.55 GB of tiers), so the 256 MB last-level cache cannot
hold the working set, and run from a captured HIP graph, so host launch
latency stays out of the measurement.  W untimed warm-up steps run first;
then a graph of exactly K steps is timed with HIP events on its stream, R
times (R >= 20), and the line reports the median.

Prints one JSON line.  Also reported (same line): the Qwen3-8B 8K layer
(batch 1, a chain of 512 layer instances), the Qwen3-8B 32K workload's 36
layers per step with the archive in HBM and, as a PCIe-inclusive figure,
in pinned host memory (gathered over PCIe); the codec encode/decode rates on
the 32K x 8-head bf16 Student-t workload on buffers cycled over more than the
last-level cache (with the pre-RoPE fetch and the TQ-QKV key path); the
decode-time append at the headline layer's shape; and the CPU oracle on a
sample of the headline workload, run on every host core.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROPE_BASE = 1e6  # the Qwen3 models' rotary base
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "compressed_decode_attention_turboquant_amd", "csrc")
# HBM byte counts of the step kernels, taken with rocprofv3 --pmc (text summary)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_step_kernels_qwen3-14b-16k.txt")
STEP_SOURCES = ("step.hip", "hsq_device.h", "hsq_internal.h")


def step_source_digest():
    """sha256 over the sources the step kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch of `kernel` ("step_kernel", "route",
    "attend") from the committed counter summary, or None when it is missing or
    was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(l.split(":", 1) for l in fh.read().splitlines()
                      if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("step_source_sha256") != step_source_digest():
        return None
    v = kv.get(f"{kernel}_traffic_bytes")
    return float(v) if v else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20, help="layer-steps per timed graph")
    p.add_argument("--warmup", type=int, default=5, help="untimed layer-steps before timing")
    p.add_argument("--reps", type=int, default=20, help="timed graph replays (median reported)")
    p.add_argument("--layers", type=int, default=8, help="independent layer instances cycled")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-codec", action="store_true")
    p.add_argument("--no-cache", action="store_true", help="skip the cache-append timing")
    p.add_argument("--no-host", action="store_true", help="skip the pinned-host archive run")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the Qwen3-8B 8K and 32K (HBM archive) lines")
    p.add_argument("--only-step", action="store_true", help="headline step only (for profiling)")
    p.add_argument("--only-codec", action="store_true", help="codec loop only (for profiling)")
    p.add_argument("--only-host", action="store_true", help="pinned-host archive run only")
    p.add_argument("--host-mb", type=int, default=2,
                   help="micro-batches (and streams) of the pinned-host archive run")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (calibrates HBM byte counters)")
    return p.parse_args()


def algorithmic_bytes(w, n1, ng, beta):
    """Per-unit algorithmic bytes of the two kernels (head dim d, G heads)."""
    d, G, N = w.d, w.G, w.group_n
    cb3, cb4 = 3 * d // 8, d // 2
    route = ng * (cb3 + 4) + (ng - beta) * (cb3 + 4) + G * d * 4   # keys, unfetched values, q
    attend = n1 * 2 * (cb4 + 4) + beta * N * 2 * (cb4 + 4) + G * d * 4  # L1, fetched, out
    return route, attend


class Layer:
    def __init__(self, w, layer, dev, hsq, W, cb, l3=None):
        import torch
        self.k_signs, self.v_signs = W.signs(w.seed, layer, w.hkv, w.d)
        self.dks = torch.from_numpy(self.k_signs.view(np.int32)).to(dev)
        self.dvs = torch.from_numpy(self.v_signs.view(np.int32)).to(dev)
        plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
                 for b in range(w.batch)]
        l1 = torch.from_numpy(np.stack([p[0] for p in plans])).to(dev)
        gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in plans])).to(dev)
        self.gp = gp  # token positions of the grouped tokens (RoPE positions)
        k, v = W.kv(w, layer, dev)
        self.tiers = hsq.build_tiers(k, v, l1, gp, w.group_n, self.dks, self.dvs, cb["thr4"],
                                     cb["thr3"], l3=l3)
        del k, v
        self.q = W.query(w, layer, dev)
        t = self.tiers
        self.beta = min(w.beta, t.ng)
        self.ws = hsq.make_workspace(w.batch, w.hq, w.hkv, w.d, t.n1, t.ng, self.beta, w.group_n,
                                     dev)
        self.out = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=dev)


def codebooks(hsq, d, dev):
    import torch
    c4, t4 = hsq.codebook(d, 4)
    c3, t3 = hsq.codebook(d, 3)
    f = lambda a: torch.from_numpy(a).to(dev)
    return {"cb4": f(c4), "thr4": f(t4), "cb3": f(c3), "thr3": f(t3)}


def time_graph(torch, graph, reps, stream):
    """Total time of `reps` back-to-back replays, bracketed by HIP events
    recorded on the stream the replays run on (ms)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_reps(torch, graph, reps, stream):
    """Each of `reps` replays timed on its own (synchronised on both sides,
    HIP events on the replay stream); returns the list of times in ms.  A
    short spin kernel (torch.cuda._sleep) goes first on the stream, outside
    the timed interval, so that the replay is queued behind the start event
    before the GPU reaches it: the interval holds the replay's kernels, not
    the host's submission latency."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1_000_000)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def capture(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            fn()
    return g


def headline(args, torch, hsq, W):
    dev = "cuda"
    w = W.QWEN3_14B_16K
    cb = codebooks(hsq, w.d, dev)
    layers = [Layer(w, i, dev, hsq, W, cb) for i in range(args.layers)]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    L = len(layers)

    def step(ly):  # one launch: route and attend on the same work-group
        hsq.decode_step(ly.q, ly.tiers, w.beta, ly.dks, ly.dvs, cb["cb4"], cb["cb3"], ws=ly.ws,
                        out=ly.out)

    def route(ly):  # the two-launch form (used with a host archive), for reference
        hsq.step_route(ly.q, ly.tiers, w.beta, ly.dks, cb["cb3"], ly.ws)

    def attend(ly):
        hsq.step_attend(ly.q, ly.tiers, w.beta, ly.dks, ly.dvs, cb["cb4"], ly.ws, ly.out)

    with torch.cuda.stream(stream):
        for ly in layers:  # eager runs first: also leave valid selections in every workspace
            route(ly)
            attend(ly)
            step(ly)
        stream.synchronize()
    K, Wm = max(1, args.steps), max(0, args.warmup)
    # exactly K (timed) and W (warm-up) layer-steps, cycling the instances
    g_steps = capture(torch, stream, lambda: [step(layers[i % L]) for i in range(K)])
    if Wm:
        g_warm = capture(torch, stream, lambda: [step(layers[i % L]) for i in range(Wm)])
        time_graph(torch, g_warm, 1, stream)
    t0 = time.perf_counter()
    reps = time_reps(torch, g_steps, max(20, args.reps), stream)
    wall = time.perf_counter() - t0
    ms_step = float(np.median(reps)) / K
    two = {}
    for name, fn in (("route", route), ("attend", attend)):
        g = capture(torch, stream, lambda fn=fn: [fn(ly) for ly in layers])
        time_graph(torch, g, 2, stream)
        two[name] = float(np.median(time_reps(torch, g, 10, stream))) / L
        del g
    # the same layers read as pre-RoPE archives (the fetched keys rotated to
    # the grouped tokens' positions before attention): three launches
    pre_ms = None
    if not args.only_step:
        pre_ws = hsq.Workspace(hsq.prerope_workspace_bytes(
            w.batch, w.hq, w.hkv, w.d, layers[0].tiers.n1, layers[0].tiers.ng, layers[0].beta,
            w.group_n), dev)

        def pre(ly):
            hsq.decode_step_prerope(ly.q, ly.tiers, w.beta, ly.dks, ly.dvs, cb["cb4"], cb["cb3"],
                                    ly.gp, 1e6, ws=pre_ws, out=ly.out)

        with torch.cuda.stream(stream):
            pre(layers[0])
            stream.synchronize()
        g = capture(torch, stream, lambda: [pre(ly) for ly in layers])
        time_graph(torch, g, 2, stream)
        pre_ms = float(np.median(time_reps(torch, g, 10, stream))) / L
        del g, pre_ws
    # the same layers with TQ-QKV token keys: seeded sketch bits and gammas
    # of every L1 and archive key (their values do not change the work)
    qjl_ms = None
    if not args.only_step:
        t0_ = layers[0].tiers
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        sk = {
            "l1s": torch.randint(0, 256, (w.batch, w.hkv, t0_.n1, w.d // 8), generator=gen,
                                 device=dev, dtype=torch.uint8),
            "l1g": torch.rand((w.batch, w.hkv, t0_.n1), generator=gen, device=dev) * 0.1,
            "l3s": torch.randint(0, 256, (w.batch, w.hkv, t0_.ng, w.group_n, w.d // 8),
                                 generator=gen, device=dev, dtype=torch.uint8),
            "l3g": torch.rand((w.batch, w.hkv, t0_.ng, w.group_n), generator=gen,
                              device=dev) * 0.1,
            "S": torch.from_numpy(W.sketch_matrices(w.seed, 0, w.hkv, w.d)).to(dev),
        }

        def qjl(ly):
            hsq.decode_step_qjl(ly.q, ly.tiers, w.beta, ly.dks, ly.dvs, cb["cb4"], cb["cb3"],
                                sk["l1s"], sk["l1g"], sk["l3s"], sk["l3g"], sk["S"], ws=ly.ws,
                                out=ly.out)

        with torch.cuda.stream(stream):
            qjl(layers[0])
            stream.synchronize()
        g = capture(torch, stream, lambda: [qjl(ly) for ly in layers])
        time_graph(torch, g, 2, stream)
        qjl_ms = float(np.median(time_reps(torch, g, 10, stream))) / L
        del g, sk
    t = layers[0].tiers
    units = w.batch * w.hkv
    rb, ab = algorithmic_bytes(w, t.n1, t.ng, layers[0].beta)
    step_bytes = (rb + ab) * units
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    kb = {"route": rb * units, "attend": ab * units}
    res = {
        "w": w, "ms_step": ms_step, "steps": K, "reps": len(reps), "wall_s": wall,
        "rep_ms_per_step": {"min": min(reps) / K, "median": ms_step, "max": max(reps) / K},
        "value": units * w.T / (ms_step * 1e-3),
        "step_gbs": achieved,
        "kernels": {"step_kernel": {"us": ms_step * 1e3, "bytes": step_bytes, "gbs": achieved}},
        "two_launch": {k: {"us": two[k] * 1e3, "bytes": kb[k],
                           "gbs": kb[k] / (two[k] * 1e-3) / 1e9} for k in two},
        "prerope_step": None if pre_ms is None else {
            "us": pre_ms * 1e3, "vs_step": pre_ms / ms_step, "launches": 3,
            "what": "same layers as pre-RoPE archives: route, fetched-key RoPE pass, attend"},
        "qjl_step": None if qjl_ms is None else {
            "us": qjl_ms * 1e3, "vs_step": qjl_ms / ms_step, "launches": 2,
            "what": "same layers with TQ-QKV token keys (QJL sketches of every L1 and "
                    "archive key): route, attend with the sketch correction"},
        "dominant": "step_kernel", "achieved": achieved, "n1": t.n1, "ng": t.ng,
        "step_bytes": step_bytes,
        "tier_bytes": t.nbytes(),
    }
    del g_steps
    return res, layers


def layer_chain(args, torch, hsq, W, w, n_inst, label):
    """One decode step of each of n_inst layer instances of workload w (archive
    in HBM), launched back to back from one captured graph; the median of R
    replays.  n_inst = w.layers for a model's layers, or a chain of
    independent instances that overflows the last-level cache."""
    dev = "cuda"
    cb = codebooks(hsq, w.d, dev)
    layers = [Layer(w, i, dev, hsq, W, cb) for i in range(n_inst)]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()

    def step(ly):
        hsq.decode_step(ly.q, ly.tiers, w.beta, ly.dks, ly.dvs, cb["cb4"], cb["cb3"], ws=ly.ws,
                        out=ly.out)

    with torch.cuda.stream(stream):
        for ly in layers:
            step(ly)
        stream.synchronize()
    g = capture(torch, stream, lambda: [step(ly) for ly in layers])
    time_graph(torch, g, 2, stream)
    reps = time_reps(torch, g, max(20, args.reps), stream)
    ms = float(np.median(reps))
    t = layers[0].tiers
    units = w.batch * w.hkv
    rb, ab = algorithmic_bytes(w, t.n1, t.ng, layers[0].beta)
    step_bytes = (rb + ab) * units * n_inst
    out = {
        "workload": w.name, "what": label, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
        "context": w.T, "group_n": w.group_n, "beta": w.beta, "n_l1": t.n1, "n_groups": t.ng,
        "archive": "hbm", "layer_launches": n_inst, "reps": len(reps),
        "ms_per_chain": ms, "us_per_layer_step": ms * 1e3 / n_inst,
        "value": units * w.T * n_inst / (ms * 1e-3), "unit": "heads*tokens/s",
        "hbm_bytes_per_chain": step_bytes, "hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "tier_bytes_per_layer": t.nbytes(),
    }
    del g, layers
    torch.cuda.empty_cache()
    return out


# (label, bits, rotation on): TurboQuant at the tier widths, and the ablation's
# 2-bit budget and Plain-KV (rotation off) variants
CODEC_VARIANTS = (("4bit", 4, True), ("3bit", 3, True), ("2bit", 2, True),
                  ("plain_4bit", 4, False), ("plain_2bit", 2, False))


def codec_rates(torch, hsq, W, n_sets=3, reps=20):
    """Encode (K and V, one launch each) and decode of the codec workload.
    The timed graphs cycle n_sets copies of the inputs and outputs (the bf16
    inputs alone are 3 x 134 MB), so the last-level cache cannot serve a
    launch from the previous one; per-launch-pair times are medians."""
    dev = "cuda"
    c = W.CODEC
    k0, v0 = W.codec_inputs(c, dev)
    ks, vs = W.codec_signs(c)
    dks = torch.from_numpy(ks.view(np.int32)).to(dev)
    dvs = torch.from_numpy(vs.view(np.int32)).to(dev)
    stream = torch.cuda.Stream()
    n = c.heads * c.tokens
    ins = [(k0.view(n, c.d), v0.view(n, c.d))] + [
        (k0.view(n, c.d).clone(), v0.view(n, c.d).clone()) for _ in range(n_sets - 1)]
    out = {"sets_cycled": n_sets, "bytes_cycled_in": n_sets * 2 * n * c.d * 2}
    for label, bits, rot in CODEC_VARIANTS:
        cen, thr = (torch.from_numpy(a).to(dev) for a in hsq.codebook(c.d, bits))
        sk, sv = (dks, dvs) if rot else (None, None)
        rk = dict(vecs_per_rot=c.tokens, n_rot=c.heads)
        with torch.cuda.stream(stream):
            codes = [(hsq.encode(ki, bits, sk, thr, **rk), hsq.encode(vi, bits, sv, thr, **rk))
                     for ki, vi in ins]
            decs = [(torch.empty((n, c.d), dtype=torch.bfloat16, device=dev),
                     torch.empty((n, c.d), dtype=torch.bfloat16, device=dev)) for _ in ins]
            stream.synchronize()
        lib = hsq.lib()

        def enc_all():
            for (ki, vi), ((kc, kn), (vc, vn)) in zip(ins, codes):
                for x, (cc, nn), sg in ((ki, (kc, kn), sk), (vi, (vc, vn), sv)):
                    hsq._check(lib.hsq_encode(x.data_ptr(), hsq.HSQ_BF16, n, c.d, bits, None, 1,
                                              sg.data_ptr() if sg is not None else None,
                                              c.tokens, c.heads, thr.data_ptr(), cc.data_ptr(),
                                              nn.data_ptr(), stream.cuda_stream))

        def dec_all():
            for ((kc, kn), (vc, vn)), (dk, dv) in zip(codes, decs):
                for (cc, nn), o, sg in (((kc, kn), dk, sk), ((vc, vn), dv, sv)):
                    hsq._check(lib.hsq_decode(cc.data_ptr(), nn.data_ptr(), n, c.d, bits,
                                              sg.data_ptr() if sg is not None else None,
                                              c.tokens, c.heads, cen.data_ptr(), o.data_ptr(),
                                              hsq.HSQ_BF16, stream.cuda_stream))

        ge = capture(torch, stream, enc_all)
        gd = capture(torch, stream, dec_all)
        time_graph(torch, ge, 2, stream)
        te = float(np.median(time_reps(torch, ge, reps, stream))) / n_sets
        time_graph(torch, gd, 2, stream)
        td = float(np.median(time_reps(torch, gd, reps, stream))) / n_sets
        in_b = 2 * n * c.d * 2
        code_b = 2 * n * (c.d * bits // 8 + 4)
        # relative round-trip error of the bf16 decode (diagnostic, cf. relMSE)
        kf = ins[0][0].float()
        rel = float(((decs[0][0].float() - kf).pow(2).sum(1) / kf.pow(2).sum(1)).mean())
        out[label] = {
            "encode_us": te * 1e3, "encode_in_gbs": in_b / (te * 1e-3) / 1e9,
            "encode_hbm_frac": (in_b + code_b) / (te * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_us": td * 1e3, "decode_out_gbs": in_b / (td * 1e-3) / 1e9,
            "decode_hbm_frac": (in_b + code_b) / (td * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "relmse_k": rel,
        }
        if label == "4bit":
            # pre-RoPE archive fetch: the keys dequantised and rotated to
            # their positions (every head's tokens at 0 .. tokens - 1)
            pos = torch.arange(c.tokens, dtype=torch.int32, device=dev).repeat(c.heads)

            def rope_all():
                for ((kc, kn), _), (dk, _) in zip(codes, decs):
                    hsq._check(lib.hsq_decode_rope(kc.data_ptr(), kn.data_ptr(), n, c.d, bits,
                                                   sk.data_ptr(), c.tokens, c.heads,
                                                   cen.data_ptr(), pos.data_ptr(), ROPE_BASE,
                                                   dk.data_ptr(), hsq.HSQ_BF16,
                                                   stream.cuda_stream))

            gr = capture(torch, stream, rope_all)
            time_graph(torch, gr, 2, stream)
            tr = float(np.median(time_reps(torch, gr, reps, stream))) / n_sets
            out[label].update({
                "rope_decode_k_us": tr * 1e3, "rope_decode_out_gbs": in_b / 2 / (tr * 1e-3) / 1e9,
                "rope_decode_hbm_frac": (in_b + code_b) / 2 / (tr * 1e-3) / 1e9 / HBM_PEAK_GBS})
            del gr, pos
        del codes, decs, ge, gd
    del k0, v0, ins
    torch.cuda.empty_cache()
    return out


def host_archive(torch, hsq, W, reps=5, n_mb=2):
    """Decode step of 36 layers with the L3 archive in pinned host memory.
    Per layer: the route launch, the gather of the selected records over PCIe
    (through the device alias of the pinned archive) into HBM staging, and the
    attend launch.  The batch runs as n_mb micro-batches of its sequences on
    n_mb streams: every sequence still takes its layers in order, the gathers
    take the PCIe link in turn, and one micro-batch's gather overlaps the
    others' route and attend.  One captured graph per decode step."""
    dev = "cuda"
    w = W.QWEN3_8B_32K
    cb = codebooks(hsq, w.d, dev)
    l1, gp = hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, 0), w.group_n)
    n1, ng = l1.shape[0], gp.shape[0]
    rec = w.group_n * (w.d + 8)
    per_layer = w.batch * w.hkv * ng * rec
    arch = hsq.HostArchive(per_layer * w.layers)
    # the tier builder writes each layer's archive straight into pinned host memory
    layers = [_host_layer(w, i, dev, hsq, W, cb, arch.dev_ptr + i * per_layer)
              for i in range(w.layers)]
    torch.cuda.synchronize()
    beta = min(w.beta, ng)
    cuts = [w.batch * k // n_mb for k in range(n_mb + 1)]
    halves = [(cuts[k], cuts[k + 1] - cuts[k]) for k in range(n_mb)]
    lib = hsq.lib()
    per_seq = w.hkv * ng * rec  # archive bytes of one sequence in one layer
    # per half: a workspace per layer (it carries the selection and the summary
    # partials from route to attend; sized for the pre-RoPE variant too), one
    # staging buffer
    mb = []
    for b0, n in halves:
        ws = [hsq.Workspace(hsq.prerope_workspace_bytes(n, w.hq, w.hkv, w.d, n1, ng, beta,
                                                        w.group_n), dev)
              for _ in layers]
        stg = torch.empty((n, w.hkv, beta, rec), dtype=torch.uint8, device=dev)
        tv = [hsq.Tiers(n, w.hkv, w.d, n1, ng, w.group_n,
                        *[getattr(ly.tiers, f)[b0:b0 + n] for f in
                          ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n")],
                        ly.tiers.l3) for ly in layers]
        mb.append((b0, n, ws, stg, tv))
    streams = [torch.cuda.Stream() for _ in halves]
    main = streams[0]
    turn = torch.zeros(1, dtype=torch.int32, device=dev)

    def one_step(prerope=False):
        # The gathers take the link in turn (micro-batch 0, 1, .. of layer 0,
        # then of layer 1, ..), each after the one before it, so that a
        # micro-batch's attend and next route run while another's records
        # cross.  The turn is taken on the device (hsq_gather_l3_ordered): an
        # event wait between two streams costs about 10 us per hand-over.
        turn.zero_()  # a fill kernel, before the streams fork
        for st in streams[1:]:
            st.wait_stream(main)
        after = 0
        for i, ly in enumerate(layers):
            for h, (b0, n, ws, stg, tv) in enumerate(mb):
                st = streams[h]
                with torch.cuda.stream(st):
                    q = ly.q[b0:b0 + n]
                    hsq.step_route(q, tv[i], w.beta, ly.dks, cb["cb3"], ws[i])
                    # the selection is read in place at the start of the workspace
                    hsq._check(lib.hsq_gather_l3_ordered(
                        arch.dev_ptr + i * per_layer + b0 * per_seq, rec, n, w.hkv, ng, ws[i].ptr,
                        beta, stg.data_ptr(), turn.data_ptr(), after & 0xFFFFFFFF,
                        st.cuda_stream))
                    after += n * w.hkv * beta
                    if prerope:  # the archive holds keys before RoPE
                        hsq.step_attend_prerope(q, tv[i], w.beta, ly.dks, ly.dvs, cb["cb4"],
                                                ly.gp[b0:b0 + n], 1e6, ws[i], ly.out[b0:b0 + n],
                                                l3=stg.data_ptr(), l3_staged=True)
                    else:
                        hsq.step_attend(q, tv[i], w.beta, ly.dks, ly.dvs, cb["cb4"], ws[i],
                                        ly.out[b0:b0 + n], l3=stg.data_ptr(), l3_staged=True)
        for st in streams[1:]:
            main.wait_stream(st)

    with torch.cuda.stream(main):
        one_step()
    torch.cuda.synchronize()
    g = capture(torch, main, one_step)
    time_graph(torch, g, 1, main)
    ms = float(np.median(time_reps(torch, g, reps, main)))
    del g
    # the same step over a pre-RoPE archive: the fetched keys are rotated to
    # their positions from the staged records before the attend
    with torch.cuda.stream(main):
        one_step(prerope=True)
    torch.cuda.synchronize()
    g = capture(torch, main, lambda: one_step(prerope=True))
    time_graph(torch, g, 1, main)
    ms_pre = float(np.median(time_reps(torch, g, reps, main)))
    del g
    link_bytes = w.layers * w.batch * w.hkv * beta * rec
    # measured pinned host -> device copy rates, for context: 1 GiB copies, and
    # copies of one layer's gathered bytes (the transfer size of a gather)
    def h2d_rate(nbytes, n_copies=5):
        hbuf = arch.view(0, nbytes)
        dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dbuf.copy_(hbuf, non_blocking=True)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(n_copies):
            dbuf.copy_(hbuf, non_blocking=True)
        c1.record()
        torch.cuda.synchronize()
        return n_copies * nbytes / (c0.elapsed_time(c1) * 1e-3) / 1e9
    h2d = h2d_rate(min(per_layer, 1 << 30))
    h2d_layer = h2d_rate(w.batch * w.hkv * beta * rec, 20)

    # the gather alone, for context: the first micro-batch's records of
    # layer 0 (its selection from the replays above), launched back to back
    def gather_rate(n_launch=20):
        b0, n, ws, stg, _ = mb[0]
        sm = main.cuda_stream
        args_ = (arch.dev_ptr + b0 * per_seq, rec, n, w.hkv, ng, ws[0].ptr, beta, stg.data_ptr(),
                 sm)
        hsq._check(lib.hsq_gather_l3(*args_))
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(main)
        for _ in range(n_launch):
            hsq._check(lib.hsq_gather_l3(*args_))
        c1.record(main)
        torch.cuda.synchronize()
        return n_launch * n * w.hkv * beta * rec / (c0.elapsed_time(c1) * 1e-3) / 1e9
    gather_gbs = gather_rate()
    pcie = link_bytes / (ms * 1e-3) / 1e9
    res = {
        "workload": w.name, "layers": w.layers, "batch": w.batch, "T": w.T, "beta": beta,
        "micro_batches": len(halves),
        "ms_per_step": ms,
        "prerope_ms_per_step": ms_pre,
        "value": w.batch * w.hkv * w.T * w.layers / (ms * 1e-3),
        "unit": "heads*tokens/s",
        "pcie_bytes_per_step": link_bytes,
        "pcie_gbs": pcie,
        "pinned_h2d_copy_gbs": h2d,
        "pinned_h2d_copy_gbs_layer_size": h2d_layer,
        "frac_of_pinned_copy": pcie / h2d,
        "gather_alone_gbs": gather_gbs,
        "archive_gib": per_layer * w.layers / 2 ** 30,
    }
    del layers, arch, mb
    torch.cuda.empty_cache()
    return res


def qjl_rates(torch, hsq, W, reps=20):
    """TQ-QKV key path on the codec workload's keys (32768 tokens x 8 heads,
    d = 128, bf16 Student-t with outlier channels): 4-bit codes plus the 1-bit
    QJL residual sketch, one launch per head (one S per head); then the
    corrected logits of 5 query rows against one head's keys, and the logit
    error of TQ-KV and TQ-QKV against the exact logits on that head (the
    page's Jensen concern: the correction is unbiased but adds variance)."""
    dev = "cuda"
    c = W.CODEC
    k, _ = W.codec_inputs(c, dev)
    ks, _ = W.codec_signs(c)
    kh = k.view(c.heads, c.tokens, c.d)
    rng = np.random.default_rng([c.seed, 7])
    S = [torch.from_numpy(rng.standard_normal((c.d, c.d)).astype(np.float32)).to(dev)
         for _ in range(c.heads)]
    sg = [torch.from_numpy(ks[h].view(np.int32)).to(dev) for h in range(c.heads)]
    cen, thr = (torch.from_numpy(a).to(dev) for a in hsq.codebook(c.d, 4))
    stream = torch.cuda.Stream()
    outs = [None] * c.heads
    with torch.cuda.stream(stream):
        for h in range(c.heads):
            outs[h] = hsq.encode_qjl(kh[h], 4, sg[h], thr, cen, S[h])
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for h in range(c.heads):
                hsq.encode_qjl(kh[h], 4, sg[h], thr, cen, S[h])
    time_graph(torch, g, 3, stream)
    te = time_graph(torch, g, reps, stream) / reps
    q = torch.from_numpy(rng.standard_normal((5, c.d)).astype(np.float32)).to(dev)
    codes, norms, sketch, gamma = outs[0]
    scale = 1.0 / math.sqrt(c.d)
    with torch.cuda.stream(stream):
        lg = hsq.qjl_logits(q, 4, codes, norms, sketch, gamma, sg[0], cen, S[0], scale)
        gl = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gl, stream=stream):
            hsq.qjl_logits(q, 4, codes, norms, sketch, gamma, sg[0], cen, S[0], scale)
    time_graph(torch, gl, 3, stream)
    tl = time_graph(torch, gl, reps, stream) / reps
    # logit errors against the exact bf16 keys: TQ-KV (decode + dot) vs TQ-QKV
    exact = scale * (q.double() @ kh[0].double().T)
    tq = scale * (q.double() @ hsq.decode(codes, norms, 4, c.d, sg[0], cen).double().T)
    e_tq, e_qjl = (tq - exact), (lg.double() - exact)
    n = c.heads * c.tokens
    in_b = n * c.d * 2
    out_b = n * (c.d // 2 + 4 + c.d // 8 + 4)
    res = {"encode_us": te * 1e3, "encode_in_gbs": in_b / (te * 1e-3) / 1e9,
           "encode_hbm_frac": (in_b + out_b) / (te * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "logits_us": tl * 1e3, "logit_rows": 5, "keys": c.tokens,
           "logit_err_mean_tq": float(e_tq.mean()), "logit_err_var_tq": float(e_tq.var()),
           "logit_err_mean_qjl": float(e_qjl.mean()), "logit_err_var_qjl": float(e_qjl.var())}
    del k, kh, outs, g, gl
    return res


def cache_append_rate(torch, hsq, W, cycles=20):
    """Decode-time tier maintenance at the headline layer's shape: one token
    appended per (sequence, kv-head), a group sealed every N appends.  One
    seal cycle (N appends) is captured in a graph and replayed; each replay
    repeats the same slots' work (the same bytes), so the figure is the GPU
    time of N appends, launch overhead excluded."""
    dev = "cuda"
    w = W.QWEN3_14B_16K
    T0 = w.T - w.group_n
    k, v = W.kv(w, 0, dev)  # the layer's raw K / V; the last N tokens are appended
    cb = codebooks(hsq, w.d, dev)
    ks, vs = W.signs(w.seed, 0, w.hkv, w.d)
    dks = torch.from_numpy(ks.view(np.int32)).to(dev)
    dvs = torch.from_numpy(vs.view(np.int32)).to(dev)
    marks = [W.marked(w.smaller(T=T0), b) for b in range(w.batch)]
    c = hsq.Cache.from_prefix(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous(), w.n_sink,
                              w.n_recent, marks, w.group_n, dks, dvs, cb["thr4"], cb["thr3"],
                              w.T // w.group_n + 1)
    new = [(k[:, :, t].contiguous(), v[:, :, t].contiguous()) for t in range(T0, w.T)]
    del k, v
    stream = torch.cuda.Stream()
    state = (c.t, c.n_pending, c.n_groups, [list(p) for p in c.pending])

    def cycle():
        c.t, c.n_pending, c.n_groups = state[0], state[1], state[2]
        c.pending = [list(p) for p in state[3]]
        for kn, vn in new:
            c.append(kn, vn, dks, dvs, cb["thr4"], cb["thr3"])

    with torch.cuda.stream(stream):
        cycle()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cycle()
    torch.cuda.synchronize()
    time_graph(torch, g, 3, stream)
    ms = time_graph(torch, g, cycles, stream) / cycles
    return {"workload": w.name, "batch": w.batch, "kv_heads": w.hkv, "group_n": w.group_n,
            "us_per_append": ms * 1e3 / w.group_n, "us_per_seal_cycle": ms * 1e3,
            "launches_per_cycle": w.group_n}


class _HostLayer:
    pass


def _host_layer(w, layer, dev, hsq, W, cb, l3_dev_ptr):
    import torch
    ly = _HostLayer()
    ly.k_signs, ly.v_signs = W.signs(w.seed, layer, w.hkv, w.d)
    ly.dks = torch.from_numpy(ly.k_signs.view(np.int32)).to(dev)
    ly.dvs = torch.from_numpy(ly.v_signs.view(np.int32)).to(dev)
    plans = [hsq.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
             for b in range(w.batch)]
    l1 = torch.from_numpy(np.stack([p[0] for p in plans])).to(dev)
    gp = torch.from_numpy(np.stack([p[1].reshape(-1) for p in plans])).to(dev)
    k, v = W.kv(w, layer, dev)
    n1, ng = l1.shape[1], gp.shape[1] // w.group_n
    t = hsq.alloc_tiers(w.batch, w.hkv, w.d, n1, ng, w.group_n, dev, l3=torch.empty(0, device=dev))
    lib = hsq.lib()
    hsq._check(lib.hsq_build_tiers(
        k.data_ptr(), v.data_ptr(), hsq.HSQ_BF16, w.batch, w.hkv, w.T, w.d, l1.data_ptr(), n1,
        gp.data_ptr(), ng, w.group_n, ly.dks.data_ptr(), ly.dvs.data_ptr(), cb["thr4"].data_ptr(),
        cb["thr3"].data_ptr(), t.l1k.data_ptr(), t.l1k_n.data_ptr(), t.l1v.data_ptr(),
        t.l1v_n.data_ptr(), t.l2k.data_ptr(), t.l2k_n.data_ptr(), t.l2v.data_ptr(),
        t.l2v_n.data_ptr(), l3_dev_ptr, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    del k, v
    ly.tiers = t
    ly.gp = gp  # the grouped tokens' positions (RoPE positions of a pre-RoPE archive)
    ly.q = W.query(w, layer, dev)
    ly.out = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=dev)
    return ly


# ---- CPU oracle baseline -------------------------------------------------
# The worker pool is forked at start-up, before anything touches the GPU, so
# no child ever inherits a GPU context; each worker runs the oracle on one
# thread (one unit per host core).

def _cpu_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _cpu_build(arg):
    """Oracle tiers of one unit from its raw K and V (compress time, untimed)."""
    from oracle import codebook as ocb
    from oracle import tiers as otiers
    k, v, l1, g, ksg, vsg, d = arg
    u = otiers.build_unit(k, v, l1, g, ksg, vsg, ocb.codebook_f32(d, 4), ocb.codebook_f32(d, 3))
    return {n: u[n] for n in ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n",
                              "l3")}


def _cpu_steps(arg):
    """Oracle decode steps (route + top-beta + attention) of one unit for
    `budget` seconds of wall time; returns (steps, start, end)."""
    from oracle import codebook as ocb
    from oracle import decode as odec
    unit, q, ksg, vsg, gn, d, beta, budget = arg
    c4, c3 = ocb.codebook_f32(d, 4), ocb.codebook_f32(d, 3)
    n, t0 = 0, time.time()
    while True:
        odec.decode_step_unit(q, unit, gn, d, ksg, vsg, c4, c3, beta, 1.0 / math.sqrt(d))
        n += 1
        t1 = time.time()
        if t1 - t0 >= budget:
            return n, t0, t1


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))  # at most the host share of one GPU


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def start_cpu_pool():
    import multiprocessing as mp
    n = cpu_workers()
    return mp.get_context("fork").Pool(processes=n, initializer=_cpu_init), n


def cpu_baseline(torch, W, layers, pool, n_workers, budget_s=10.0):
    """The oracle (fp64 numpy) on n_workers units of the headline workload's
    layer 0, one unit per host core, all running at once for budget_s."""
    w = W.QWEN3_14B_16K
    ly = layers[0]
    sample = [((37 * i) % w.batch, i % w.hkv) for i in range(n_workers)]
    k, v = W.kv(w, 0, "cuda")  # layer 0 of the timed workload, regenerated from its seed
    build_args = []
    for (b, h) in sample:
        from oracle import tiers as otiers
        l1, g = otiers.tier_plan(w.T, w.n_sink, w.n_recent, W.marked(w, b), w.group_n)
        build_args.append((k[b, h].float().cpu().numpy(), v[b, h].float().cpu().numpy(), l1, g,
                           ly.k_signs[h], ly.v_signs[h], w.d))
    del k, v
    torch.cuda.empty_cache()
    units = pool.map(_cpu_build, build_args, chunksize=1)
    del build_args
    run_args = [(u, ly.q[b, h * w.G:(h + 1) * w.G].double().cpu().numpy(), ly.k_signs[h],
                 ly.v_signs[h], w.group_n, w.d, w.beta, budget_s)
                for u, (b, h) in zip(units, sample)]
    res = pool.map(_cpu_steps, run_args, chunksize=1)
    steps = sum(r[0] for r in res)
    el = max(r[2] for r in res) - min(r[1] for r in res)
    return {"value": steps * w.T / el, "unit": "heads*tokens/s", "cores": n_workers,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{steps} (sequence, kv-head) decode steps of the {w.name} workload "
                      f"(route + top-beta + attention over T={w.T}, tiers built beforehand) on "
                      f"{n_workers} units {sample}, one per worker process and core, all "
                      f"running for {el:.1f} s; fp64 numpy oracle"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode step runs on one GPU and bench.py measures one "
                                   "GPU (--gpus must be 1)", "n_gpus": args.gpus}))
        sys.exit(2)
    pool = n_workers = None
    if not (args.only_step or args.only_codec or args.only_host) and not args.no_cpu:
        pool, n_workers = start_cpu_pool()  # before the GPU is touched
    import torch
    from compressed_decode_attention_turboquant_amd import hsq
    from compressed_decode_attention_turboquant_amd import workloads as W
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    hsq.lib()
    if args.only_codec:
        print(json.dumps({"codec": codec_rates(torch, hsq, W, reps=args.reps)}))
        return
    if args.only_host:
        print(json.dumps({"host_archive": host_archive(torch, hsq, W, n_mb=args.host_mb)}))
        return
    res, layers = headline(args, torch, hsq, W)
    w = res["w"]
    k = res["kernels"]
    dom = res["dominant"]
    line = {
        "metric": "HSQ decode-step KV heads·tokens/s + % HBM roofline; codec encode GB/s",
        "value": res["value"],
        "unit": "heads*tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": args.warmup,
        "reps": res["reps"],
        "ms_per_step": res["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (fp16 MFMA operands, fp32 accumulate; 4-bit/3-bit codes)",
        "data": "synthetic (seeded Student-t keys, normal values; no trained weights)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.d, "context": w.T, "group_n": w.group_n, "beta": w.beta,
                   "n_l1": res["n1"], "n_groups": res["ng"], "archive": "hbm",
                   "layer_instances": args.layers, "parallelism": "single-gpu"},
        "timing": {"per_rep_steps": res["steps"], "reps": res["reps"],
                   "ms_per_step": res["rep_ms_per_step"], "statistic": "median over reps"},
        "step_hbm_gbs": res["step_gbs"],
        "step_hbm_frac": res["step_gbs"] / HBM_PEAK_GBS,
        "kernels": k,
        "two_launch": res["two_launch"],
        "prerope_step": res["prerope_step"],
        "qjl_step": res["qjl_step"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": res["achieved"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": res["achieved"] / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dom)},
    }
    print(json.dumps({"progress": "headline", "ms_per_step": res["ms_step"]}), file=sys.stderr,
          flush=True)
    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if not args.only_step and not args.no_configs:
        line["qwen3_8b_8k"] = layer_chain(args, torch, hsq, W, W.QWEN3_8B_8K, 512,
                                          "512 independent layer instances, one launch each")
        print(json.dumps({"progress": "qwen3-8b-8k"}), file=sys.stderr, flush=True)
        line["qwen3_8b_32k_hbm"] = layer_chain(args, torch, hsq, W, W.QWEN3_8B_32K,
                                               W.QWEN3_8B_32K.layers,
                                               "one decode step: 36 layers, archive in HBM")
        print(json.dumps({"progress": "qwen3-8b-32k-hbm"}), file=sys.stderr, flush=True)
    if not args.only_step and not args.no_codec:
        line["codec"] = codec_rates(torch, hsq, W)
        line["qjl"] = qjl_rates(torch, hsq, W)
        print(json.dumps({"progress": "codec"}), file=sys.stderr, flush=True)
    if not args.only_step and not args.no_cache:
        line["cache_append"] = cache_append_rate(torch, hsq, W)
    if not args.only_step and not args.no_host:
        try:
            line["host_archive"] = host_archive(torch, hsq, W, n_mb=args.host_mb)
        except Exception as e:  # reported, never hides the headline
            line["host_archive"] = {"error": repr(e)}
        print(json.dumps({"progress": "host archive"}), file=sys.stderr, flush=True)
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(torch, W, layers, pool, n_workers)
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
