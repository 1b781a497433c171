"""Seeded synthetic workloads for the HSQ decode path and the TurboQuant codec.

This module only draws inputs; it holds none of the method's arithmetic.  The
same tensors feed the HIP library and the CPU oracle.

Workload shapes follow the pages' Qwen3 settings ("Tamarin (HSQ)" summary,
section 4 "Results": Qwen3 0.6B-14B at up to 32K context; section 2: groups of
N in {8, 16}; "Ablation, Statistical Inference, and Validation for KV-Cache
Compression", "Key contributions" 3: heavy-tailed Student-t regimes).  Trained
weights and real activations are not available, so keys, values and queries
are drawn from the distributions listed per workload below.

Random draws (all reproducible from the workload seed):
  raw K / V / q       torch generator on the target device (Philox on GPU),
                      drawn in fp32, rounded to bf16 (round-to-nearest-even)
                      where the workload is bf16.
  rotation signs      numpy PCG64, one uint32 mask row per (layer, kv-head,
                      K|V); bit i set means coordinate i is negated.
  reader marks        numpy PCG64 per sequence: n_marked positions drawn
                      uniformly without replacement from the positions that
                      are neither sinks nor in the recent window, shared by
                      every head and layer of the sequence.
  Student-t(nu)       z0 / sqrt(sum_{i=1..nu} z_i^2 / nu) with standard normal z,
                      exact for integer nu.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    T: int
    dtype: str          # "f32" or "bf16": dtype of the raw K / V
    n_sink: int
    n_recent: int
    n_marked: int
    group_n: int
    beta: int
    keys: str           # key distribution, see _draw_rows
    values: str
    queries: str
    archive: str        # "hbm" or "host"
    seed: int

    @property
    def G(self):
        return self.hq // self.hkv

    def smaller(self, **kw):
        return replace(self, **kw)


# The five configurations.  Marked counts are round(p * T) for the stated
# fraction p; Tiny states 16 directly.
TINY = Workload("tiny", 1, 1, 2, 2, 64, 512, "f32", 4, 32, 16, 8, 4,
                "normal", "normal", "normal", "hbm", 0)
QWEN3_8B_8K = Workload("qwen3-8b-8k", 1, 1, 32, 8, 128, 8192, "bf16", 4, 64, 164, 16, 32,
                       "rmsnorm_plus_noise", "normal", "rmsnorm_plus_noise", "hbm", 1)
QWEN3_8B_32K = Workload("qwen3-8b-32k-host", 36, 8, 32, 8, 128, 32768, "bf16", 4, 64, 655, 16, 64,
                        "rmsnorm_plus_noise", "normal", "rmsnorm_plus_noise", "host", 2)
QWEN3_14B_16K = Workload("qwen3-14b-16k", 1, 64, 40, 8, 128, 16384, "bf16", 4, 64, 164, 8, 128,
                         "student_t5_rms", "normal", "normal", "hbm", 4)

WORKLOADS = {w.name: w for w in (TINY, QWEN3_8B_8K, QWEN3_8B_32K, QWEN3_14B_16K)}


@dataclass(frozen=True)
class CodecWorkload:
    name: str
    tokens: int
    heads: int
    d: int
    nu: int
    n_outlier: int
    outlier_scale: float
    seed: int


CODEC = CodecWorkload("codec-32k-x8-d128", 32768, 8, 128, 3, 4, 20.0, 3)


def _seed(*parts):
    """Deterministic 63-bit seed from integers/strings."""
    h = 1469598103934665603
    for p in parts:
        for ch in str(p).encode() + b"|":
            h ^= ch
            h = (h * 1099511628211) % (1 << 64)
    return h & ((1 << 63) - 1)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _student_t(shape, nu, g, device):
    z0 = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    acc = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(nu):
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        acc.add_(z * z)
    return z0 / torch.sqrt(acc / nu)


def _draw_rows(kind, shape, g, device):
    """Rows of length shape[-1] drawn from the named distribution (fp32)."""
    if kind == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if kind == "rmsnorm_plus_noise":
        # per-vector RMS-normalised N(0,1) draw plus independent N(0,1) noise
        a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        rms = torch.sqrt(torch.mean(a * a, dim=-1, keepdim=True))
        return a / rms + n
    if kind == "student_t5_rms":
        # Student-t(5) entries, each vector divided by its RMS
        t = _student_t(shape, 5, g, device)
        rms = torch.sqrt(torch.mean(t * t, dim=-1, keepdim=True))
        return t / rms
    raise ValueError(kind)


def _cast(x, dtype):
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def kv(w, layer=0, device="cpu"):
    """Raw keys and values, [B, Hkv, T, d] in the workload dtype."""
    shape = (w.batch, w.hkv, w.T, w.d)
    k = _draw_rows(w.keys, shape, _gen(device, w.seed, layer, "K"), device)
    v = _draw_rows(w.values, shape, _gen(device, w.seed, layer, "V"), device)
    return _cast(k, w.dtype).contiguous(), _cast(v, w.dtype).contiguous()


def query(w, layer=0, device="cpu", step=0):
    """Decode-step queries, [B, Hq, d] fp32."""
    shape = (w.batch, w.hq, w.d)
    return _draw_rows(w.queries, shape, _gen(device, w.seed, layer, "q", step), device).contiguous()


def signs(w_seed, layer, hkv, d):
    """Rotation sign masks: (k_signs, v_signs), uint32 [hkv, d // 32] each."""
    rng = np.random.default_rng([_seed(w_seed, layer, "signs") & 0xFFFFFFFF, layer])
    m = rng.integers(0, 1 << 32, size=(2, hkv, d // 32), dtype=np.uint64).astype(np.uint32)
    return np.ascontiguousarray(m[0]), np.ascontiguousarray(m[1])


def sketch_matrices(w_seed, layer, hkv, d):
    """QJL sketch matrices of the TQ-QKV keys: i.i.d. N(0, 1), fp32
    [hkv, d, d] (row j = sketch direction j of kv-head h)."""
    rng = np.random.default_rng([_seed(w_seed, layer, "qjl-S") & 0xFFFFFFFF, layer])
    return rng.standard_normal((hkv, d, d)).astype(np.float32)


def marked(w, b):
    """Reader-marked positions of sequence b (sorted int64)."""
    lo, hi = w.n_sink, w.T - w.n_recent
    pool = np.arange(max(lo, 0), max(hi, lo))
    if w.n_marked > pool.size:
        raise ValueError("more marks than eligible positions")
    rng = np.random.default_rng([_seed(w.seed, "marks") & 0xFFFFFFFF, b])
    return np.sort(rng.choice(pool, size=w.n_marked, replace=False)).astype(np.int64)


def codec_inputs(c, device="cpu"):
    """Codec workload: (K, V) bf16 [heads, tokens, d] with Student-t(nu) entries
    and n_outlier channels per (head, K|V) scaled by outlier_scale."""
    out = []
    for tag in ("K", "V"):
        g = _gen(device, c.seed, tag)
        x = _student_t((c.heads, c.tokens, c.d), c.nu, g, device)
        rng = np.random.default_rng([_seed(c.seed, tag, "outliers") & 0xFFFFFFFF])
        for h in range(c.heads):
            ch = rng.choice(c.d, size=c.n_outlier, replace=False)
            x[h, :, torch.as_tensor(ch, device=device)] *= c.outlier_scale
        out.append(x.to(torch.bfloat16).contiguous())
    return out[0], out[1]


def codec_signs(c):
    """Codec workload rotation signs: (k_signs, v_signs) uint32 [heads, d // 32]."""
    return signs(c.seed, 0, c.heads, c.d)
