"""Thin Python binding of libhsq (ctypes).  Argument marshalling only: every
step of the path runs in the library's kernels; torch provides device memory
and streams.  The names mirror the C ABI in include/hsq.h.
"""
import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhsq.so")

HSQ_F32, HSQ_BF16 = 0, 1
HSQ_AGG_MAX, HSQ_AGG_MEAN = 0, 1

_c = ctypes
_vp, _i, _i64, _f, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t

_SIGNATURES = {
    "hsq_version": ([], _c.c_char_p),
    "hsq_last_error": ([], _c.c_char_p),
    "hsq_codebook": ([_i, _i, _vp, _vp], _i),
    "hsq_tier_plan": ([_i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp], _i),
    "hsq_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i, _i], _sz),
    "hsq_encode": ([_vp, _i, _i64, _i, _i, _vp, _i, _vp, _i64, _i, _vp, _vp, _vp, _vp], _i),
    "hsq_decode": ([_vp, _vp, _i64, _i, _i, _vp, _i64, _i, _vp, _vp, _i, _vp], _i),
    "hsq_decode_rope": ([_vp, _vp, _i64, _i, _i, _vp, _i64, _i, _vp, _vp, _c.c_double, _vp, _i,
                         _vp], _i),
    "hsq_build_tiers": ([_vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _i, _i, _vp, _vp, _vp, _vp,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i),
    "hsq_route_topk": ([_vp, _i, _i, _i, _i, _vp, _vp, _i, _vp, _vp, _f, _i, _i, _vp, _vp, _vp,
                        _sz, _vp], _i),
    "hsq_decode_attn": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i,
                         _vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _f, _f, _vp, _sz, _vp, _vp],
                        _i),
    "hsq_decode_step": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i,
                         _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _sz, _vp, _vp],
                        _i),
    "hsq_prerope_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i, _i], _sz),
    "hsq_decode_step_prerope": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                                 _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp,
                                 _c.c_double, _vp, _vp, _sz, _vp, _vp], _i),
    "hsq_decode_step_qjl": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                             _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _sz, _vp, _vp], _i),
    "hsq_build_sketches": ([_vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _i, _i, _vp, _vp, _vp, _vp,
                            _vp, _vp, _vp, _vp, _vp], _i),
    "hsq_step_attend_prerope": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _i,
                                 _i, _vp, _vp, _vp, _f, _vp, _c.c_double, _vp, _sz, _vp, _vp],
                                _i),
    "hsq_decode_step_static": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                                _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _vp],
                               _i),
    "hsq_step_route": ([_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp,
                        _f, _f, _vp, _vp, _sz, _vp], _i),
    "hsq_step_attend": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _vp,
                         _vp, _vp, _f, _vp, _sz, _vp, _vp], _i),
    "hsq_gather_l3": ([_vp, _sz, _i, _i, _i, _vp, _i, _vp, _vp], _i),
    "hsq_gather_l3_ordered": ([_vp, _sz, _i, _i, _i, _vp, _i, _vp, _vp, _c.c_uint32, _vp], _i),
    "hsq_cache_append": ([_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i64, _i, _i, _i, _i]
                         + [_vp] * 16, _i),
    "hsq_encode_qjl": ([_vp, _i, _i64, _i, _i] + [_vp] * 9, _i),
    "hsq_qjl_logits": ([_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _f, _vp, _vp],
                       _i),
    "hsq_cache_decode_step": ([_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp,
                               _vp, _i, _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _f, _f, _vp,
                               _vp, _sz, _vp, _vp], _i),
}

_lib = None


class HSQError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libhsq error {code}: {msg}")
        self.code = code


def lib():
    """Load libhsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m compressed_decode_attention_turboquant_amd.build`")
        lb = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lb, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lb
    return _lib


def exported_symbols():
    return sorted(_SIGNATURES)


def _check(rc):
    if rc != 0:
        raise HSQError(rc, lib().hsq_last_error().decode())


def _dev(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    if t.dtype == torch.float32:
        return HSQ_F32
    if t.dtype == torch.bfloat16:
        return HSQ_BF16
    raise TypeError("only float32 and bfloat16 are supported")


# ------------------------------------------------------------------ host ----

def codebook(d, bits):
    """(centroids fp32 [2^bits], thresholds fp32 [2^bits-1]) from the library."""
    c = np.zeros(1 << bits, dtype=np.float32)
    t = np.zeros((1 << bits) - 1, dtype=np.float32)
    _check(lib().hsq_codebook(d, bits, c.ctypes.data, t.ctypes.data))
    return c, t


def tier_plan(T, n_sink, n_recent, marked, group_n):
    """(l1 positions int32 [n1], group positions int32 [ng, group_n])."""
    m = np.ascontiguousarray(np.asarray(marked, dtype=np.int32).reshape(-1))
    l1 = np.zeros(T, dtype=np.int32)
    gp = np.zeros(T, dtype=np.int32)
    n1 = ctypes.c_int(0)
    ng = ctypes.c_int(0)
    _check(lib().hsq_tier_plan(T, n_sink, n_recent, m.ctypes.data if m.size else None, m.size,
                               group_n, l1.ctypes.data, ctypes.byref(n1), gp.ctypes.data,
                               ctypes.byref(ng)))
    return l1[: n1.value].copy(), gp[: ng.value * group_n].reshape(ng.value, group_n).copy()


def workspace_bytes(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n):
    return int(lib().hsq_workspace_bytes(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n))


# ---------------------------------------------------------------- device ----

def encode(x, bits, signs, thresholds, vecs_per_rot=None, n_rot=1, row_idx=None, group_n=1,
           n_vec=None):
    """Encode rows of x ([rows, d] fp32/bf16).  Returns (codes u8 [n, bits*d/8], norms f32 [n])."""
    d = x.shape[-1]
    if n_vec is None:
        n_vec = (row_idx.numel() if row_idx is not None else x.numel() // d) // group_n
    if vecs_per_rot is None:
        vecs_per_rot = max(n_vec, 1)
    codes = torch.empty((n_vec, bits * d // 8), dtype=torch.uint8, device=x.device)
    norms = torch.empty((n_vec,), dtype=torch.float32, device=x.device)
    _check(lib().hsq_encode(_dev(x, name="x"), _dtype_code(x), n_vec, d, bits,
                            _dev(row_idx, torch.int64, "row_idx"), group_n,
                            _dev(signs, torch.int32, "signs"), vecs_per_rot, n_rot,
                            _dev(thresholds, torch.float32, "thresholds"), _dev(codes),
                            _dev(norms), _stream()))
    return codes, norms


def decode(codes, norms, bits, d, signs, centroids, vecs_per_rot=None, n_rot=1,
           out_dtype=torch.float32):
    n_vec = norms.numel()
    if vecs_per_rot is None:
        vecs_per_rot = max(n_vec, 1)
    out = torch.empty((n_vec, d), dtype=out_dtype, device=codes.device)
    _check(lib().hsq_decode(_dev(codes, torch.uint8, "codes"), _dev(norms, torch.float32, "norms"),
                            n_vec, d, bits, _dev(signs, torch.int32, "signs"), vecs_per_rot,
                            n_rot, _dev(centroids, torch.float32, "centroids"), _dev(out),
                            _dtype_code(out), _stream()))
    return out


def decode_rope(codes, norms, bits, d, signs, centroids, positions, rope_base,
                vecs_per_rot=None, n_rot=1, out_dtype=torch.float32):
    """hsq_decode_rope: dequantise, then rotate row i to position positions[i]."""
    n_vec = norms.numel()
    if positions.numel() != n_vec:
        raise ValueError("positions must hold one entry per vector")
    if vecs_per_rot is None:
        vecs_per_rot = max(n_vec, 1)
    out = torch.empty((n_vec, d), dtype=out_dtype, device=codes.device)
    _check(lib().hsq_decode_rope(_dev(codes, torch.uint8, "codes"),
                                 _dev(norms, torch.float32, "norms"), n_vec, d, bits,
                                 _dev(signs, torch.int32, "signs"), vecs_per_rot, n_rot,
                                 _dev(centroids, torch.float32, "centroids"),
                                 _dev(positions, torch.int32, "positions"), float(rope_base),
                                 _dev(out), _dtype_code(out), _stream()))
    return out


@dataclass
class Tiers:
    """Device tiers of one layer (layouts as in include/hsq.h)."""
    B: int
    Hkv: int
    d: int
    n1: int
    ng: int
    group_n: int
    l1k: torch.Tensor
    l1k_n: torch.Tensor
    l1v: torch.Tensor
    l1v_n: torch.Tensor
    l2k: torch.Tensor
    l2k_n: torch.Tensor
    l2v: torch.Tensor
    l2v_n: torch.Tensor
    l3: torch.Tensor

    @property
    def rec_bytes(self):
        return self.group_n * (self.d + 8)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.l1k, self.l1k_n, self.l1v, self.l1v_n, self.l2k, self.l2k_n,
                    self.l2v, self.l2v_n, self.l3))

    def batch_slice(self, b0, b1):
        """Tiers of sequences b0 .. b1-1 (views; the arrays are batch-major)."""
        v = {k: getattr(self, k)[b0:b1] for k in
             ("l1k", "l1k_n", "l1v", "l1v_n", "l2k", "l2k_n", "l2v", "l2v_n", "l3")}
        return Tiers(b1 - b0, self.Hkv, self.d, self.n1, self.ng, self.group_n, **v)


def alloc_tiers(B, Hkv, d, n1, ng, group_n, device, l3=None):
    e = lambda *s, dt=torch.uint8: torch.empty(s, dtype=dt, device=device)
    f = torch.float32
    if l3 is None:
        l3 = e(B, Hkv, ng, group_n * (d + 8))
    return Tiers(B, Hkv, d, n1, ng, group_n,
                 e(B, Hkv, n1, d // 2), e(B, Hkv, n1, dt=f), e(B, Hkv, n1, d // 2),
                 e(B, Hkv, n1, dt=f),
                 e(B, Hkv, ng, 3 * d // 8), e(B, Hkv, ng, dt=f), e(B, Hkv, ng, 3 * d // 8),
                 e(B, Hkv, ng, dt=f), l3)


def build_tiers(k, v, l1_pos, group_pos, group_n, k_signs, v_signs, thr4, thr3, l3=None):
    """Build L1/L2/L3 of one layer from raw k, v [B, Hkv, T, d].

    l1_pos int32 [B, n1], group_pos int32 [B, ng*group_n] (device).  l3 may be
    a caller-provided device-visible buffer (e.g. the alias of pinned host memory).
    """
    B, Hkv, T, d = k.shape
    n1 = l1_pos.shape[1]
    ng = group_pos.shape[1] // group_n
    t = alloc_tiers(B, Hkv, d, n1, ng, group_n, k.device, l3)
    _check(lib().hsq_build_tiers(
        _dev(k, name="k"), _dev(v, name="v"), _dtype_code(k), B, Hkv, T, d,
        _dev(l1_pos, torch.int32, "l1_pos"), n1, _dev(group_pos, torch.int32, "group_pos"), ng,
        group_n, _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(thr4, torch.float32, "thr4"), _dev(thr3, torch.float32, "thr3"),
        t.l1k.data_ptr(), t.l1k_n.data_ptr(), t.l1v.data_ptr(), t.l1v_n.data_ptr(),
        t.l2k.data_ptr(), t.l2k_n.data_ptr(), t.l2v.data_ptr(), t.l2v_n.data_ptr(),
        t.l3.data_ptr(), _stream()))
    return t


class Workspace:
    """Device workspace for the decode-step calls (256-byte aligned).  It
    carries the selection and the summary partials from the route launch to
    the attend launch; it needs no initial contents."""

    def __init__(self, nbytes, device):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.buf.data_ptr()) % 256
        self.ptr = self.buf.data_ptr() + off


def prerope_workspace_bytes(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n):
    return int(lib().hsq_prerope_workspace_bytes(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n))


def make_workspace(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n, device):
    n = workspace_bytes(B, Hq, Hkv, d, n_l1, n_groups, beta, group_n)
    if n == 0:
        raise HSQError(-1, "invalid sizes for hsq_workspace_bytes")
    return Workspace(n, device)


def route_topk(q, tiers, k_signs, cb3, beta, scale=None, agg=HSQ_AGG_MAX, ws=None,
               want_scores=False):
    B, Hq, d = q.shape
    Hkv, ng = tiers.Hkv, tiers.ng
    b = min(beta, ng)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ws is None:
        ws = make_workspace(B, Hq, Hkv, d, 0, ng, b, tiers.group_n, q.device)
    idx = torch.empty((B, Hkv, b), dtype=torch.int32, device=q.device)
    scores = torch.empty((B, Hkv, ng), dtype=torch.float32, device=q.device) if want_scores else None
    _check(lib().hsq_route_topk(
        _dev(q, torch.float32, "q"), B, Hq, Hkv, d, _dev(tiers.l2k), _dev(tiers.l2k_n), ng,
        _dev(k_signs, torch.int32, "k_signs"), _dev(cb3, torch.float32, "cb3"), scale, agg,
        beta, idx.data_ptr() if b > 0 else None, _dev(scores), ws.ptr, ws.nbytes, _stream()))
    return idx, scores


def decode_attn(q, tiers, idx, k_signs, v_signs, cb4, cb3, scale=None, summary_bias=0.0,
                ws=None, l3=None, l3_staged=False):
    B, Hq, d = q.shape
    beta = idx.shape[-1] if idx is not None else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ws is None:
        ws = make_workspace(B, Hq, tiers.Hkv, d, tiers.n1, tiers.ng, beta, tiers.group_n,
                            q.device)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    l3p = l3 if l3 is not None else tiers.l3.data_ptr()
    _check(lib().hsq_decode_attn(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, _dev(tiers.l2k), _dev(tiers.l2k_n),
        _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, l3p, tiers.group_n, int(l3_staged),
        _dev(idx, torch.int32, "idx") if beta > 0 else None, beta,
        _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale, summary_bias,
        ws.ptr, ws.nbytes, out.data_ptr(), _stream()))
    return out


def decode_step(q, tiers, beta, k_signs, v_signs, cb4, cb3, scale=None, summary_bias=0.0,
                agg=HSQ_AGG_MAX, ws=None, out=None, idx=None, l3=None):
    """Route + top-beta + attention for one layer.  Returns (out, idx)."""
    B, Hq, d = q.shape
    b = min(beta, tiers.ng)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ws is None:
        ws = make_workspace(B, Hq, tiers.Hkv, d, tiers.n1, tiers.ng, b, tiers.group_n, q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if idx is None and b > 0:
        idx = torch.empty((B, tiers.Hkv, b), dtype=torch.int32, device=q.device)
    l3p = l3 if l3 is not None else tiers.l3.data_ptr()
    _check(lib().hsq_decode_step(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, _dev(tiers.l2k), _dev(tiers.l2k_n),
        _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, l3p, tiers.group_n, beta, agg,
        _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale, summary_bias,
        idx.data_ptr() if idx is not None else None, ws.ptr, ws.nbytes, out.data_ptr(),
        _stream()))
    return out, idx


def decode_step_prerope(q, tiers, beta, k_signs, v_signs, cb4, cb3, group_pos, rope_base,
                        scale=None, summary_bias=0.0, agg=HSQ_AGG_MAX, ws=None, out=None,
                        idx=None):
    """hsq_decode_step_prerope: the decode step over an archive whose keys
    hold no RoPE; the fetched keys are rotated to group_pos [B][ng*group_n]
    with rope_base.  Returns (out, idx)."""
    B, Hq, d = q.shape
    b = min(beta, tiers.ng)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ws is None:
        n = prerope_workspace_bytes(B, Hq, tiers.Hkv, d, tiers.n1, tiers.ng, b, tiers.group_n)
        if n == 0:
            raise HSQError(-1, "invalid sizes for hsq_prerope_workspace_bytes")
        ws = Workspace(n, q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if idx is None and b > 0:
        idx = torch.empty((B, tiers.Hkv, b), dtype=torch.int32, device=q.device)
    _check(lib().hsq_decode_step_prerope(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, _dev(tiers.l2k), _dev(tiers.l2k_n),
        _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, tiers.l3.data_ptr(), tiers.group_n, beta,
        agg, _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale, summary_bias,
        _dev(group_pos, torch.int32, "group_pos") if tiers.ng > 0 else None, float(rope_base),
        idx.data_ptr() if idx is not None else None, ws.ptr, ws.nbytes, out.data_ptr(),
        _stream()))
    return out, idx


def decode_step_qjl(q, tiers, beta, k_signs, v_signs, cb4, cb3, l1_sketch, l1_gamma, l3_sketch,
                    l3_gamma, S, scale=None, summary_bias=0.0, agg=HSQ_AGG_MAX, ws=None,
                    out=None, idx=None):
    """hsq_decode_step_qjl: the decode step with TQ-QKV token keys (sketches
    and gammas of the L1 and archive keys, S [Hkv][d][d]).  Returns (out, idx)."""
    B, Hq, d = q.shape
    b = min(beta, tiers.ng)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if ws is None:
        ws = make_workspace(B, Hq, tiers.Hkv, d, tiers.n1, tiers.ng, b, tiers.group_n, q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if idx is None and b > 0:
        idx = torch.empty((B, tiers.Hkv, b), dtype=torch.int32, device=q.device)
    has1, has3 = tiers.n1 > 0, tiers.ng > 0
    _check(lib().hsq_decode_step_qjl(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, _dev(tiers.l2k), _dev(tiers.l2k_n),
        _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, tiers.l3.data_ptr(), tiers.group_n, beta,
        agg, _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale, summary_bias,
        _dev(l1_sketch, torch.uint8, "l1_sketch") if has1 else None,
        _dev(l1_gamma, torch.float32, "l1_gamma") if has1 else None,
        _dev(l3_sketch, torch.uint8, "l3_sketch") if has3 else None,
        _dev(l3_gamma, torch.float32, "l3_gamma") if has3 else None,
        _dev(S, torch.float32, "S"), idx.data_ptr() if idx is not None else None, ws.ptr,
        ws.nbytes, out.data_ptr(), _stream()))
    return out, idx


def build_sketches(k, l1_pos, group_pos, group_n, k_signs, thr4, cb4, S):
    """hsq_build_sketches: QJL sketches and gammas of the L1 and grouped keys
    of k [B][Hkv][T][d].  Returns (l1_sketch, l1_gamma, l3_sketch, l3_gamma)."""
    B, Hkv, T, d = k.shape
    dtype = HSQ_F32 if k.dtype == torch.float32 else HSQ_BF16
    n1 = l1_pos.shape[1]
    ng = group_pos.shape[1] // group_n
    dev = k.device
    l1s = torch.empty((B, Hkv, n1, d // 8), dtype=torch.uint8, device=dev)
    l1g = torch.empty((B, Hkv, n1), dtype=torch.float32, device=dev)
    l3s = torch.empty((B, Hkv, ng, group_n, d // 8), dtype=torch.uint8, device=dev)
    l3g = torch.empty((B, Hkv, ng, group_n), dtype=torch.float32, device=dev)
    _check(lib().hsq_build_sketches(
        _dev(k, None, "k"), dtype, B, Hkv, T, d, _dev(l1_pos, torch.int32, "l1_pos"), n1,
        _dev(group_pos, torch.int32, "group_pos"), ng, group_n,
        _dev(k_signs, torch.int32, "k_signs"), _dev(thr4, torch.float32, "thr4"),
        _dev(cb4, torch.float32, "cb4"), _dev(S, torch.float32, "S"), l1s.data_ptr(),
        l1g.data_ptr(), l3s.data_ptr(), l3g.data_ptr(), _stream()))
    return l1s, l1g, l3s, l3g


def decode_step_static(q, tiers, beta, k_signs, v_signs, cb4, cb3, scale=None,
                       summary_bias=0.0, agg=HSQ_AGG_MAX, out=None, idx=None):
    """hsq_decode_step_static: the decode step with the library's static
    device scratch as its workspace.  Returns (out, idx)."""
    B, Hq, d = q.shape
    b = min(beta, tiers.ng)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if idx is None and b > 0:
        idx = torch.empty((B, tiers.Hkv, b), dtype=torch.int32, device=q.device)
    _check(lib().hsq_decode_step_static(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, _dev(tiers.l2k), _dev(tiers.l2k_n),
        _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, tiers.l3.data_ptr(), tiers.group_n, beta,
        agg, _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
        _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale, summary_bias,
        idx.data_ptr() if idx is not None else None, out.data_ptr(), _stream()))
    return out, idx


def gather_l3(l3_src_ptr, rec_bytes, B, Hkv, ng, idx, staging):
    beta = idx.shape[-1]
    _check(lib().hsq_gather_l3(l3_src_ptr, rec_bytes, B, Hkv, ng, _dev(idx, torch.int32, "idx"),
                               beta, _dev(staging, torch.uint8, "staging"), _stream()))
    return staging


def gather_l3_ordered(l3_src_ptr, rec_bytes, B, Hkv, ng, idx, staging, turn, after):
    """gather_l3 after the gathers before it in a chain (turn: int32 [1] on
    the device, zeroed before the chain; after: records of those gathers)."""
    beta = idx.shape[-1]
    _check(lib().hsq_gather_l3_ordered(
        l3_src_ptr, rec_bytes, B, Hkv, ng, _dev(idx, torch.int32, "idx"), beta,
        _dev(staging, torch.uint8, "staging"), _dev(turn, torch.int32, "turn"),
        after & 0xFFFFFFFF, _stream()))
    return staging


def step_route(q, tiers, beta, k_signs, cb3, ws, scale=None, summary_bias=0.0, agg=HSQ_AGG_MAX,
               idx=None, stream=None):
    """First launch of the decode step: router, top-beta, summary partials (into ws)."""
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().hsq_step_route(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, tiers.n1, _dev(tiers.l2k),
        _dev(tiers.l2k_n), _dev(tiers.l2v), _dev(tiers.l2v_n), tiers.ng, tiers.group_n, beta, agg,
        _dev(k_signs, torch.int32, "k_signs"), _dev(cb3, torch.float32, "cb3"), scale,
        summary_bias, idx.data_ptr() if idx is not None else None, ws.ptr, ws.nbytes,
        stream if stream is not None else _stream()))


def step_attend(q, tiers, beta, k_signs, v_signs, cb4, ws, out, scale=None, l3=None,
                l3_staged=False, stream=None):
    """Second launch: L1 + fetched-token attention, merge, inverse rotation."""
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    l3p = l3 if l3 is not None else tiers.l3.data_ptr()
    _check(lib().hsq_step_attend(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, tiers.ng, l3p, tiers.group_n,
        int(l3_staged), beta, _dev(k_signs, torch.int32, "k_signs"),
        _dev(v_signs, torch.int32, "v_signs"), _dev(cb4, torch.float32, "cb4"), scale, ws.ptr,
        ws.nbytes, _dev(out, torch.float32, "out"), stream if stream is not None else _stream()))
    return out


def step_attend_prerope(q, tiers, beta, k_signs, v_signs, cb4, group_pos, rope_base, ws, out,
                        scale=None, l3=None, l3_staged=False, stream=None):
    """Second half of the pre-RoPE step (after step_route on ws, a workspace
    of prerope_workspace_bytes): RoPE on the fetched keys, then attention."""
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    l3p = l3 if l3 is not None else tiers.l3.data_ptr()
    _check(lib().hsq_step_attend_prerope(
        _dev(q, torch.float32, "q"), B, Hq, tiers.Hkv, d, _dev(tiers.l1k), _dev(tiers.l1k_n),
        _dev(tiers.l1v), _dev(tiers.l1v_n), tiers.n1, tiers.ng, l3p, tiers.group_n,
        int(l3_staged), beta, _dev(k_signs, torch.int32, "k_signs"),
        _dev(v_signs, torch.int32, "v_signs"), _dev(cb4, torch.float32, "cb4"), scale,
        _dev(group_pos, torch.int32, "group_pos") if tiers.ng > 0 else None, float(rope_base),
        ws.ptr, ws.nbytes, _dev(out, torch.float32, "out"),
        stream if stream is not None else _stream()))
    return out


_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), _vp, _c.c_uint]
        _hip.hipHostGetDevicePointer.restype = _i
    return _hip


class HostArchive:
    """L3 records of one or more layers in pinned host memory (torch
    pin_memory, i.e. hipHostMalloc), with the device alias kernels read over
    PCIe."""

    def __init__(self, nbytes):
        self.host = torch.empty(int(nbytes), dtype=torch.uint8, pin_memory=True)
        dptr = ctypes.c_void_p()
        rc = _hiprt().hipHostGetDevicePointer(ctypes.byref(dptr), self.host.data_ptr(), 0)
        if rc != 0:
            raise HSQError(-3, f"hipHostGetDevicePointer failed ({rc})")
        self.dev_ptr = dptr.value

    def view(self, offset, nbytes):
        return self.host[offset:offset + nbytes]


# ------------------------------------------------- decode-time tier cache ----

class Cache:
    """Tiers of one layer that grow during decoding, in the capacity layout of
    include/hsq.h ("Cache layout").  The arrays have fixed capacities; the
    counts (context length t, pending tokens, groups) are kept here on the
    host and passed to every call.  pos_l1[b] lists the position held by each
    used L1 row of sequence b (the same for every kv-head)."""

    def __init__(self, B, Hkv, d, group_n, n_fix, n_recent, ng_cap, raw_dtype, device):
        self.B, self.Hkv, self.d, self.group_n = B, Hkv, d, group_n
        self.n_fix, self.n_recent, self.ng_cap = n_fix, n_recent, ng_cap
        self.l1_cap = n_fix + n_recent + group_n
        e = lambda *sh, dt=torch.uint8: torch.zeros(sh, dtype=dt, device=device)
        f = torch.float32
        c4, c3 = d // 2, 3 * d // 8
        self.l1k, self.l1v = e(B, Hkv, self.l1_cap, c4), e(B, Hkv, self.l1_cap, c4)
        self.l1k_n, self.l1v_n = e(B, Hkv, self.l1_cap, dt=f), e(B, Hkv, self.l1_cap, dt=f)
        self.raw_k = e(B, Hkv, n_recent + group_n, d, dt=raw_dtype)
        self.raw_v = e(B, Hkv, n_recent + group_n, d, dt=raw_dtype)
        self.l2k, self.l2v = e(B, Hkv, ng_cap, c3), e(B, Hkv, ng_cap, c3)
        self.l2k_n, self.l2v_n = e(B, Hkv, ng_cap, dt=f), e(B, Hkv, ng_cap, dt=f)
        self.l3 = e(B, Hkv, ng_cap, group_n * (d + 8))
        self.t = 0
        self.n_pending = 0
        self.n_groups = 0
        self.fixed = [[] for _ in range(B)]
        self.pending = [[] for _ in range(B)]

    @property
    def n1(self):
        return self.n_fix + self.n_recent + self.n_pending

    def pos_l1(self, b):
        """Positions of the used L1 rows of sequence b, row by row."""
        W, t = self.n_recent, self.t
        ring = [0] * W
        for p in range(t - W, t):
            ring[p % W] = p
        return list(self.fixed[b]) + ring + list(self.pending[b])

    @classmethod
    def from_prefix(cls, k, v, n_sink, n_recent, marked, group_n, k_signs, v_signs, thr4, thr3,
                    ng_cap):
        """Compress-time build of the prefix k, v [B, Hkv, T, d] (hsq_build_tiers)
        placed into a cache.  marked[b]: reader marks of sequence b, all of
        the same count, between the sinks and the window."""
        B, Hkv, T, d = k.shape
        W = n_recent
        if T < n_sink + W:
            raise ValueError("the prefix must hold the sinks and a full recent window")
        rows, fixed, pend, gps = [], [], [], []
        for b in range(B):
            mk = sorted(set(int(x) for x in np.asarray(marked[b]).reshape(-1)))
            if mk and (mk[0] < n_sink or mk[-1] >= T - W):
                raise ValueError("marks must lie between the sinks and the recent window")
            l1, gp_b = tier_plan(T, n_sink, n_recent, mk, group_n)
            gps.append(gp_b.reshape(-1))
            fx = list(range(n_sink)) + mk
            ring = [0] * W
            for p in range(T - W, T):
                ring[p % W] = p
            rest = sorted(set(l1.tolist()) - set(fx) - set(range(T - W, T)))
            fixed.append(fx)
            pend.append(rest)
            rows.append(fx + ring + rest)
        if len({len(r) for r in rows}) != 1:
            raise ValueError("every sequence needs the same number of marks")
        gp = np.stack(gps)
        dev = k.device
        l1_pos = torch.from_numpy(np.array(rows, dtype=np.int32)).to(dev)
        t = build_tiers(k, v, l1_pos, torch.from_numpy(gp.astype(np.int32)).to(dev), group_n,
                        k_signs, v_signs, thr4, thr3)
        n_fix = len(fixed[0])
        c = cls(B, Hkv, d, group_n, n_fix, W, ng_cap, k.dtype, dev)
        if t.ng > ng_cap:
            raise ValueError("ng_cap is below the prefix's group count")
        n1 = t.n1
        for name in ("l1k", "l1k_n", "l1v", "l1v_n"):
            getattr(c, name)[:, :, :n1].copy_(getattr(t, name))
        for name in ("l2k", "l2k_n", "l2v", "l2v_n", "l3"):
            getattr(c, name)[:, :, :t.ng].copy_(getattr(t, name))
        # raw vectors of the window (row p % W) and of the pending tokens
        idx = torch.from_numpy(np.array([r[n_fix:] for r in rows], dtype=np.int64)).to(dev)
        for raw, src in ((c.raw_k, k), (c.raw_v, v)):
            g = torch.gather(src, 2, idx[:, None, :, None].expand(B, Hkv, idx.shape[1], d))
            raw[:, :, :idx.shape[1]].copy_(g)
        c.t, c.n_pending, c.n_groups = T, len(pend[0]), t.ng
        c.fixed, c.pending = fixed, pend
        return c

    def append(self, k_new, v_new, k_signs, v_signs, thr4, thr3):
        """Append one token per (sequence, kv-head): k_new, v_new [B, Hkv, d]."""
        if k_new.dtype != self.raw_k.dtype or v_new.dtype != self.raw_k.dtype:
            raise TypeError("k_new / v_new must have the cache's raw dtype")
        _check(lib().hsq_cache_append(
            _dev(k_new, name="k_new"), _dev(v_new, name="v_new"), _dtype_code(k_new), self.B,
            self.Hkv, self.d, self.group_n, self.n_fix, self.n_recent, self.t, self.n_pending,
            self.n_groups, self.l1_cap, self.ng_cap, _dev(k_signs, torch.int32, "k_signs"),
            _dev(v_signs, torch.int32, "v_signs"), _dev(thr4, torch.float32, "thr4"),
            _dev(thr3, torch.float32, "thr3"), self.l1k.data_ptr(), self.l1k_n.data_ptr(),
            self.l1v.data_ptr(), self.l1v_n.data_ptr(), self.raw_k.data_ptr(),
            self.raw_v.data_ptr(), self.l2k.data_ptr(), self.l2k_n.data_ptr(),
            self.l2v.data_ptr(), self.l2v_n.data_ptr(), self.l3.data_ptr(), _stream()))
        ev = self.t - self.n_recent
        for b in range(self.B):
            self.pending[b].append(ev)
        if self.n_pending + 1 == self.group_n:
            self.n_groups += 1
            self.n_pending = 0
            self.pending = [[] for _ in range(self.B)]
        else:
            self.n_pending += 1
        self.t += 1

    def tiers(self):
        """Dense copies of the used rows as a Tiers (for comparisons)."""
        n1, ng = self.n1, self.n_groups
        return Tiers(self.B, self.Hkv, self.d, n1, ng, self.group_n,
                     *(getattr(self, x)[:, :, :n1].contiguous() for x in
                       ("l1k", "l1k_n", "l1v", "l1v_n")),
                     *(getattr(self, x)[:, :, :ng].contiguous() for x in
                       ("l2k", "l2k_n", "l2v", "l2v_n", "l3")))

    def decode_step(self, q, beta, k_signs, v_signs, cb4, cb3, scale=None, summary_bias=0.0,
                    agg=HSQ_AGG_MAX, ws=None, out=None, idx=None):
        """Route + top-beta + attention over the cache.  Returns (out, idx)."""
        B, Hq, d = q.shape
        ng = self.n_groups
        b = min(beta, ng)
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if ws is None:
            ws = make_workspace(B, Hq, self.Hkv, d, self.n1, ng, b, self.group_n, q.device)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if idx is None and b > 0:
            idx = torch.empty((B, self.Hkv, b), dtype=torch.int32, device=q.device)
        _check(lib().hsq_cache_decode_step(
            _dev(q, torch.float32, "q"), B, Hq, self.Hkv, d, self.l1k.data_ptr(),
            self.l1k_n.data_ptr(), self.l1v.data_ptr(), self.l1v_n.data_ptr(), self.n1,
            self.l1_cap, self.l2k.data_ptr(), self.l2k_n.data_ptr(), self.l2v.data_ptr(),
            self.l2v_n.data_ptr(), ng, self.ng_cap, self.l3.data_ptr(), self.group_n, beta, agg,
            _dev(k_signs, torch.int32, "k_signs"), _dev(v_signs, torch.int32, "v_signs"),
            _dev(cb4, torch.float32, "cb4"), _dev(cb3, torch.float32, "cb3"), scale,
            summary_bias, idx.data_ptr() if idx is not None else None, ws.ptr, ws.nbytes,
            out.data_ptr(), _stream()))
        return out, idx


# -------------------------------------------------------- TQ-QKV key path ----

def encode_qjl(x, bits, signs, thresholds, centroids, S):
    """TurboQuant codes of the rows of x ([n, d], one rotation) plus the 1-bit
    QJL sketch of each residual.  Returns (codes, norms, sketch, gamma)."""
    n, d = x.shape
    dev = x.device
    codes = torch.empty((n, bits * d // 8), dtype=torch.uint8, device=dev)
    norms = torch.empty((n,), dtype=torch.float32, device=dev)
    sketch = torch.empty((n, d // 8), dtype=torch.uint8, device=dev)
    gamma = torch.empty((n,), dtype=torch.float32, device=dev)
    _check(lib().hsq_encode_qjl(_dev(x, name="x"), _dtype_code(x), n, d, bits,
                                _dev(signs, torch.int32, "signs"),
                                _dev(thresholds, torch.float32, "thresholds"),
                                _dev(centroids, torch.float32, "centroids"),
                                _dev(S, torch.float32, "S"), codes.data_ptr(), norms.data_ptr(),
                                sketch.data_ptr(), gamma.data_ptr(), _stream()))
    return codes, norms, sketch, gamma


def qjl_logits(q, bits, codes, norms, sketch, gamma, signs, centroids, S, scale):
    """TQ-QKV logits [n_q, n_keys] of query rows q [n_q, d] (n_q <= 8)."""
    n_q, d = q.shape
    n = norms.numel()
    out = torch.empty((n_q, n), dtype=torch.float32, device=q.device)
    _check(lib().hsq_qjl_logits(_dev(q, torch.float32, "q"), n_q, d, bits,
                                _dev(codes, torch.uint8, "codes"),
                                _dev(norms, torch.float32, "norms"),
                                _dev(sketch, torch.uint8, "sketch"),
                                _dev(gamma, torch.float32, "gamma"), n,
                                _dev(signs, torch.int32, "signs"),
                                _dev(centroids, torch.float32, "centroids"),
                                _dev(S, torch.float32, "S"), scale, out.data_ptr(), _stream()))
    return out
