"""HSQ tier plan and tier build (oracle, fp64).  TEST INFRASTRUCTURE ONLY.

Source: "Tamarin (HSQ)" summary, section 2, "Three-tier architecture":
* L1 (focal tier, GPU): a small set of tokens kept unsummarised at 4 bits:
  attention sinks, an optional recent window and tokens a learned reader marks
  as important.
* L2 (summary tier, GPU): the remaining tokens are split into groups of size
  N in {8, 16}; each group is compressed to two representative vectors
  (k_hat, v_hat) stored at 3 bits, used as routing keys.
* L3 (archive tier, CPU RAM): the original keys and values of every compressed
  token at 4 bits; the source of truth for content.
And "Key technical components": the reader sends tokens to L1 or L2; the
compressor (a trained pooler) produces the 3-bit routing keys.

Readings taken:
* The trained reader and compressor are not available.  Reader marks are
  input data (positions drawn by the seeded input generator, the same for all
  heads and layers of a sequence); the summary of a group is the mean of its
  N raw vectors (K and V separately), encoded at 3 bits.
* Groups are the non-L1 positions in ascending order, cut into consecutive
  chunks of exactly N; a remainder of fewer than N trailing positions is
  promoted to L1.  L1 lists its positions in ascending order.
* L3 holds only grouped tokens; every position is therefore in exactly one of
  L1 or L3.
* L3 record of one group: [K codes N x d/2][K norms N x fp32][V codes N x d/2]
  [V norms N x fp32], group-contiguous.
"""
import numpy as np

from . import codec


def tier_plan(T, n_sink, n_recent, marked, group_n):
    """Return (l1_positions ascending int64, groups int64 [ng, group_n])."""
    marked = np.asarray(marked, dtype=np.int64).reshape(-1)
    if np.any(marked < 0) or np.any(marked >= T):
        raise ValueError("marked position out of range")
    in_l1 = np.zeros(T, dtype=bool)
    in_l1[: min(n_sink, T)] = True
    if n_recent > 0:
        in_l1[max(T - n_recent, 0):] = True
    in_l1[marked] = True
    rest = np.nonzero(~in_l1)[0]
    ng = rest.size // group_n
    grouped = rest[: ng * group_n]
    remainder = rest[ng * group_n:]
    in_l1[remainder] = True
    l1 = np.nonzero(in_l1)[0].astype(np.int64)
    return l1, grouped.reshape(ng, group_n).astype(np.int64)


def build_unit(k_raw, v_raw, l1_pos, groups, k_signs, v_signs, cb4, cb3):
    """Build the three tiers of one (sequence, kv-head) unit.

    k_raw, v_raw: [T, d] (any float dtype, widened exactly).
    cb4, cb3: (centroids, thresholds) fp32 tables for 4 and 3 bits.
    Returns a dict of numpy arrays:
      l1k, l1k_n, l1v, l1v_n      packed 4-bit codes [n1, d/2], norms [n1]
      l2k, l2k_n, l2v, l2v_n      packed 3-bit codes [ng, 3d/8], norms [ng]
      l3                          records uint8 [ng, group_n * (d + 8)]
      plus the unpacked codes and rotated coordinates y for every encode
      ("*_codes", "*_y") for threshold-distance checks.
    """
    k = codec.to_f64(k_raw)
    v = codec.to_f64(v_raw)
    d = k.shape[1]
    ng, gn = groups.shape
    out = {}
    for name, x, signs in (("k", k, k_signs), ("v", v, v_signs)):
        c1, n1, y1 = codec.encode(x[l1_pos], signs, cb4[1])
        out[f"l1{name}"] = codec.pack(c1, 4)
        out[f"l1{name}_n"] = n1
        out[f"l1{name}_codes"], out[f"l1{name}_y"] = c1, y1
        mean = x[groups.reshape(-1)].reshape(ng, gn, d).mean(axis=1) if ng else np.zeros((0, d))
        c2, n2, y2 = codec.encode(mean, signs, cb3[1])
        out[f"l2{name}"] = codec.pack(c2, 3)
        out[f"l2{name}_n"] = n2
        out[f"l2{name}_codes"], out[f"l2{name}_y"] = c2, y2
        c3, n3, y3 = codec.encode(x[groups.reshape(-1)], signs, cb4[1])
        out[f"l3{name}_packed"] = codec.pack(c3, 4).reshape(ng, gn, d // 2)
        out[f"l3{name}_n"] = n3.reshape(ng, gn)
        out[f"l3{name}_codes"], out[f"l3{name}_y"] = c3, y3
    cbytes = gn * (d // 2)
    rec = np.concatenate(
        [
            out["l3k_packed"].reshape(ng, cbytes),
            out["l3k_n"].astype("<f4").view(np.uint8).reshape(ng, 4 * gn),
            out["l3v_packed"].reshape(ng, cbytes),
            out["l3v_n"].astype("<f4").view(np.uint8).reshape(ng, 4 * gn),
        ],
        axis=1,
    )
    out["l3"] = np.ascontiguousarray(rec, dtype=np.uint8)
    return out


def split_l3_record(rec, group_n, d):
    """Inverse of the record layout: (k_packed, k_norms, v_packed, v_norms)."""
    rec = np.asarray(rec, dtype=np.uint8)
    cb = d // 2
    o = 0
    kp = rec[..., o:o + group_n * cb].reshape(rec.shape[:-1] + (group_n, cb)); o += group_n * cb
    kn = rec[..., o:o + 4 * group_n].copy().view("<f4"); o += 4 * group_n
    vp = rec[..., o:o + group_n * cb].reshape(rec.shape[:-1] + (group_n, cb)); o += group_n * cb
    vn = rec[..., o:o + 4 * group_n].copy().view("<f4")
    return kp, kn, vp, vn
