"""HSQ decode step (oracle, fp64).  TEST INFRASTRUCTURE ONLY.

Source: "Tamarin (HSQ)" summary, section 2, "Decode process":
1. Routing: a per-head router scores the L2 summary keys against the current
   query.
2. Fetching: under a routing budget beta the router picks the best-scoring
   groups; their original tokens come from the L3 archive, are dequantised on
   the GPU and rotated back to their semantic positions.
3. Attention runs over the union of L1 tokens, L2 summaries and the recovered
   L3 originals; the summaries of fetched groups are masked so nothing is
   counted twice.

Readings taken:
* Query head h uses kv-head h // G (grouped-query attention, G = Hq / Hkv).
  One selection is made per (sequence, kv-head); its score for group g
  aggregates the scaled logits scale * q_h . k_hat_g of the G query heads of
  that kv-head: max (default) or mean.
* top-beta: the beta largest scores, ties to the lower group index, returned
  in ascending group order; beta is clamped to [0, ng].
* "Rotated back to their semantic positions" is the inverse TurboQuant
  rotation, i.e. dequantisation; the archive holds the same (post-RoPE) keys
  the model caches, so no positional re-rotation happens.  The other reading
  (an archive of keys before RoPE, each fetched key rotated to its token's
  position) is the group_pos variant of hsq_attention_unit.
* Each unfetched summary is one softmax entry with logit scale * q . k_hat_g
  (+ summary_bias, default 0); one joint softmax over all entries;
  scale defaults to 1 / sqrt(d).
* TQ-QKV token keys (the qjl variant of hsq_attention_unit): the 4-bit token
  keys carry QJL residual sketches and their logits the QJL estimate; the
  summaries carry none.
"""
import numpy as np

from . import codec, qjl as qjl_mod, rope, tiers


def dequant_unit(unit, d, group_n, k_signs, v_signs, cb4, cb3):
    """Dequantised tiers of one unit: dict of fp64 arrays."""
    out = {}
    for name, signs in (("k", k_signs), ("v", v_signs)):
        c1 = codec.unpack(unit[f"l1{name}"], 4, d)
        out[f"l1{name}"] = codec.decode(c1, unit[f"l1{name}_n"], signs, cb4[0])
        c2 = codec.unpack(unit[f"l2{name}"], 3, d)
        out[f"l2{name}"] = codec.decode(c2, unit[f"l2{name}_n"], signs, cb3[0])
    return out


def dequant_l3_groups(l3_records, sel, group_n, d, k_signs, v_signs, cb4):
    """Dequantised K and V of the tokens of groups sel: ([len(sel)*N, d], same)."""
    kp, kn, vp, vn = tiers.split_l3_record(l3_records[np.asarray(sel, dtype=np.int64)], group_n, d)
    kc = codec.unpack(kp.reshape(-1, d // 2), 4, d)
    vc = codec.unpack(vp.reshape(-1, d // 2), 4, d)
    return (codec.decode(kc, kn.reshape(-1), k_signs, cb4[0]),
            codec.decode(vc, vn.reshape(-1), v_signs, cb4[0]))


def route_scores(q_heads, l2k_hat, scale, agg="max"):
    """Aggregated router score per group.

    q_heads: [G, d] queries of the kv-head's query heads; l2k_hat: [ng, d].
    Returns (agg scores [ng], per-head logits [G, ng]).
    """
    logits = scale * (np.asarray(q_heads, dtype=np.float64) @ l2k_hat.T)
    if logits.shape[1] == 0:
        return np.zeros(0), logits
    if agg == "max":
        return logits.max(axis=0), logits
    if agg == "mean":
        return logits.mean(axis=0), logits
    raise ValueError("agg must be 'max' or 'mean'")


def top_beta(scores, beta):
    """Indices of the beta largest scores, ties to the lower index, ascending."""
    scores = np.asarray(scores, dtype=np.float64)
    ng = scores.size
    beta = max(0, min(int(beta), ng))
    order = sorted(range(ng), key=lambda g: (-scores[g], g))
    return np.array(sorted(order[:beta]), dtype=np.int64)


def softmax_attention(q, keys, values, scale, bias=None):
    """Textbook single-query softmax attention: sum_e softmax(scale q.k_e + b_e) v_e."""
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1] if values.ndim == 2 else q.shape[0])
    s = scale * (keys @ np.asarray(q, dtype=np.float64))
    if bias is not None:
        s = s + bias
    s = s - s.max()
    w = np.exp(s)
    return (w[:, None] * values).sum(axis=0) / w.sum()


def hsq_attention_unit(q_heads, deq, l3_records, sel, group_n, d, k_signs, v_signs,
                       cb4, scale, summary_bias=0.0, group_pos=None, rope_base=None, qjl=None):
    """HSQ attention for the G query heads of one unit, given the fetched set sel.

    Entries: L1 tokens, summaries of unfetched groups, tokens of fetched groups.
    Pre-RoPE archive (group_pos given, [ng, N] token positions of each group):
    the archive holds keys before the rotary position embedding, so each
    fetched key is dequantised and then rotated to its token's position
    (rope.rope with rope_base) before its logit is formed ("rotated to their
    semantic positions", read as re-applying RoPE); L1 and L2 hold the
    embedded keys as usual.
    TQ-QKV token keys (qjl given: dict of S [m, d] and the unit's sketches as
    qjl.unit_sketches returns them): the logit of every L1 token and every
    fetched token gains the QJL estimate of its key residual's share,
    scale * qjl.correction (Ablation page, "Key contributions" 1: TQ-QKV adds
    the 1-bit residual sketch on the key path); the summaries' logits are
    unchanged.  Returns [G, d].
    """
    ng = deq["l2k"].shape[0]
    sel = np.asarray(sel, dtype=np.int64)
    fetched = np.zeros(ng, dtype=bool)
    fetched[sel] = True
    kf, vf = dequant_l3_groups(l3_records, sel, group_n, d, k_signs, v_signs, cb4)
    if group_pos is not None:
        pos = np.asarray(group_pos, dtype=np.int64)[sel].reshape(-1)
        kf = rope.rope(kf, pos, rope_base)
    keys = np.concatenate([deq["l1k"], deq["l2k"][~fetched], kf], axis=0)
    vals = np.concatenate([deq["l1v"], deq["l2v"][~fetched], vf], axis=0)
    bias = np.concatenate([
        np.zeros(deq["l1k"].shape[0]),
        np.full(int((~fetched).sum()), float(summary_bias)),
        np.zeros(kf.shape[0]),
    ])
    if qjl is None:
        return np.stack([softmax_attention(qh, keys, vals, scale, bias) for qh in q_heads])
    m = np.asarray(qjl["S"]).shape[0]
    c1 = qjl_mod.correction(q_heads, qjl["l1_bits"], qjl["l1_gamma"], k_signs, qjl["S"])
    cf = qjl_mod.correction(q_heads, np.asarray(qjl["l3_bits"])[sel].reshape(-1, m),
                            np.asarray(qjl["l3_gamma"])[sel].reshape(-1), k_signs, qjl["S"])
    n_sum = int((~fetched).sum())
    out = []
    for h, qh in enumerate(q_heads):
        corr = np.concatenate([c1[h], np.zeros(n_sum), cf[h]])
        out.append(softmax_attention(qh, keys, vals, scale, bias + scale * corr))
    return np.stack(out)


def decode_step_unit(q_heads, unit, group_n, d, k_signs, v_signs, cb4, cb3, beta,
                     scale, agg="max", summary_bias=0.0):
    """Route + top-beta + attention for one unit.  Returns (out [G, d], sel, scores)."""
    deq = dequant_unit(unit, d, group_n, k_signs, v_signs, cb4, cb3)
    scores, _ = route_scores(q_heads, deq["l2k"], scale, agg)
    sel = top_beta(scores, beta)
    out = hsq_attention_unit(q_heads, deq, unit["l3"], sel, group_n, d, k_signs, v_signs,
                             cb4, scale, summary_bias)
    return out, sel, scores


def decode_step_from_raw(q_heads, k_raw, v_raw, l1_pos, groups, k_signs, v_signs, cb4, cb3,
                         beta, scale, agg="max", summary_bias=0.0, sel=None):
    """Route + top-beta + attention for one unit straight from its raw K and V.

    The same result as tiers.build_unit followed by decode_step_unit: every
    vector is encoded on its own, so encoding only the vectors the step reads
    (the L1 tokens, the group summaries and the tokens of the fetched groups)
    changes nothing.  sel, if given, is the fetched set the attention uses
    (the oracle's own top-beta is still computed and returned).

    Returns (out [G, d], oracle selection, scores, l2k) with l2k a dict of
    the summary keys' codes, rotated unit vectors y and norms.
    """
    k = codec.to_f64(k_raw)
    v = codec.to_f64(v_raw)
    groups = np.asarray(groups, dtype=np.int64)
    l1_pos = np.asarray(l1_pos, dtype=np.int64)
    ng, gn = groups.shape
    d = k.shape[1]

    def deq(x, signs, cbk, bits):
        c, n, y = codec.encode(x, signs, cbk[1])
        c = codec.unpack(codec.pack(c, bits), bits, d)
        return codec.decode(c, n, signs, cbk[0]), c, y, n

    l1k = deq(k[l1_pos], k_signs, cb4, 4)[0]
    l1v = deq(v[l1_pos], v_signs, cb4, 4)[0]
    if ng:
        mk = k[groups.reshape(-1)].reshape(ng, gn, d).mean(axis=1)
        mv = v[groups.reshape(-1)].reshape(ng, gn, d).mean(axis=1)
    else:
        mk = mv = np.zeros((0, d))
    l2k, l2k_codes, l2k_y, l2k_n = deq(mk, k_signs, cb3, 3)
    l2v = deq(mv, v_signs, cb3, 3)[0]
    scores, _ = route_scores(q_heads, l2k, scale, agg)
    osel = top_beta(scores, beta)
    use = osel if sel is None else np.asarray(sel, dtype=np.int64)
    fetched = np.zeros(ng, dtype=bool)
    fetched[use] = True
    pos = groups[use].reshape(-1)
    kf = deq(k[pos], k_signs, cb4, 4)[0]
    vf = deq(v[pos], v_signs, cb4, 4)[0]
    keys = np.concatenate([l1k, l2k[~fetched], kf], axis=0)
    vals = np.concatenate([l1v, l2v[~fetched], vf], axis=0)
    bias = np.concatenate([np.zeros(l1k.shape[0]),
                           np.full(int((~fetched).sum()), float(summary_bias)),
                           np.zeros(kf.shape[0])])
    out = np.stack([softmax_attention(qh, keys, vals, scale, bias) for qh in q_heads])
    return out, osel, scores, {"codes": l2k_codes, "y": l2k_y, "n": l2k_n}

