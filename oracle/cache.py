"""Decode-time tier maintenance of one unit (oracle, fp64).  TEST INFRASTRUCTURE ONLY.

Source: "Tamarin (HSQ)" summary, section 2, "Three-tier architecture": L1
holds the attention sinks, an optional recent window and the reader-marked
tokens at 4 bits; the remaining tokens form groups of N, each with a 3-bit
summary in L2 and its 4-bit originals in L3.  The pages describe the tiers of
a context; they do not say how the tiers change as decoding appends tokens.

Reading taken: after every appended token the tiers are exactly the ones the
compress-time build (``tiers.tier_plan`` + ``tiers.build_unit``) gives for the
longer context with the same reader marks.  New tokens are not marked (the
reader is not available), so step by step:

* the new token at position t joins the recent window: it is encoded at 4 bits
  into L1;
* position t - W leaves the window.  A sink or marked position stays in L1 as
  it is; any other becomes a pending token, still in L1 (the build keeps the
  trailing remainder of the grouping in L1);
* when N tokens are pending they are sealed, in position order, as the next
  group: its L3 record holds their 4-bit codes and its L2 summary is the 3-bit
  code of the mean of their raw vectors (summary reading of ``tiers``).

A summary needs the raw vectors of its group, so the raw K and V of the window
and of the pending tokens are kept until their group is sealed.

Parity of this module is pinned against the compress-time build on the longer
context (tests/test_oracle_cache.py), which is pinned on its own.
"""
import numpy as np

from . import codec, tiers


class UnitCache:
    """Tiers of one (sequence, kv-head) unit under decode-time appends.

    Built from a compressed prefix of T0 tokens whose recent window lies past
    the sinks and holds no marked position (T0 >= n_sink + n_recent, marks in
    [n_sink, T0 - n_recent)), so every token that leaves the window is grouped.
    """

    def __init__(self, k_raw, v_raw, n_sink, n_recent, marked, group_n, k_signs, v_signs, cb4,
                 cb3):
        k = codec.to_f64(k_raw)
        v = codec.to_f64(v_raw)
        T0, self.d = k.shape
        marked = np.unique(np.asarray(marked, dtype=np.int64).reshape(-1))
        if n_recent < 1 or T0 < n_sink + n_recent:
            raise ValueError("the prefix must hold the sinks and a full recent window")
        if marked.size and (marked.min() < n_sink or marked.max() >= T0 - n_recent):
            raise ValueError("marks must lie between the sinks and the recent window")
        self.n_sink, self.n_recent, self.gn = n_sink, n_recent, group_n
        self.marked = set(marked.tolist())
        self.ks, self.vs, self.cb4, self.cb3 = k_signs, v_signs, cb4, cb3
        l1, groups = tiers.tier_plan(T0, n_sink, n_recent, marked, group_n)
        self.T = T0
        # L1: position -> (k codes, k norm, v codes, v norm), unpacked codes
        self.l1 = {}
        for p in l1.tolist():
            self.l1[p] = self._encode4(k[p], v[p])
        # groups in order: positions, L2 summary codes/norms, L3 codes/norms
        self.groups = []
        for g in groups:
            self._seal(list(g.tolist()), k[g], v[g])
        # pending = the grouping remainder: L1 positions that are neither
        # sinks, marked nor in the window
        window = set(range(T0 - n_recent, T0))
        self.pending = [p for p in l1.tolist()
                        if p >= n_sink and p not in self.marked and p not in window]
        # raw vectors of the window and of the pending tokens
        self.raw = {p: (k[p].copy(), v[p].copy()) for p in sorted(window | set(self.pending))}

    def _encode4(self, kx, vx):
        kc, kn, _ = codec.encode(kx[None], self.ks, self.cb4[1])
        vc, vn, _ = codec.encode(vx[None], self.vs, self.cb4[1])
        return kc[0], kn[0], vc[0], vn[0]

    def _seal(self, pos, kx, vx):
        """Append a group of N positions with their raw vectors kx, vx [N, d]."""
        kx = np.asarray(kx, dtype=np.float64)
        vx = np.asarray(vx, dtype=np.float64)
        g = {"pos": pos}
        for name, x, signs in (("k", kx, self.ks), ("v", vx, self.vs)):
            c2, n2, _ = codec.encode(x[None].mean(axis=1), signs, self.cb3[1])
            g[f"l2{name}"], g[f"l2{name}_n"] = c2[0], n2[0]
            c3, n3, _ = codec.encode(x, signs, self.cb4[1])
            g[f"l3{name}"], g[f"l3{name}_n"] = c3, n3
        self.groups.append(g)

    def append(self, k_new, v_new):
        """Append the token at position self.T (raw K and V rows of length d)."""
        t = self.T
        kx = codec.to_f64(np.asarray(k_new).reshape(1, -1) if not hasattr(k_new, "detach")
                          else k_new.reshape(1, -1))[0]
        vx = codec.to_f64(np.asarray(v_new).reshape(1, -1) if not hasattr(v_new, "detach")
                          else v_new.reshape(1, -1))[0]
        self.l1[t] = self._encode4(kx, vx)
        self.raw[t] = (kx, vx)
        ev = t - self.n_recent  # leaves the window
        if ev >= self.n_sink and ev not in self.marked:
            self.pending.append(ev)
        else:
            self.raw.pop(ev, None)
        if len(self.pending) == self.gn:
            pos = self.pending
            self._seal(pos, np.stack([self.raw[p][0] for p in pos]),
                       np.stack([self.raw[p][1] for p in pos]))
            for p in pos:
                del self.l1[p]
                del self.raw[p]
            self.pending = []
        self.T = t + 1

    @property
    def n_groups(self):
        return len(self.groups)

    def as_unit(self):
        """The tiers in ``tiers.build_unit``'s layout (L1 ascending by
        position), plus "l1_pos" and "groups" (positions [ng, N])."""
        d, gn = self.d, self.gn
        pos = np.array(sorted(self.l1), dtype=np.int64)
        out = {"l1_pos": pos,
               "groups": np.array([g["pos"] for g in self.groups], dtype=np.int64).reshape(-1, gn)}
        for j, name in ((0, "k"), (2, "v")):
            codes = np.stack([self.l1[p][j] for p in pos]) if pos.size else np.zeros((0, d), np.uint8)
            out[f"l1{name}"] = codec.pack(codes, 4)
            out[f"l1{name}_n"] = np.array([self.l1[p][j + 1] for p in pos], dtype=np.float32)
        ng = self.n_groups
        for name in ("k", "v"):
            c2 = (np.stack([g[f"l2{name}"] for g in self.groups]) if ng
                  else np.zeros((0, d), np.uint8))
            out[f"l2{name}"] = codec.pack(c2, 3)
            out[f"l2{name}_n"] = np.array([g[f"l2{name}_n"] for g in self.groups], dtype=np.float32)
            c3 = (np.concatenate([g[f"l3{name}"] for g in self.groups]) if ng
                  else np.zeros((0, d), np.uint8))
            out[f"l3{name}_packed"] = codec.pack(c3, 4).reshape(ng, gn, d // 2)
            out[f"l3{name}_n"] = (np.stack([g[f"l3{name}_n"] for g in self.groups]) if ng
                                  else np.zeros((0, gn), np.float32))
        cbytes = gn * (d // 2)
        out["l3"] = np.ascontiguousarray(np.concatenate(
            [out["l3k_packed"].reshape(ng, cbytes),
             out["l3k_n"].astype("<f4").view(np.uint8).reshape(ng, 4 * gn),
             out["l3v_packed"].reshape(ng, cbytes),
             out["l3v_n"].astype("<f4").view(np.uint8).reshape(ng, 4 * gn)], axis=1),
            dtype=np.uint8)
        return out
