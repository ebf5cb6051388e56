"""Scalar brute force over the visibility predicate (oracle, test-only).

A second, deliberately different formulation of the same result: no
expansion, no matrices, pure Python loops with ``math.fsum`` on the flat
layout, using the block-causal visibility that PrefixSharing PR #50
("设计简介") proposes in place of the physical copy:

    visible(r, c)  <=>  c <= r  and  (c < P  or  seg(c) == seg(r))

Only for tiny inputs.  Used to pin ``attention.attn_flat``.
"""
import math


def seg_of(pos: int, prefix_len: int, seg_offsets) -> int:
    """-1 for a prefix token, else the index i with o_i <= pos < o_{i+1}."""
    if pos < prefix_len:
        return -1
    for i in range(len(seg_offsets) - 1):
        if seg_offsets[i] <= pos < seg_offsets[i + 1]:
            return i
    raise ValueError("position outside the packed buffer")


def visible(r: int, c: int, prefix_len: int, seg_offsets) -> bool:
    if c > r:
        return False
    if c < prefix_len:
        return True
    return seg_of(c, prefix_len, seg_offsets) == seg_of(r, prefix_len, seg_offsets)


def brute_flat(q, k, v, prefix_len, seg_offsets, sm_scale):
    """q: nested lists / arrays [T][Hq][D] of floats, k/v [T][Hkv][D]."""
    t_n = len(q)
    hq = len(q[0]) if t_n else 0
    hkv = len(k[0]) if t_n else 0
    d = len(q[0][0]) if t_n else 0
    g = hq // hkv if hkv else 1
    offs = [int(x) for x in seg_offsets]
    o = [[[0.0] * d for _ in range(hq)] for _ in range(t_n)]
    lse = [[0.0] * hq for _ in range(t_n)]
    for r in range(t_n):
        cols = [c for c in range(t_n) if visible(r, c, prefix_len, offs)]
        for h in range(hq):
            kh = h // g
            z = [sm_scale * math.fsum(float(q[r][h][e]) * float(k[c][kh][e]) for e in range(d))
                 for c in cols]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            s = math.fsum(w)
            lse[r][h] = m + math.log(s)
            for e in range(d):
                o[r][h][e] = math.fsum(w[j] * float(v[c][kh][e]) for j, c in enumerate(cols)) / s
    return o, lse
