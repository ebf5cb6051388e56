"""Pins for the float64 backward oracle of multi-level sharing (CPU only).

``oracle.backward.attn_flat_tree_bwd`` is the expansion route extended down
the segment tree (each segment copies the prefix and its ancestors'
tokens).  It is tied to:

* the one-level oracle ``attn_flat_bwd`` when every parent is the prefix;
* central finite differences of the tree forward oracle's loss <dO, O>;
* PyTorch autograd through dense attention over the flat buffer with the tree
  visibility written as a mask, built here from the rule itself (prefix keys
  to every later row, an ancestor segment's keys to every row of its
  descendants, a segment's own keys causally): no expansion, no hand-written
  backward;
* exact invariants: per kv head, sum_c dV[c] = sum of dO over its query heads
  and rows, and sum_c dK[c] = 0.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attn_flat_tree
from oracle.backward import attn_flat_bwd, attn_flat_tree_bwd
from oracle.decode import decode
from psattn_inputs import BF16

TREES = [
    # P, segment lengths, parents, Hq, Hkv, D
    (3, [2, 3, 2], [-1, 0, 1], 4, 2, 3),
    (2, [3, 0, 2, 2], [-1, 0, 0, 2], 2, 1, 4),
    (0, [2, 3], [-1, 0], 2, 2, 2),
    (4, [1, 2, 2, 1], [-1, -1, 1, 1], 3, 1, 2),
]


def _rand(seed, p, lens, hq, hkv, d):
    rng = np.random.default_rng(seed)
    t = p + sum(lens)
    offs = [p] + [int(x) for x in p + np.cumsum(lens)]
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    do = rng.standard_normal((t, hq, d))
    return q, k, v, do, offs


def _tree_visible(t, p, offs, parents):
    """vis[r, c]: row r sees key c.  Prefix rows: prefix keys c <= r.  A row
    of segment s: every prefix key, every key of a segment on s's parent
    chain, and its own segment's keys c <= r."""
    seg = np.full(t, -1)
    for i in range(len(offs) - 1):
        seg[offs[i]:offs[i + 1]] = i
    vis = np.zeros((t, t), dtype=bool)
    for r in range(t):
        s = seg[r]
        anc = set()
        j = parents[s] if s >= 0 else -1
        while j >= 0:
            anc.add(j)
            j = parents[j]
        for c in range(t):
            if c < p:
                vis[r, c] = c <= r
            elif seg[c] == s:
                vis[r, c] = c <= r
            else:
                vis[r, c] = seg[c] in anc
    return vis


def _torch_grads(q, k, v, do, vis, scale):
    t, hq, _ = q.shape
    g = hq // k.shape[1]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    kr = kt.repeat_interleave(g, dim=1)
    vr = vt.repeat_interleave(g, dim=1)
    z = torch.einsum("rhd,chd->hrc", qt, kr) * scale
    z = z.masked_fill(~torch.from_numpy(vis)[None], float("-inf"))
    o = torch.einsum("hrc,chd->rhd", torch.softmax(z, dim=-1), vr)
    o.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("tree", TREES)
def test_tree_backward_matches_autograd_on_the_mask_route(tree):
    p, lens, par, hq, hkv, d = tree
    q, k, v, do, offs = _rand(21 + len(lens), p, lens, hq, hkv, d)
    scale = 0.8
    dq, dk, dv = attn_flat_tree_bwd(q, k, v, do, p, offs, par, scale, dtype=None)
    tq, tk, tv = _torch_grads(q, k, v, do, _tree_visible(q.shape[0], p, offs, par), scale)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("tree", TREES[:2])
def test_tree_backward_matches_finite_differences(tree):
    p, lens, par, hq, hkv, d = tree
    q, k, v, do, offs = _rand(5 + p, p, lens, hq, hkv, d)
    scale = 0.6
    dq, dk, dv = attn_flat_tree_bwd(q, k, v, do, p, offs, par, scale, dtype=None)

    def loss(q, k, v):
        o, _ = attn_flat_tree(q, k, v, p, offs, par, scale, dtype=None)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p[name], args_m[name] = xp, xm
            fd[i] = (loss(**args_p) - loss(**args_m)) / (2 * eps)
        assert np.max(np.abs(fd - grad)) < 1e-7, name


def test_tree_backward_reduces_to_one_level():
    p, lens, hq, hkv, d = 5, [3, 4, 0, 2], 4, 2, 3
    q, k, v, do, offs = _rand(9, p, lens, hq, hkv, d)
    got = attn_flat_tree_bwd(q, k, v, do, p, offs, [-1] * len(lens), 0.5, dtype=None)
    want = attn_flat_bwd(q, k, v, do, p, offs, 0.5, dtype=None)
    for a, b in zip(got, want):
        assert np.max(np.abs(a - b)) <= 1e-12


def test_tree_backward_invariants_and_restrictions():
    p, lens, par, hq, hkv, d = 6, [4, 3, 5, 2], [-1, 0, 1, 0], 8, 2, 4
    q, k, v, do, offs = _rand(13, p, lens, hq, hkv, d)
    dq, dk, dv = attn_flat_tree_bwd(q, k, v, do, p, offs, par, 0.4, dtype=None)
    g = hq // hkv
    for h in range(hkv):
        assert np.allclose(dv[:, h, :].sum(axis=0), do[:, h * g:(h + 1) * g, :].sum(axis=(0, 1)), atol=1e-12)
        assert np.allclose(dk[:, h, :].sum(axis=0), 0.0, atol=1e-12)
    rows, keys = [0, 7, 12, 19], [1, 6, 9, 16, 18]
    rq, rk, rv = attn_flat_tree_bwd(q, k, v, do, p, offs, par, 0.4, dtype=None, rows=rows, keys=keys)
    for a, b in ((rq, dq[rows]), (rk, dk[keys]), (rv, dv[keys])):
        assert np.max(np.abs(a - b)) <= 1e-13  # the same sums, blocked differently by the matrix products


def test_tree_backward_reads_bf16_storage():
    p, lens, par, hq, hkv, d = 3, [2, 3], [-1, 0], 2, 1, 4
    rng = np.random.default_rng(4)
    t = p + sum(lens)
    bits = lambda shape: (rng.integers(0x3c00, 0x4000, size=shape) | (rng.integers(0, 2, size=shape) << 15)).astype(np.uint16)
    q, k, v, do = bits((t, hq, d)), bits((t, hkv, d)), bits((t, hkv, d)), bits((t, hq, d))
    offs = [p, p + 2, t]
    got = attn_flat_tree_bwd(q, k, v, do, p, offs, par, 0.5, dtype=BF16)
    want = attn_flat_tree_bwd(decode(q, BF16), decode(k, BF16), decode(v, BF16), decode(do, BF16), p, offs, par,
                              0.5, dtype=None)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
