"""Pins for multi-level prefix sharing in the oracle (CPU only).

``attn_flat_tree`` expands every segment to [prefix | ancestors | own] and runs
causal attention.  Tied to the one-level flat oracle (every parent is the
prefix), to plain causal attention over the whole buffer (each segment
continues the previous one, so the buffer is one sequence), and to a scalar
brute force over the tree visibility."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attn_flat, attn_flat_tree, chain_of


def _rand(seed, p, lens, hq, hkv, d):
    rng = np.random.default_rng(seed)
    t = p + sum(lens)
    offs = [p] + [int(x) for x in p + np.cumsum(lens)] if lens else [p]
    return (rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hkv, d)),
            offs)


def test_one_level_tree_is_the_flat_oracle():
    q, k, v, offs = _rand(1, 9, [4, 0, 7, 3], 4, 2, 5)
    a = attn_flat(q, k, v, 9, offs, 0.4, dtype=None)
    b = attn_flat_tree(q, k, v, 9, offs, [-1, -1, -1, -1], 0.4, dtype=None)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_a_chain_of_consecutive_segments_is_one_causal_sequence():
    q, k, v, offs = _rand(2, 6, [5, 3, 8], 4, 2, 6)
    o, lse = attn_flat_tree(q, k, v, 6, offs, [-1, 0, 1], 0.7, dtype=None)
    g = 2
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.7)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("parents", [[-1, 0, 0, 1, -1], [-1, -1, 1, 2, 0]])
def test_tree_matches_scalar_brute_force(parents):
    lens = [3, 2, 4, 1, 2]
    q, k, v, offs = _rand(3, 4, lens, 2, 1, 3)
    o, lse = attn_flat_tree(q, k, v, 4, offs, parents, 0.9, dtype=None)
    seg = np.full(q.shape[0], -1)
    for i in range(len(lens)):
        seg[offs[i]:offs[i + 1]] = i
    for r in range(q.shape[0]):
        anc = set() if seg[r] < 0 else set(chain_of(seg[r], parents))
        keys = [c for c in range(r + 1) if seg[c] < 0 or seg[c] in anc]
        for h in range(2):
            z = [0.9 * math.fsum(float(a) * float(b) for a, b in zip(q[r, h], k[c, 0])) for c in keys]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            s = math.fsum(w)
            want = [math.fsum(wi * float(v[c, 0, dd]) for wi, c in zip(w, keys)) / s for dd in range(3)]
            assert np.allclose(o[r, h], want, rtol=0, atol=1e-12)
            assert abs(lse[r, h] - (m + math.log(s))) < 1e-12
