"""Pins for the dense causal shared-latent MLA oracle (CPU only).

``oracle.mla.mla_dense``: the T query tokens are the last T rows of the
S-row latent cache and token t attends to rows 0 .. S - T + t, one latent row
serving as key and value for every head.  Tied to:

* PyTorch SDPA (float64) with that bottom-right causal mask, the latent rows
  broadcast as the single kv head of all query heads;
* a scalar per-key brute force (math.fsum) with and without sinks;
* the sparse oracle given every visible row as an explicit, shuffled list;
* the sink's closed form: o_sink = o * L / (L + e^sigma),
  lse_sink = ln(L + e^sigma), L = e^lse of the sink-free result.
"""
import math

import numpy as np
import pytest
import torch

from oracle.mla import mla_dense, mla_sparse


def _rand(seed, t, h, d, s):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((t, h, d)), rng.standard_normal((s, d))


@pytest.mark.parametrize("t,s", [(7, 7), (5, 12), (1, 9)])
def test_matches_sdpa_bottom_right_causal(t, s):
    h, d = 4, 6
    q, c = _rand(t + s, t, h, d, s)
    o, lse = mla_dense(q, c, 0.45, dtype=None)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(c)[None].expand(h, s, d)
    mask = torch.from_numpy(np.arange(s)[None, :] <= (s - t + np.arange(t))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=0.45)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    z = np.einsum("thd,sd->ths", q, c) * 0.45
    z = np.where(mask.numpy()[:, None, :], z, -np.inf)
    m = z.max(axis=2)
    assert np.allclose(lse, m + np.log(np.exp(z - m[..., None]).sum(axis=2)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_sink", [False, True])
def test_scalar_brute_force(with_sink):
    t, h, d, s = 3, 2, 3, 5
    q, c = _rand(3, t, h, d, s)
    sink = np.array([0.5, -0.8]) if with_sink else None
    o, lse = mla_dense(q, c, 0.6, sink=sink, dtype=None)
    for i in range(t):
        rows = range(s - t + i + 1)
        for hh in range(h):
            z = [0.6 * math.fsum(q[i, hh, k] * c[r, k] for k in range(d)) for r in rows]
            terms = [math.exp(x) for x in z] + ([math.exp(sink[hh])] if with_sink else [])
            den = math.fsum(terms)
            for k in range(d):
                want = math.fsum(math.exp(z[j]) * c[r, k] for j, r in enumerate(rows)) / den
                assert abs(o[i, hh, k] - want) <= 1e-12
            assert abs(lse[i, hh] - math.log(den)) <= 1e-12


def test_equals_the_sparse_oracle_on_full_lists():
    t, h, d, s = 6, 3, 5, 10
    q, c = _rand(5, t, h, d, s)
    rng = np.random.default_rng(6)
    idx = np.full((t, s), -1)
    for i in range(t):
        idx[i, : s - t + i + 1] = rng.permutation(s - t + i + 1)
    a = mla_dense(q, c, 0.3, dtype=None)
    b = mla_sparse(q, c, idx, 0.3, dtype=None)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=0, atol=1e-12)


def test_sink_closed_form():
    t, h, d, s = 4, 3, 4, 8
    q, c = _rand(7, t, h, d, s)
    sink = np.array([1.0, -2.0, 0.25])
    o0, l0 = mla_dense(q, c, 0.5, dtype=None)
    o1, l1 = mla_dense(q, c, 0.5, sink=sink, dtype=None)
    big_l = np.exp(l0)
    assert np.allclose(o1, o0 * (big_l / (big_l + np.exp(sink)[None, :]))[..., None], rtol=0, atol=1e-12)
    assert np.allclose(l1, np.log(big_l + np.exp(sink)[None, :]), rtol=0, atol=1e-12)


def test_cache_shorter_than_the_queries_is_refused():
    q, c = _rand(8, 5, 2, 3, 4)
    with pytest.raises(ValueError):
        mla_dense(q, c, 0.5, dtype=None)
