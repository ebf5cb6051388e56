"""Pins for the sparse shared-latent MLA oracle (CPU only).

``oracle.mla.mla_sparse`` gathers each token's listed latent rows and runs one
softmax over them (plus an optional sink logit).  Tied to:

* PyTorch SDPA (float64, is_causal) when every token lists all positions up to
  itself: the latent rows are then the keys and values of ordinary causal
  attention with one kv head shared by all query heads;
* a scalar per-entry brute force (math.fsum) on tiny cases with scattered
  padding, duplicate and out-of-range entries, with and without sinks;
* the sink's closed form: o_sink = o * L / (L + e^sigma) and
  lse_sink = ln(L + e^sigma), where L = e^lse of the sink-free result;
* invariance of the result under any permutation of a token's list;
* the empty list: o = 0 and lse = -inf (lse = sigma with a sink).
"""
import math

import numpy as np
import pytest
import torch

from oracle.decode import decode
from oracle.mla import mla_sparse
from psattn_inputs import BF16, make_mla, make_mla_indices


def _rand(seed, t, h, d, s=None):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((t, h, d)), rng.standard_normal((t if s is None else s, d))


def test_full_causal_lists_are_causal_attention():
    t, h, d = 9, 4, 6
    q, c = _rand(1, t, h, d)
    idx = np.full((t, 12), -1)
    for i in range(t):
        idx[i, :i + 1] = np.arange(i + 1)[::-1]
    o, lse = mla_sparse(q, c, idx, 0.4, dtype=None)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(c)[None].expand(h, t, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True, scale=0.4)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    z = np.einsum("thd,sd->ths", q, c) * 0.4
    z = np.where(np.arange(t)[None, None, :] <= np.arange(t)[:, None, None], z, -np.inf)
    m = z.max(axis=2)
    assert np.allclose(lse, m + np.log(np.exp(z - m[..., None]).sum(axis=2)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_sink", [False, True])
def test_scalar_brute_force(with_sink):
    t, h, d, s = 5, 3, 4, 7
    q, c = _rand(2, t, h, d, s)
    idx = np.array([[3, -1, 0, 6, 3],      # a duplicate counts twice
                    [-1, -1, -1, -1, -1],  # no key
                    [9, 2, -5, 1, 4],      # out-of-range entries are skipped
                    [0, 1, 2, 3, 4],
                    [6, -1, -1, 5, -1]])
    sink = np.array([0.3, -1.2, 2.0]) if with_sink else None
    o, lse = mla_sparse(q, c, idx, 0.7, sink=sink, dtype=None)
    for i in range(t):
        keys = [int(x) for x in idx[i] if 0 <= x < s]
        for hh in range(h):
            z = [0.7 * math.fsum(float(a) * float(b) for a, b in zip(q[i, hh], c[k])) for k in keys]
            terms = [math.exp(x) for x in z] + ([math.exp(sink[hh])] if with_sink else [])
            if not terms:
                assert np.all(o[i, hh] == 0) and lse[i, hh] == -np.inf
                continue
            den = math.fsum(terms)
            want = [math.fsum(math.exp(zz) * float(c[k, dd]) for zz, k in zip(z, keys)) / den for dd in range(d)]
            assert np.allclose(o[i, hh], want, rtol=0, atol=1e-13)
            assert abs(lse[i, hh] - math.log(den)) < 1e-13


def test_sink_closed_form():
    t, h, d = 6, 4, 5
    q, c = _rand(3, t, h, d)
    idx = make_mla_indices(t, 4, seed=3)
    sink = np.array([0.5, -3.0, 4.0, 1.0])
    o0, l0 = mla_sparse(q, c, idx, 0.9, dtype=None)
    o1, l1 = mla_sparse(q, c, idx, 0.9, sink=sink, dtype=None)
    big_l = np.exp(l0)
    frac = big_l / (big_l + np.exp(sink)[None, :])
    assert np.allclose(o1, o0 * frac[..., None], rtol=0, atol=1e-13)
    assert np.allclose(l1, np.logaddexp(l0, sink[None, :]), rtol=0, atol=1e-13)


def test_list_order_does_not_matter():
    t, h, d = 8, 2, 4
    q, c = _rand(4, t, h, d)
    idx = make_mla_indices(t, 5, seed=4, scatter_pad=True)
    rng = np.random.default_rng(0)
    perm = np.stack([rng.permutation(row) for row in idx])
    a = mla_sparse(q, c, idx, 0.5, dtype=None)
    b = mla_sparse(q, c, perm, 0.5, dtype=None)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-13) and np.allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_empty_lists():
    q, c = _rand(5, 2, 3, 4)
    idx = np.full((2, 3), -1)
    o, lse = mla_sparse(q, c, idx, 1.0, dtype=None)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    o, lse = mla_sparse(q, c, idx, 1.0, sink=np.array([0.1, 0.2, 0.3]), dtype=None)
    assert np.all(o == 0) and np.allclose(lse, [[0.1, 0.2, 0.3]] * 2, rtol=0, atol=0)


def test_reads_bf16_storage_and_token_subsets():
    inst = make_mla(12, 4, 16, 6, seed=7, sink=True)
    full = mla_sparse(inst.q, inst.ckv, inst.indices, inst.sm_scale, sink=inst.sink, dtype=BF16)
    ref = mla_sparse(decode(inst.q, BF16), decode(inst.ckv, BF16), inst.indices, inst.sm_scale,
                     sink=inst.sink, dtype=None)
    assert all(np.array_equal(a, b) for a, b in zip(full, ref))
    sub = mla_sparse(inst.q, inst.ckv, inst.indices, inst.sm_scale, sink=inst.sink, dtype=BF16, tokens=[0, 5, 11])
    assert np.array_equal(sub[0], full[0][[0, 5, 11]]) and np.array_equal(sub[1], full[1][[0, 5, 11]])


def test_index_lists_are_causal_and_distinct():
    idx = make_mla_indices(300, 64, seed=8)
    for t in range(300):
        row = idx[t]
        keys = row[row >= 0]
        assert keys.size == min(t + 1, 64)
        assert np.unique(keys).size == keys.size and keys.max() <= t
        assert np.all(row[keys.size:] == -1)  # padding at the end
