"""Pins of the oracle's paged layout for page sizes other than 16 slots.

The paged pool of the sglang PR #27382 report ("关键源码片段": a ``k_buffer``
addressed through ``kv_indptr`` / ``kv_indices``) fixes no page size.  The
oracle's ``attn_paged`` gathers a request's prefix with one vectorised
division per token; these tests pin it to two other formulations:

* a scalar brute force that walks the request's page list page by page and
  slot by slot until the prefix is consumed (no division), then runs
  per-pair softmax attention with ``math.fsum``;
* repacking the same logical prefix into pools of different page sizes
  (different permutations, partial last pages) leaves the oracle's result
  bitwise unchanged, since only the token order matters.
"""
import math

import numpy as np
import pytest

from oracle.attention import attn_paged
from oracle.decode import decode
from psattn_inputs import BF16, FP8, make_paged


def _brute_paged(inst):
    """Pure-Python scalar reference: page walk, then per-pair softmax."""
    kp = decode(inst.k_pool, inst.kv_dtype)
    vp = decode(inst.v_pool, inst.kv_dtype)
    kx = decode(inst.k_ext, inst.kv_dtype)
    vx = decode(inst.v_ext, inst.kv_dtype)
    q = decode(inst.q, inst.q_dtype)
    g = inst.hq // inst.hkv
    lx = inst.draft_len
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for b in range(inst.batch):
        keys, vals = [], []
        left = int(inst.prefix_lens[b])
        for j in range(int(inst.kv_indptr[b]), int(inst.kv_indptr[b + 1])):
            page = int(inst.kv_indices[j])
            for slot in range(inst.page_size):
                if left == 0:
                    break
                keys.append(kp[page, slot])
                vals.append(vp[page, slot])
                left -= 1
        assert left == 0
        for t in range(lx):
            row = b * lx + t
            ks = keys + [kx[b * lx + j] for j in range(t + 1)]
            vs = vals + [vx[b * lx + j] for j in range(t + 1)]
            for h in range(inst.hq):
                kh = h // g
                z = [inst.sm_scale * inst.k_scale * math.fsum(float(q[row, h, e]) * float(kk[kh, e])
                                                              for e in range(inst.d)) for kk in ks]
                m = max(z)
                w = [math.exp(x - m) for x in z]
                s = math.fsum(w)
                lse[row, h] = m + math.log(s)
                for e in range(inst.d):
                    o[row, h, e] = inst.v_scale * math.fsum(w[i] * float(vv[kh, e]) for i, vv in enumerate(vs)) / s
    return o, lse


def _oracle(inst):
    return attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                      inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, k_scale=inst.k_scale,
                      v_scale=inst.v_scale, q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype, page_size=inst.page_size)


@pytest.mark.parametrize("page_size,kv", [(1, BF16), (3, BF16), (5, FP8), (8, FP8), (16, BF16), (24, BF16)])
def test_paged_oracle_matches_page_walk(page_size, kv):
    inst = make_paged([13, 0, 29], 3, 4, 2, 8, kv_dtype=kv, seed=40 + page_size, num_pages=None,
                      scales=(kv == FP8), page_size=page_size)
    o, lse = _oracle(inst)
    bo, bl = _brute_paged(inst)
    assert np.max(np.abs(o - bo)) <= 1e-12 and np.max(np.abs(lse - bl)) <= 1e-12


def _repack(inst, page_size, seed):
    """The same logical prefix of every request stored in pages of another size."""
    rng = np.random.default_rng(seed)
    logical_k, logical_v = [], []
    for b in range(inst.batch):
        t = np.arange(int(inst.prefix_lens[b]))
        pages = inst.kv_indices[inst.kv_indptr[b] + t // inst.page_size]
        logical_k.append(inst.k_pool[pages, t % inst.page_size])
        logical_v.append(inst.v_pool[pages, t % inst.page_size])
    n_b = [(int(p) + page_size - 1) // page_size for p in inst.prefix_lens]
    n_pages = sum(n_b) + 5
    perm = rng.permutation(n_pages)
    shape = (n_pages, page_size) + inst.k_pool.shape[2:]
    kp = np.zeros(shape, dtype=inst.k_pool.dtype)
    vp = np.zeros(shape, dtype=inst.v_pool.dtype)
    indptr = np.zeros(inst.batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n_b)
    indices = perm[:indptr[-1]].astype(np.int32)
    for b in range(inst.batch):
        t = np.arange(int(inst.prefix_lens[b]))
        pg = indices[indptr[b] + t // page_size]
        kp[pg, t % page_size] = logical_k[b]
        vp[pg, t % page_size] = logical_v[b]
    return kp, vp, indptr, indices


@pytest.mark.parametrize("kv", [BF16, FP8])
def test_paged_oracle_invariant_under_repacking(kv):
    inst = make_paged([70, 33, 1, 0], 4, 8, 2, 16, kv_dtype=kv, seed=44, scales=(kv == FP8))
    o16, l16 = _oracle(inst)
    for ps in (1, 2, 3, 7, 12, 24, 64):
        kp, vp, indptr, indices = _repack(inst, ps, seed=ps)
        o, lse = attn_paged(inst.q, kp, vp, indptr, indices, inst.prefix_lens, inst.k_ext, inst.v_ext,
                            inst.draft_len, inst.sm_scale, k_scale=inst.k_scale, v_scale=inst.v_scale,
                            q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype, page_size=ps)
        assert np.array_equal(o, o16) and np.array_equal(lse, l16), ps


def test_generator_page_size_16_draws_unchanged():
    """page_size=16 passed explicitly gives the same bytes as the default."""
    a = make_paged([40, 17], 3, 4, 2, 16, kv_dtype=BF16, seed=9, num_pages=9)
    b = make_paged([40, 17], 3, 4, 2, 16, kv_dtype=BF16, seed=9, num_pages=9, page_size=16)
    for f in ("q", "k_pool", "v_pool", "kv_indices", "k_ext", "v_ext"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("page_size", [1, 4, 12])
def test_generator_poisons_the_tail_of_a_partial_page(page_size):
    inst = make_paged([37, 8], 2, 2, 1, 8, kv_dtype=BF16, seed=3, num_pages=None, page_size=page_size)
    for b in range(inst.batch):
        pl = int(inst.prefix_lens[b])
        n = int(inst.kv_indptr[b + 1] - inst.kv_indptr[b])
        assert n == (pl + page_size - 1) // page_size
        tail = pl % page_size
        if tail:
            last = inst.kv_indices[inst.kv_indptr[b + 1] - 1]
            assert np.all(inst.k_pool[last, tail:] == 0x7FC0)
