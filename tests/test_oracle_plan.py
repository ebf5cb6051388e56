"""Pins for oracle.plan: the enumerated work items cover exactly the visible
(row, key) pairs of the prefix-sharing visibility, each exactly once."""
import numpy as np
import pytest

from oracle.brute import visible
from oracle.plan import (FLAT_PREFIX, FLAT_SUFFIX, NONE, coverage_flat, enumerate_flat,
                         enumerate_paged, flat_items_per_head_ub)


def _visible_matrix(p, offs):
    t_n = offs[-1]
    return np.array([[visible(r, c, p, offs) for c in range(t_n)] for r in range(t_n)], dtype=np.int64)


@pytest.mark.parametrize("case", range(40))
def test_flat_items_cover_visible_pairs_exactly_once(case):
    rng = np.random.default_rng(case)
    p = int(rng.integers(0, 20))
    n = int(rng.integers(0, 5))
    lens = [int(x) for x in rng.integers(0, 13, size=n)]
    offs = [p] + list(p + np.cumsum(lens)) if n else [p]
    hkv = int(rng.integers(1, 4))
    bmt = [1, 2, 3, 4, 8, 16][case % 6]
    items = enumerate_flat(p, offs, hkv, bmt)
    assert items.shape[0] == hkv * flat_items_per_head_ub(p, offs[-1], n, bmt)
    cnt = coverage_flat(items, p, offs, hkv)
    vis = _visible_matrix(p, offs)
    for h in range(hkv):
        assert np.array_equal(cnt[h], vis)
    # tiles never cross a segment boundary and never exceed bmt rows
    for it in items:
        kind, h, seg, qb, qe = it[:5]
        if kind == NONE:
            continue
        assert 0 < qe - qb <= bmt
        if kind == FLAT_PREFIX:
            assert qe <= p
        else:
            assert kind == FLAT_SUFFIX and offs[seg] <= qb and qe <= offs[seg + 1]


@pytest.mark.parametrize("prefix_lens,n_splits,split_len", [
    ([100, 0, 64, 17], 3, 48), ([16384] * 2, 8, 2048), ([5], 4, 16), ([0, 0], 1, 64)])
def test_paged_splits_partition_each_prefix(prefix_lens, n_splits, split_len):
    hkv = 3
    items = enumerate_paged(prefix_lens, hkv, 4, n_splits, split_len)
    assert items.shape[0] == len(prefix_lens) * hkv * n_splits
    for b, pl in enumerate(prefix_lens):
        for h in range(hkv):
            cov = np.zeros(pl, dtype=np.int64)
            for it in items:
                if it[2] == b and it[1] == h:
                    assert it[3] == 0 and it[4] == 4
                    cov[it[5]:it[6]] += 1
            if pl <= n_splits * split_len:
                assert np.all(cov == 1)
