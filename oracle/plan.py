"""Enumeration of the library's tile work items (oracle, test-only).

PrefixSharing PR #50 ("设计简介", "关键变更" §2) proposes to express the
prefix-sharing visibility as rectangles plus causal blocks instead of a full
mask.  The library's planner turns that into one work item per workgroup;
this module writes the same list down independently, in the canonical order
documented below, so that the device planner can be compared bit-exactly, and
``coverage`` checks from the items alone that every visible (row, key) pair is
covered exactly once and no invisible pair is covered.

Record layout (10 int32 per item):
    kind, h_kv, seg, q_begin, q_end, r0_begin, r0_end, r1_begin, r1_end, split
kind: 0 none (an idle workgroup), 1 flat prefix tile, 2 flat suffix tile,
      3 paged split.
A row r of an item sees keys (r0 U r1) intersected with [0, r] (flat), or all of
r0 (paged: every prefix key precedes every draft row; the draft block itself is
folded in by the combine stage).

Flat order: workgroup b handles kv head b % Hkv and per-head item j = b // Hkv.
Per head, suffix tiles come first (segments in order, each segment's tiles
from the last to the first), then prefix tiles from the last to the first;
the remaining slots of the launch (an upper bound the host computes without
reading device memory: ceil(P/BMt) + floor((T-P)/BMt) + N) are idle.

Paged order: workgroup b handles split b % n_splits, kv head
(b // n_splits) % Hkv, request b // (n_splits * Hkv).
"""
from __future__ import annotations

import numpy as np

NONE, FLAT_PREFIX, FLAT_SUFFIX, PAGED_SPLIT = 0, 1, 2, 3
FIELDS = 10


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def flat_items_per_head_ub(prefix_len: int, total: int, n_seg: int, bmt: int) -> int:
    return _cdiv(prefix_len, bmt) + (total - prefix_len) // bmt + n_seg


def enumerate_flat(prefix_len: int, seg_offsets, hkv: int, bmt: int) -> np.ndarray:
    offs = [int(x) for x in seg_offsets]
    p = int(prefix_len)
    n = len(offs) - 1
    t_total = offs[-1] if n >= 0 else p
    per_head = []
    for i in range(n):
        a, b = offs[i], offs[i + 1]
        nt = _cdiv(b - a, bmt)
        for t in reversed(range(nt)):
            qb = a + t * bmt
            qe = min(qb + bmt, b)
            per_head.append([FLAT_SUFFIX, i, qb, qe, 0, p, a, qe, 0])
    npre = _cdiv(p, bmt)
    for t in reversed(range(npre)):
        qb = t * bmt
        qe = min(qb + bmt, p)
        per_head.append([FLAT_PREFIX, -1, qb, qe, 0, qe, 0, 0, 0])
    ub = flat_items_per_head_ub(p, t_total, n, bmt)
    assert len(per_head) <= ub
    out = np.zeros((hkv * ub, FIELDS), dtype=np.int32)
    for blk in range(hkv * ub):
        h = blk % hkv
        j = blk // hkv
        if j < len(per_head):
            kind, seg, qb, qe, r0b, r0e, r1b, r1e, sp = per_head[j]
            out[blk] = [kind, h, seg, qb, qe, r0b, r0e, r1b, r1e, sp]
        else:
            out[blk] = [NONE, h, -1, 0, 0, 0, 0, 0, 0, 0]
    return out


def enumerate_paged(prefix_lens, hkv: int, draft_len: int, n_splits: int, split_len: int) -> np.ndarray:
    b_n = len(prefix_lens)
    out = np.zeros((b_n * hkv * n_splits, FIELDS), dtype=np.int32)
    for blk in range(out.shape[0]):
        s = blk % n_splits
        h = (blk // n_splits) % hkv
        b = blk // (n_splits * hkv)
        pl = int(prefix_lens[b])
        lo = min(s * split_len, pl)
        hi = min((s + 1) * split_len, pl)
        out[blk] = [PAGED_SPLIT, h, b, 0, draft_len, lo, hi, 0, 0, s]
    return out


def coverage_flat(items: np.ndarray, prefix_len: int, seg_offsets, hkv: int) -> np.ndarray:
    """Count, per kv head, how often each (row, key) pair is covered.

    Returns an int array [Hkv, T, T]; the visible set must be covered exactly
    once and nothing else at all.
    """
    offs = [int(x) for x in seg_offsets]
    t_n = offs[-1]
    cnt = np.zeros((hkv, t_n, t_n), dtype=np.int64)
    for it in items:
        kind, h, seg, qb, qe, r0b, r0e, r1b, r1e, _ = [int(x) for x in it]
        if kind == NONE:
            continue
        for r in range(qb, qe):
            for (lo, hi) in ((r0b, r0e), (r1b, r1e)):
                for c in range(lo, min(hi, r + 1)):
                    cnt[h, r, c] += 1
    return cnt
