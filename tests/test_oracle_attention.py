"""Pins for the float64 oracle (CPU only).

Each check ties ``oracle.attention`` to something other than itself: a
different formulation (scalar brute force over the visibility predicate),
PyTorch's own causal attention in special cases the method reduces to,
closed forms, a hand-worked example, and invariants of the definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import attn_flat, attn_paged, causal_attention
from oracle.brute import brute_flat, visible
from psattn_inputs import BF16, F32, FP8, make_config, make_flat, make_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_flat(rng, p, lens, hq, hkv, d):
    t = p + sum(lens)
    offs = np.concatenate([[p], p + np.cumsum(lens)]).astype(np.int32) if lens else np.array([p], np.int32)
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    return q, k, v, offs


def _sdpa_causal(q, k, v, scale):
    """PyTorch causal attention in float64; q [L,Hq,D], k/v [L,Hkv,D]."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    z = (qt @ kt.transpose(1, 2)) * scale
    mask = torch.ones(z.shape[-2:], dtype=torch.bool).triu(1)
    z = z.masked_fill(mask, -math.inf)
    lse = torch.logsumexp(z, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ---------------------------------------------------------------------------
# brute force (different formulation: predicate on the flat layout, scalars)
# ---------------------------------------------------------------------------
def test_brute_force_tiny_config():
    inst = make_config("tiny")
    from oracle.decode import decode
    q, k, v = (decode(x, F32) for x in (inst.q, inst.k, inst.v))
    o, lse = attn_flat(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, inst.sm_scale, dtype=F32)
    bo, bl = brute_flat(q.tolist(), k.tolist(), v.tolist(), inst.prefix_len, inst.seg_offsets, inst.sm_scale)
    assert np.max(np.abs(o - np.array(bo))) <= 1e-12
    assert np.max(np.abs(lse - np.array(bl))) <= 1e-12


@pytest.mark.parametrize("case", range(50))
def test_brute_force_random_descriptors(case):
    rng = np.random.default_rng(1000 + case)
    p = int(rng.integers(0, 9))
    n = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(0, 7, size=n)]
    if p + sum(lens) == 0:
        lens[0] = 1
    hq, hkv = [(1, 1), (2, 1), (4, 2), (3, 1)][case % 4]
    d = [2, 4][case % 2]
    q, k, v, offs = _rand_flat(rng, p, lens, hq, hkv, d)
    sc = float(rng.uniform(0.2, 1.5))
    o, lse = attn_flat(q, k, v, p, offs, sc, dtype=None, check_prefix=True)
    bo, bl = brute_flat(q.tolist(), k.tolist(), v.tolist(), p, offs, sc)
    assert np.max(np.abs(o - np.array(bo))) <= 1e-12
    assert np.max(np.abs(lse - np.array(bl))) <= 1e-12


# ---------------------------------------------------------------------------
# library special cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(2, 2), (8, 2), (6, 1)])
def test_single_segment_is_plain_causal(hq, hkv):
    rng = np.random.default_rng(7)
    q, k, v, offs = _rand_flat(rng, 37, [29], hq, hkv, 16)
    o, lse = attn_flat(q, k, v, 37, offs, 0.25, dtype=None)
    ro, rl = _sdpa_causal(q, k, v, 0.25)
    assert np.max(np.abs(o - ro)) <= 1e-10
    assert np.max(np.abs(lse - rl)) <= 1e-10


def test_empty_prefix_is_per_segment_causal():
    rng = np.random.default_rng(8)
    lens = [5, 17, 1, 9]
    q, k, v, offs = _rand_flat(rng, 0, lens, 4, 2, 8)
    o, lse = attn_flat(q, k, v, 0, offs, 0.4, dtype=None)
    for a, b in zip(offs[:-1], offs[1:]):
        ro, rl = _sdpa_causal(q[a:b], k[a:b], v[a:b], 0.4)
        assert np.max(np.abs(o[a:b] - ro)) <= 1e-10
        assert np.max(np.abs(lse[a:b] - rl)) <= 1e-10


def test_expansion_equals_sdpa_on_each_expanded_sequence():
    """Definition check at a mid size: rollout i's rows == SDPA on [P | S_i]."""
    rng = np.random.default_rng(9)
    p, lens = 70, [33, 64, 1]
    q, k, v, offs = _rand_flat(rng, p, lens, 8, 2, 32)
    o, lse = attn_flat(q, k, v, p, offs, 0.2, dtype=None)
    for a, b in zip(offs[:-1], offs[1:]):
        idx = np.r_[0:p, a:b]
        ro, rl = _sdpa_causal(q[idx], k[idx], v[idx], 0.2)
        assert np.max(np.abs(o[a:b] - ro[p:])) <= 1e-10
        assert np.max(np.abs(o[:p] - ro[:p])) <= 1e-10
        assert np.max(np.abs(lse[a:b] - rl[p:])) <= 1e-10


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_zero_queries_give_uniform_attention():
    rng = np.random.default_rng(10)
    p, lens = 11, [4, 0, 7]
    q, k, v, offs = _rand_flat(rng, p, lens, 2, 1, 4)
    q[:] = 0.0
    o, lse = attn_flat(q, k, v, p, offs, 0.5, dtype=None)
    t_n = offs[-1]
    for r in range(t_n):
        vis = [c for c in range(t_n) if visible(r, c, p, offs)]
        n_vis = r + 1 if r < p else p + (r - max(a for a in offs[:-1] if a <= r)) + 1
        assert len(vis) == n_vis
        assert np.allclose(lse[r], math.log(n_vis), atol=1e-14, rtol=0)
        assert np.allclose(o[r, :, :], v[vis, 0, :].mean(axis=0), atol=1e-13, rtol=0)


def test_constant_values_and_first_row():
    rng = np.random.default_rng(11)
    q, k, v, offs = _rand_flat(rng, 6, [3, 5], 4, 2, 8)
    v[:] = 0.0
    v[:, 0, :] = 1.75
    v[:, 1, :] = -3.0
    o, lse = attn_flat(q, k, v, 6, offs, 0.3, dtype=None)
    assert np.allclose(o[:, :2, :], 1.75, atol=1e-13) and np.allclose(o[:, 2:, :], -3.0, atol=1e-13)
    q2, k2, v2, _ = _rand_flat(rng, 6, [3, 5], 4, 2, 8)
    o2, lse2 = attn_flat(q2, k2, v2, 6, offs, 0.3, dtype=None)
    for h in range(4):
        assert np.array_equal(o2[0, h], v2[0, h // 2])
        assert abs(lse2[0, h] - 0.3 * float(q2[0, h] @ k2[0, h // 2])) <= 1e-14


def test_ones_values_rows_sum_to_one():
    rng = np.random.default_rng(12)
    q, k, v, offs = _rand_flat(rng, 9, [4, 6], 2, 2, 3)
    q *= 4.0
    v[:] = 1.0
    o, _ = attn_flat(q, k, v, 9, offs, 1.0, dtype=None)
    assert np.max(np.abs(o - 1.0)) <= 1e-14


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(13)
    q, k, v, offs = _rand_flat(rng, 8, [6, 6], 1, 1, 4)
    # make key 3 (a prefix key) dominate for every row that can see it
    q[:] = np.abs(q) + 0.1
    k[:] = 0.0
    k[3, 0, :] = 200.0
    o, _ = attn_flat(q, k, v, 8, offs, 1.0, dtype=None)
    for r in range(3, offs[-1]):
        assert np.allclose(o[r, 0], v[3, 0], atol=1e-20 + 1e-12)


def test_hand_worked_example():
    """Values derived by hand in tests/golden/hand_example.json."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[:, None, None]
    k = np.array(g["k"], dtype=np.float64)[:, None, None]
    v = np.array(g["v"], dtype=np.float64)[:, None, None]
    o, lse = attn_flat(q, k, v, g["prefix_len"], g["seg_offsets"], g["sm_scale"], dtype=None)
    assert np.allclose(o[:, 0, 0], g["expected_o"], atol=1e-14, rtol=0)
    assert np.allclose(lse[:, 0], g["expected_lse"], atol=1e-14, rtol=0)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_segment_rows_unchanged_when_others_added_removed_permuted():
    rng = np.random.default_rng(14)
    p = 13
    lens = [5, 9, 3, 7]
    q, k, v, offs = _rand_flat(rng, p, lens, 4, 2, 8)
    o, lse = attn_flat(q, k, v, p, offs, 0.3, dtype=None)
    segs = [np.arange(offs[i], offs[i + 1]) for i in range(4)]
    for order in ([2, 0], [3, 2, 1, 0], [1]):
        idx = np.concatenate([np.arange(p)] + [segs[i] for i in order])
        new_lens = [lens[i] for i in order]
        noffs = np.concatenate([[p], p + np.cumsum(new_lens)])
        o2, l2 = attn_flat(q[idx], k[idx], v[idx], p, noffs, 0.3, dtype=None)
        pos = p
        for i in order:
            assert np.array_equal(o2[pos:pos + lens[i]], o[offs[i]:offs[i + 1]])
            assert np.array_equal(l2[pos:pos + lens[i]], lse[offs[i]:offs[i + 1]])
            pos += lens[i]
        assert np.array_equal(o2[:p], o[:p])


def test_row_subset_matches_full():
    inst = make_flat(40, [9, 23, 2], 4, 2, 16, dtype=BF16, seed=3)
    o, lse = attn_flat(inst.q, inst.k, inst.v, 40, inst.seg_offsets, inst.sm_scale, dtype=BF16)
    rows = [0, 39, 40, 48, 49, 71, 73]
    o2, l2 = attn_flat(inst.q, inst.k, inst.v, 40, inst.seg_offsets, inst.sm_scale, dtype=BF16, rows=rows)
    # BLAS may block a different number of rows differently: equal to rounding
    assert np.max(np.abs(o2 - o[rows])) <= 1e-13 and np.max(np.abs(l2 - lse[rows])) <= 1e-13


# ---------------------------------------------------------------------------
# paged mode
# ---------------------------------------------------------------------------
def test_paged_equals_flat_reencoding():
    """A flat instance rewritten as paged requests (prefix in shuffled pages,
    each rollout a request whose draft block is its suffix) gives the same
    suffix rows."""
    rng = np.random.default_rng(15)
    p, s, n, hq, hkv, d = 37, 5, 3, 4, 2, 8
    q, k, v, offs = _rand_flat(rng, p, [s] * n, hq, hkv, d)
    o, lse = attn_flat(q, k, v, p, offs, 0.35, dtype=None)
    n_pages = -(-p // 16)
    pool_pages = n_pages * n + 3
    perm = rng.permutation(pool_pages)
    kp = np.full((pool_pages, 16, hkv, d), np.nan)
    vp = np.full((pool_pages, 16, hkv, d), np.nan)
    indptr = [0]
    indices = []
    for b in range(n):
        pages = perm[b * n_pages:(b + 1) * n_pages]
        for t in range(p):
            kp[pages[t // 16], t % 16] = k[t]
            vp[pages[t // 16], t % 16] = v[t]
        indices.extend(pages.tolist())
        indptr.append(len(indices))
    qd = np.concatenate([q[offs[b]:offs[b + 1]] for b in range(n)])
    kd = np.concatenate([k[offs[b]:offs[b + 1]] for b in range(n)])
    vd = np.concatenate([v[offs[b]:offs[b + 1]] for b in range(n)])
    # float32-exact storage is not needed: pass float64 through the f32 path
    # by decoding with dtype 0 on float64 arrays is lossy, so use bit-exact
    # float32 inputs instead
    q32, kp32, vp32, kd32, vd32 = (x.astype(np.float32) for x in (qd, kp, vp, kd, vd))
    o32, l32 = attn_flat(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), p, offs, 0.35, dtype=F32)
    po, pl = attn_paged(q32, kp32, vp32, indptr, indices, [p] * n, kd32, vd32, s, 0.35,
                        q_dtype=F32, kv_dtype=F32)
    assert np.max(np.abs(po - o32[p:])) <= 1e-12
    assert np.max(np.abs(pl - l32[p:])) <= 1e-12


def test_paged_scales_are_linear():
    inst = make_paged([40, 0, 17], 3, 4, 2, 16, kv_dtype=FP8, seed=5, num_pages=9, scales=False)
    args = (inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
            inst.k_ext, inst.v_ext, inst.draft_len)
    o1, l1 = attn_paged(*args, 0.25, k_scale=1.0, v_scale=1.0, kv_dtype=FP8)
    o2, l2 = attn_paged(*args, 0.125, k_scale=2.0, v_scale=1.0, kv_dtype=FP8)
    o3, l3 = attn_paged(*args, 0.25, k_scale=1.0, v_scale=1.5, kv_dtype=FP8)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12
    assert np.max(np.abs(o3 - 1.5 * o1)) <= 1e-12 and np.array_equal(l3, l1)


def test_paged_zero_prefix_is_draft_causal():
    inst = make_paged([0, 0], 5, 2, 1, 8, kv_dtype=BF16, seed=6, num_pages=1)
    from oracle.decode import decode
    o, lse = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices,
                        inst.prefix_lens, inst.k_ext, inst.v_ext, 5, 0.3)
    for b in range(2):
        sl = slice(b * 5, b * 5 + 5)
        ro, rl = _sdpa_causal(decode(inst.q[sl], BF16), decode(inst.k_ext[sl], BF16),
                              decode(inst.v_ext[sl], BF16), 0.3)
        assert np.max(np.abs(o[sl] - ro)) <= 1e-12 and np.max(np.abs(lse[sl] - rl)) <= 1e-12


@pytest.mark.parametrize("cuts", [[0, 7, 7, 40, 64], [0, 1, 2, 64], [0, 33, 64]])
def test_split_merge_equals_unsplit(cuts):
    """Associativity of the log-sum-exp: attention over arbitrary key splits
    (including an empty one) merged with O = sum_s e^(LSE_s - LSE) O_s,
    LSE = log sum_s e^LSE_s equals attention over all keys at once."""
    rng = np.random.default_rng(31)
    L, hq, hkv, d = 64, 6, 2, 8
    kx = rng.standard_normal((L, hkv, d))
    vx = rng.standard_normal((L, hkv, d))
    qr = rng.standard_normal((5, hq, d))
    qpos = np.full(5, L - 1)
    o_all, l_all = causal_attention(qr, qpos, kx, vx, 0.3)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b > a:
            parts.append(causal_attention(qr, np.full(5, b - a - 1), kx[a:b], vx[a:b], 0.3))
        else:
            parts.append((np.zeros_like(o_all), np.full(l_all.shape, -np.inf)))  # empty split
    lses = np.stack([p[1] for p in parts])
    lse = np.logaddexp.reduce(lses, axis=0)
    w = np.exp(lses - lse[None])
    o = np.einsum("shr,shrd->hrd", w.transpose(0, 2, 1), np.stack([p[0] for p in parts]).transpose(0, 2, 1, 3))
    assert np.allclose(lse, l_all, atol=1e-12, rtol=0)
    assert np.allclose(o.transpose(1, 0, 2), o_all, atol=1e-12, rtol=0)


def test_causal_attention_rejects_bad_heads():
    with pytest.raises(ValueError):
        causal_attention(np.zeros((1, 3, 2)), np.array([0]), np.zeros((1, 2, 2)), np.zeros((1, 2, 2)), 1.0)
