"""Pins for the tree-mask verify of the oracle (CPU only).

``attn_paged(..., draft_mask=M)`` lets draft row t see draft key j iff M[t, j]
(and every prefix key).  It is tied to the causal path (the chain mask is the
lower triangle), to a scalar brute force over the visibility, and to the
invariance of the result under a relabelling of the draft tokens.
"""
import math

import numpy as np

from oracle.attention import attn_paged
from oracle.decode import decode
from psattn_inputs import BF16, make_paged, make_tree_mask


def _paged(seed, prefix_lens=(37, 0, 70), lx=5, hq=4, hkv=2, d=8):
    return make_paged(list(prefix_lens), lx, hq, hkv, d, kv_dtype=BF16, seed=seed, num_pages=40)


def _run(inst, mask=None, requests=None):
    return attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                      inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, q_dtype=inst.q_dtype,
                      kv_dtype=inst.kv_dtype, requests=requests, draft_mask=mask)


def test_chain_mask_is_the_causal_path():
    inst = _paged(1)
    chain = make_tree_mask(len(inst.prefix_lens), inst.draft_len, 0, chain=True)
    o0, l0 = _run(inst)
    o1, l1 = _run(inst, chain)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_tree_mask_matches_scalar_brute_force():
    inst = _paged(2)
    lx = inst.draft_len
    mask = make_tree_mask(len(inst.prefix_lens), lx, 5)
    o, lse = _run(inst, mask)
    q = decode(inst.q, BF16)
    kx = decode(inst.k_ext, BF16)
    vx = decode(inst.v_ext, BF16)
    kp = decode(inst.k_pool, BF16)
    vp = decode(inst.v_pool, BF16)
    g = inst.hq // inst.hkv
    for b, pl in enumerate(inst.prefix_lens):
        pages = inst.kv_indices[inst.kv_indptr[b]:inst.kv_indptr[b + 1]]
        for t in range(lx):
            for h in range(inst.hq):
                kvh = h // g
                keys, vals = [], []
                for j in range(int(pl)):
                    pg, sl = pages[j // 16], j % 16
                    keys.append(kp[pg, sl, kvh])
                    vals.append(vp[pg, sl, kvh])
                for j in range(lx):
                    if mask[b, t, j]:
                        keys.append(kx[b * lx + j, kvh])
                        vals.append(vx[b * lx + j, kvh])
                qv = q[b * lx + t, h]
                z = [inst.sm_scale * math.fsum(float(a) * float(c) for a, c in zip(qv, kk)) for kk in keys]
                m = max(z)
                w = [math.exp(x - m) for x in z]
                s = math.fsum(w)
                want = [math.fsum(wi * float(vv[dd]) for wi, vv in zip(w, vals)) / s for dd in range(inst.d)]
                assert np.allclose(o[b * lx + t, h], want, rtol=0, atol=1e-12)
                assert abs(lse[b * lx + t, h] - (m + math.log(s))) < 1e-12


def test_relabelling_the_draft_tokens_permutes_the_rows():
    inst = _paged(3, prefix_lens=(20, 45), lx=6)
    lx = inst.draft_len
    mask = make_tree_mask(2, lx, 9)
    o, lse = _run(inst, mask)
    perm = np.array([3, 0, 5, 1, 4, 2])
    rows = np.concatenate([b * lx + perm for b in range(2)])
    inst.q = inst.q[rows]
    inst.k_ext = inst.k_ext[rows]
    inst.v_ext = inst.v_ext[rows]
    pmask = mask[:, perm][:, :, perm]
    o2, l2 = _run(inst, pmask)
    assert np.allclose(o2, o[rows], rtol=0, atol=1e-13) and np.allclose(l2, lse[rows], rtol=0, atol=1e-13)
