"""Pins for ragged draft lengths in the verify oracle (CPU only).

With ``qo_indptr`` request b's draft rows are qo_indptr[b] .. qo_indptr[b+1].
Tied to the uniform path (equal lengths) and, request by request, to a
one-request uniform call of that request's own length (with and without a
draft tree)."""
import numpy as np

from oracle.attention import attn_paged
from psattn_inputs import BF16, make_paged, make_tree_mask


def _run(inst, mask=None, qo=None, **kw):
    return attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                      inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, q_dtype=inst.q_dtype,
                      kv_dtype=inst.kv_dtype, draft_mask=mask, qo_indptr=qo, **kw)


def test_equal_lengths_are_the_uniform_path():
    inst = make_paged([40, 0, 77], 5, 4, 2, 8, kv_dtype=BF16, seed=4, num_pages=40)
    qo = np.arange(4) * 5
    a = _run(inst)
    b = _run(inst, qo=qo)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_each_request_equals_its_own_uniform_call():
    lens = [3, 0, 6, 1]
    inst = make_paged([50, 20, 0, 33], 0, 4, 2, 8, kv_dtype=BF16, seed=8, num_pages=40, draft_lens=lens)
    qo = inst.qo_indptr
    assert inst.draft_len == 6 and qo[-1] == sum(lens)
    mask = make_tree_mask(4, 6, 3)
    for m in (None, mask):
        o, lse = _run(inst, m, qo)
        for b, n in enumerate(lens):
            r0 = qo[b]
            if n == 0:
                continue
            pages = inst.kv_indices[inst.kv_indptr[b]:inst.kv_indptr[b + 1]]
            o1, l1 = attn_paged(inst.q[r0:r0 + n], inst.k_pool, inst.v_pool, np.array([0, len(pages)]), pages,
                                inst.prefix_lens[b:b + 1], inst.k_ext[r0:r0 + n], inst.v_ext[r0:r0 + n], n,
                                inst.sm_scale, q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype,
                                draft_mask=None if m is None else m[b:b + 1, :n, :n])
            assert np.array_equal(o[r0:r0 + n], o1) and np.array_equal(lse[r0:r0 + n], l1)
        assert o.shape[0] == sum(lens) and np.all(np.isfinite(o))
