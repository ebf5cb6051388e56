"""GPU parity of verify with ragged draft lengths (qo_indptr) against the
float64 oracle, on the register, wide and split + combine paths, with the
causal chain and with draft trees; requests without draft rows included."""
import numpy as np
import pytest

from gpu_util import compare, kind_of, run_paged, to_f64
from oracle.attention import attn_paged
from psattn_inputs import BF16, F32, FP8, make_paged, make_tree_mask

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prefix_lens,lens,hq,hkv,d,kvdt,tree", [
    ([1000, 0, 17, 300], [4, 2, 0, 3], 8, 2, 128, BF16, False),    # register kernel (16 rows)
    ([1000, 0, 17, 300], [4, 2, 0, 3], 8, 2, 128, BF16, True),
    ([3000, 1500, 0], [2, 1, 2], 8, 2, 128, FP8, True),            # register kernel, fp8
    ([3000, 70, 0], [8, 3, 5], 16, 4, 128, BF16, False),           # wide kernel (32 rows)
    ([2500, 63], [16, 9], 8, 2, 256, FP8, True),                   # wide kernel, 64 rows, D = 256
    ([777, 50], [16, 7], 8, 1, 128, FP8, False),                   # split + combine (128 rows)
    ([777, 50], [16, 7], 8, 1, 128, FP8, True),
    ([257, 1024], [4, 1], 4, 2, 128, F32, True),                   # fp32: split + combine
])
def test_verify_ragged_draft_lengths(gpu_lib, prefix_lens, lens, hq, hkv, d, kvdt, tree):
    n_pages = int(sum((x + 15) // 16 for x in prefix_lens)) + 7
    inst = make_paged(prefix_lens, 0, hq, hkv, d, kv_dtype=kvdt, seed=13 + sum(lens), num_pages=n_pages,
                      scales=(kvdt == FP8), draft_lens=lens)
    mask = make_tree_mask(len(lens), inst.draft_len, seed=sum(lens)) if tree else None
    o, lse = run_paged(gpu_lib, inst, draft_mask=mask)
    assert o.shape[0] == sum(lens)
    ro, rl = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                        inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, k_scale=inst.k_scale,
                        v_scale=inst.v_scale, q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype, draft_mask=mask, page_size=inst.page_size,
                        qo_indptr=inst.qo_indptr)
    compare(to_f64(o), to_f64(lse), ro, rl, kind_of(inst.q_dtype, inst.kv_dtype),
            f"ragged {prefix_lens} lens={lens} {hq}/{hkv} D={d} tree={tree}")


def test_verify_equal_ragged_lengths_match_the_uniform_call(gpu_lib):
    import torch

    a = make_paged([2000, 513, 90], 6, 16, 2, 128, kv_dtype=BF16, seed=5, num_pages=200)
    b = make_paged([2000, 513, 90], 6, 16, 2, 128, kv_dtype=BF16, seed=5, num_pages=200)
    b.qo_indptr = np.arange(4, dtype=np.int32) * 6
    o0, l0 = run_paged(gpu_lib, a)
    o1, l1 = run_paged(gpu_lib, b)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
