"""GPU parity of tree-mask verify (draft_mask) against the float64 oracle.

Seeded draft trees (each token's parent drawn from the earlier tokens, or none)
over the three draft-block paths: the register kernel (up to 16 stacked rows),
the wide kernel (17..64) and the split pass plus combine (more rows, fp32)."""
import numpy as np
import pytest

from gpu_util import compare, kind_of, run_paged, to_f64
from oracle.attention import attn_paged
from psattn_inputs import BF16, F32, FP8, make_paged, make_tree_mask

pytestmark = pytest.mark.gpu


def _tree_check(lib, inst, mask, label):
    o, lse = run_paged(lib, inst, draft_mask=mask)
    ro, rl = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                        inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, k_scale=inst.k_scale,
                        v_scale=inst.v_scale, q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype, draft_mask=mask, page_size=inst.page_size)
    return compare(to_f64(o), to_f64(lse), ro, rl, kind_of(inst.q_dtype, inst.kv_dtype), label)


@pytest.mark.parametrize("prefix_lens,lx,hq,hkv,d,kvdt", [
    ([1000, 0, 17], 4, 8, 2, 128, BF16),       # register kernel, 16 rows, an empty prefix
    ([300, 301], 8, 4, 2, 128, BF16),          # register kernel, 16 rows, 8-token trees
    ([3000, 1500, 0], 2, 8, 2, 128, FP8),      # register kernel, fp8
    ([4100], 4, 8, 2, 256, FP8),               # register kernel, fp8, D = 256
    ([3000, 70, 0], 8, 16, 4, 128, BF16),      # wide kernel, 32 rows
    ([2500, 63], 16, 8, 2, 128, FP8),          # wide kernel, 64 rows, 16-token trees
    ([1000, 4097], 6, 16, 2, 64, FP8),         # wide kernel, D = 64
    ([777], 16, 8, 1, 128, FP8),               # split pass + combine, 128 rows
    ([257, 1024], 4, 4, 2, 128, F32),          # fp32: split pass + combine
])
def test_verify_tree_mask(gpu_lib, prefix_lens, lx, hq, hkv, d, kvdt):
    n_pages = int(sum((x + 15) // 16 for x in prefix_lens)) + 7
    inst = make_paged(prefix_lens, lx, hq, hkv, d, kv_dtype=kvdt, seed=7 + sum(prefix_lens) % 997,
                      num_pages=n_pages, scales=(kvdt == FP8))
    mask = make_tree_mask(len(prefix_lens), lx, seed=lx + hq + d)
    _tree_check(gpu_lib, inst, mask, f"tree {prefix_lens} Lx={lx} {hq}/{hkv} D={d}")


def test_verify_chain_mask_equals_the_causal_call(gpu_lib):
    import torch

    inst = make_paged([2000, 513], 8, 16, 2, 128, kv_dtype=BF16, seed=3, num_pages=200)
    chain = make_tree_mask(2, 8, 0, chain=True)
    o0, l0 = run_paged(gpu_lib, inst)
    o1, l1 = run_paged(gpu_lib, inst, draft_mask=chain)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_verify_tree_fullsize_c3_shape(gpu_lib):
    # the verify16k shape (8 x 16384 prefix, 32 / 8 heads, D = 128) with 4-token trees
    from psattn_inputs import make_config

    inst = make_config("verify16k")
    mask = make_tree_mask(8, inst.draft_len, seed=11)
    _tree_check(gpu_lib, inst, mask, "tree verify16k")
