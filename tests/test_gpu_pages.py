"""GPU parity of the verify path for page sizes other than 16 slots.

The paged pool (sglang PR #27382 report, "关键源码片段": ``k_buffer`` addressed
by ``kv_indptr`` / ``kv_indices``) fixes no page size.  The planner routes
power-of-two pages of fewer than 16 slots to the LDS-streaming split kernel,
other page sizes to the tiled split kernel, and power-of-two pages of 16 or
more slots to the register / wide streaming kernels; every route is compared
with the float64 oracle on the same seeded bytes, with partial last pages, an
empty prefix, several splits per request, fp8 scales, draft trees and ragged
draft lengths.
"""
import numpy as np
import pytest

from gpu_util import compare, kind_of, run_paged, to_f64
from oracle.attention import attn_paged
from psattn_inputs import BF16, FP8, make_paged, make_paged_spikes, make_tree_mask

pytestmark = pytest.mark.gpu

# (prefix lengths, Lx, Hq, Hkv, D, kv dtype): stacked rows R = Lx * Hq / Hkv
SHAPES = [
    ([700, 129, 0, 37], 4, 8, 2, 128, BF16),     # R = 16
    ([513, 1000, 3], 5, 16, 2, 128, BF16),       # R = 40
    ([900, 77], 8, 16, 2, 256, FP8),             # R = 64, D = 256
    ([650, 31, 200], 3, 8, 4, 64, FP8),          # R = 6, D = 64
    ([1200, 50], 3, 8, 1, 128, FP8),             # R = 24
]
PAGE_SIZES = [1, 4, 8, 12, 24, 32, 64]


def _check(lib, inst, label, mask=None):
    o, lse = run_paged(lib, inst, draft_mask=mask)
    ro, rl = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices, inst.prefix_lens,
                        inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale, k_scale=inst.k_scale,
                        v_scale=inst.v_scale, q_dtype=inst.q_dtype, kv_dtype=inst.kv_dtype, draft_mask=mask,
                        qo_indptr=inst.qo_indptr, page_size=inst.page_size)
    return compare(to_f64(o), to_f64(lse), ro, rl, kind_of(inst.q_dtype, inst.kv_dtype), label)


def _pool(prefix_lens, ps):
    return int(sum((x + ps - 1) // ps for x in prefix_lens)) + 11


@pytest.mark.parametrize("ps", PAGE_SIZES)
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_verify_page_sizes(gpu_lib, ps, shape):
    pl, lx, hq, hkv, d, kv = SHAPES[shape]
    inst = make_paged(pl, lx, hq, hkv, d, kv_dtype=kv, seed=500 + 7 * ps + shape, num_pages=_pool(pl, ps),
                      scales=(kv == FP8), page_size=ps)
    info = gpu_lib.plan_info(gpu_lib.paged_desc(inst.batch, lx, ps, inst.num_pages, 1, 1, 1, inst.max_prefix_len,
                                                1, 1), hq, hkv, d, inst.q_dtype, inst.kv_dtype)
    _check(gpu_lib, inst, f"page {ps} {pl} Lx={lx} {hq}/{hkv} D={d} kv={kv} splits={info.n_splits}")


@pytest.mark.parametrize("ps", [1, 4, 8, 12])
def test_verify_small_pages_tree_and_ragged(gpu_lib, ps):
    lens = [3, 0, 6, 1]
    pl = [400, 90, 0, 257]
    inst = make_paged(pl, 0, 16, 4, 128, kv_dtype=BF16, seed=900 + ps, num_pages=_pool(pl, ps), draft_lens=lens,
                      page_size=ps)
    mask = make_tree_mask(len(lens), inst.draft_len, seed=ps)
    _check(gpu_lib, inst, f"page {ps} ragged tree {pl} lens={lens}", mask=mask)


@pytest.mark.parametrize("ps,kv", [(2, BF16), (8, FP8), (24, BF16)])
def test_verify_small_pages_spikes(gpu_lib, ps, kv):
    """Spike keys far above the rest: a softmax that lost its row maximum
    overflows here."""
    pl = [600, 301]
    inst = make_paged_spikes(pl, 4, 16, 2, 128, spikes=[5, 290, 599], kv_dtype=kv, seed=61 + ps,
                             num_pages=_pool(pl, ps), page_size=ps)
    _check(gpu_lib, inst, f"page {ps} spikes kv={kv}")


def test_verify_long_prefix_one_slot_pages(gpu_lib):
    """One-slot pages over a long prefix: many splits, each limited by the
    page list the streaming kernel keeps in LDS."""
    pl = [5000, 4093]
    inst = make_paged(pl, 4, 32, 8, 128, kv_dtype=BF16, seed=77, num_pages=_pool(pl, 1), page_size=1)
    info = gpu_lib.plan_info(gpu_lib.paged_desc(inst.batch, 4, 1, inst.num_pages, 1, 1, 1, inst.max_prefix_len,
                                                1, 1), 32, 8, 128, BF16, BF16)
    assert info.n_splits >= 8
    _check(gpu_lib, inst, f"page 1 long prefix splits={info.n_splits}")
