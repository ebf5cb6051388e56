"""GPU test of the allocation-free forward (psattn_fwd_noalloc) through the C
ABI: its outputs equal those of psattn_fwd with a caller workspace on the
same inputs, bit for bit, over two calls in a row (the second smaller, so
the shared device array still holds the first call's partials), and the
smaller call also meets the oracle's tolerance."""
import numpy as np
import pytest

from gpu_util import compare, kind_of, to_dev, to_f64
from oracle.attention import attn_paged
from psattn_inputs import BF16, FP8, make_config, make_flat, make_paged

pytestmark = pytest.mark.gpu


def _paged_both(ps, inst):
    import torch

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    q = to_dev(inst.q, inst.q_dtype)
    kp, vp = to_dev(inst.k_pool, inst.kv_dtype), to_dev(inst.v_pool, inst.kv_dtype)
    kx, vx = to_dev(inst.k_ext, inst.kv_dtype), to_dev(inst.v_ext, inst.kv_dtype)
    ind, idx, pl = i32(inst.kv_indptr), i32(inst.kv_indices), i32(inst.prefix_lens)
    args = (q, kp, vp, ind, idx, pl, kx, vx, inst.draft_len, inst.max_prefix_len)
    kw = dict(sm_scale=inst.sm_scale, k_scale=inst.k_scale, v_scale=inst.v_scale, kv_dtype=inst.kv_dtype)
    o_ref, l_ref = ps.fwd_paged(*args, **kw)
    o_na, l_na = ps.fwd_paged(*args, **kw, noalloc=True)
    torch.cuda.synchronize()
    return o_ref, l_ref, o_na, l_na


def test_noalloc_matches_psattn_fwd_twice_second_smaller(gpu_lib):
    import torch

    big = make_config("verify_fp8")  # 16.8 MB of partials
    small = make_paged([700, 33, 0, 129], 4, 16, 2, 128, kv_dtype=BF16, seed=91, num_pages=80)
    assert gpu_lib.psattn_workspace_size(
        gpu_lib.paged_desc(small.batch, 4, 16, small.num_pages, 1, 1, 1, small.max_prefix_len, 1, 1),
        16, 2, 128, BF16, BF16) < 16 << 20
    for inst in (big, small):
        o_ref, l_ref, o_na, l_na = _paged_both(gpu_lib, inst)
        assert torch.equal(o_ref, o_na) and torch.equal(l_ref, l_na), inst.name
    ro, rl = attn_paged(small.q, small.k_pool, small.v_pool, small.kv_indptr, small.kv_indices, small.prefix_lens,
                        small.k_ext, small.v_ext, small.draft_len, small.sm_scale, q_dtype=small.q_dtype,
                        kv_dtype=small.kv_dtype, page_size=small.page_size)
    compare(to_f64(o_na), to_f64(l_na), ro, rl, kind_of(small.q_dtype, small.kv_dtype), "noalloc small")


def test_noalloc_flat_needs_no_scratch(gpu_lib):
    import torch

    inst = make_flat(300, [100, 41], 16, 4, 128, dtype=BF16, seed=92)
    q, k, v = (to_dev(x, BF16) for x in (inst.q, inst.k, inst.v))
    seg = torch.from_numpy(inst.seg_offsets).cuda()
    o1, l1 = gpu_lib.fwd_flat(q, k, v, inst.prefix_len, seg, inst.max_seg_len, sm_scale=inst.sm_scale)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    desc = gpu_lib.flat_desc(inst.total_tokens, inst.prefix_len, inst.num_segments, seg.data_ptr(),
                             inst.max_seg_len)
    st = gpu_lib.psattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), desc,
                                    16, 4, 128, inst.sm_scale, BF16, BF16, 1.0, 1.0,
                                    torch.cuda.current_stream().cuda_stream)
    gpu_lib.check(st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
