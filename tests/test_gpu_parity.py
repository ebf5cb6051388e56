"""GPU parity: the HIP library (through its C ABI) against the float64 oracle
on the same seeded bytes.

Small instances are compared element by element on every row; the full-size
workloads are compared on every row where the oracle is cheap (paged verify)
and on sampled rows otherwise (flat GRPO), with the sample spanning the
prefix, every rollout, tile boundaries and ragged tails.
"""
import math

import numpy as np
import pytest

from gpu_util import compare, kind_of, run_flat, run_paged, sample_rows as _sample_rows, to_dev, to_f64
from oracle.attention import attn_flat, attn_paged
from psattn_inputs import (BF16, F32, FP8, make_config, make_flat, make_flat_random_lens, make_flat_spikes,
                           make_paged, make_paged_spikes)

pytestmark = pytest.mark.gpu


def _flat_check(lib, inst, rows=None, label=""):
    o, lse = run_flat(lib, inst)
    o64, l64 = to_f64(o), to_f64(lse)
    ro, rl = attn_flat(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, inst.sm_scale,
                       dtype=inst.dtype, rows=rows)
    if rows is not None:
        o64, l64 = o64[rows], l64[rows]
    return compare(o64, l64, ro, rl, kind_of(inst.dtype), label or inst.name)


def _paged_check(lib, inst, label=""):
    o, lse = run_paged(lib, inst)
    ro, rl = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices,
                        inst.prefix_lens, inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale,
                        k_scale=inst.k_scale, v_scale=inst.v_scale, q_dtype=inst.q_dtype,
                        kv_dtype=inst.kv_dtype, page_size=inst.page_size)
    return compare(to_f64(o), to_f64(lse), ro, rl, kind_of(inst.q_dtype, inst.kv_dtype), label or inst.name)


# --------------------------------------------------------------------------- flat
def test_tiny_fp32(gpu_lib):
    _flat_check(gpu_lib, make_config("tiny"))


def test_grpo_small_full(gpu_lib):
    inst = make_flat(512, [200, 128, 1, 77], 32, 8, 128, dtype=BF16, seed=21, name="grpo_small")
    _flat_check(gpu_lib, inst)


def test_grpo_fullsize_sampled(gpu_lib):
    inst = make_config("grpo")
    _flat_check(gpu_lib, inst, rows=_sample_rows(inst))


@pytest.mark.parametrize("n", [1, 16])
def test_grpo_rollout_count_sampled(gpu_lib, n):
    # the read-once sweep's extremes: one rollout, and sixteen (T = 10240)
    inst = make_flat(2048, [512] * n, 32, 8, 128, dtype=BF16, seed=200 + n, name=f"grpo_n{n}")
    _flat_check(gpu_lib, inst, rows=_sample_rows(inst))


@pytest.mark.parametrize("d", [64, 128])
def test_flat_reversed_prefix_walk_every_row(gpu_lib, d):
    # 64 kv heads leave 512 / 64 = 8 workgroup slots per head, so items 8..15
    # of every head (a second generation) walk the prefix's clean tiles last
    # to first; G = 1 gives 128-token tiles: 8 prefix items and 9 rollout
    # items per head.  Every row is compared.
    inst = make_flat(1000, [300, 300, 257], 64, 64, d, dtype=BF16, seed=31 + d, name=f"rev_walk_d{d}")
    _flat_check(gpu_lib, inst)


def test_grpo_ragged_fullsize_sampled(gpu_lib):
    inst = make_config("grpo_ragged")
    _flat_check(gpu_lib, inst, rows=_sample_rows(inst, n_random=24))


def test_grpo_ragged_small_full_with_outliers(gpu_lib):
    inst = make_flat_random_lens(300, 5, 20, 150, 16, 2, 128, dtype=BF16, seed=22, outlier_frac=0.01)
    _flat_check(gpu_lib, inst, label="ragged_small_outliers")


@pytest.mark.parametrize("p,lens,hq,hkv,d,dt", [
    (100, [37], 8, 2, 128, BF16),                 # N = 1
    (0, [33, 5, 70], 8, 2, 128, BF16),            # no prefix
    (64, [1, 1, 1, 1], 4, 4, 64, BF16),           # one-token rollouts, Hq = Hkv
    (50, [0, 20, 0, 9], 16, 4, 128, BF16),        # empty rollouts
    (130, [3, 200], 12, 4, 128, BF16),            # G = 3 (42-token tiles)
    (96, [40, 41], 32, 2, 256, BF16),             # D = 256, G = 16
    (77, [19, 64], 64, 1, 64, BF16),              # G = 64 (2-token tiles)
    (40, [9, 10], 128, 1, 64, BF16),              # G = 128, the largest group (1-token tiles)
    (1, [], 2, 1, 64, BF16),                      # prefix of one token only
    (0, [1], 1, 1, 128, BF16),                    # a single token in total
    (70, [15, 33], 4, 2, 128, F32),               # fp32, D = 128
    (40, [9, 10], 2, 1, 256, F32),                # fp32, D = 256
])
def test_flat_edge_cases(gpu_lib, p, lens, hq, hkv, d, dt):
    inst = make_flat(p, lens, hq, hkv, d, dtype=dt, seed=p + len(lens) + d)
    _flat_check(gpu_lib, inst, label=f"edge P={p} lens={lens} {hq}/{hkv} D={d}")


def test_flat_zero_queries_closed_form(gpu_lib):
    """Q = 0: every row attends uniformly, LSE = ln(#visible keys)."""
    inst = make_flat(45, [10, 0, 23], 8, 2, 128, dtype=BF16, seed=5)
    inst.q[:] = 0
    o, lse = run_flat(gpu_lib, inst)
    l64 = to_f64(lse)
    offs = inst.seg_offsets
    for r in range(inst.total_tokens):
        if r < inst.prefix_len:
            n_vis = r + 1
        else:
            seg = int(np.searchsorted(offs, r, side="right")) - 1
            n_vis = inst.prefix_len + (r - int(offs[seg])) + 1
        assert np.allclose(l64[r], math.log(n_vis), atol=1e-5), (r, l64[r], math.log(n_vis))


def test_flat_deterministic_and_segment_invariant(gpu_lib):
    """Two identical calls are bitwise equal, and a rollout's rows are bitwise
    unchanged when the other rollouts are removed or permuted."""
    import torch

    inst = make_flat(150, [40, 70, 25], 16, 4, 128, dtype=BF16, seed=9)
    o1, l1 = run_flat(gpu_lib, inst)
    o2, l2 = run_flat(gpu_lib, inst)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    p = inst.prefix_len
    offs = inst.seg_offsets
    order = [2, 0]
    idx = np.concatenate([np.arange(p)] + [np.arange(offs[i], offs[i + 1]) for i in order])
    lens = [int(offs[i + 1] - offs[i]) for i in order]
    inst2 = make_flat(p, lens, 16, 4, 128, dtype=BF16, seed=9)
    inst2.q, inst2.k, inst2.v = inst.q[idx], inst.k[idx], inst.v[idx]
    o3, l3 = run_flat(gpu_lib, inst2)
    pos = p
    for i in order:
        n = int(offs[i + 1] - offs[i])
        assert torch.equal(o3[pos:pos + n], o1[offs[i]:offs[i + 1]])
        assert torch.equal(l3[pos:pos + n], l1[offs[i]:offs[i + 1]])
        pos += n
    assert torch.equal(o3[:p], o1[:p])


# --------------------------------------------------------------------------- paged
def test_verify16k_fullsize(gpu_lib):
    _paged_check(gpu_lib, make_config("verify16k"))


def test_verify_fp8_fullsize(gpu_lib):
    _paged_check(gpu_lib, make_config("verify_fp8"))


def test_verify_head_dim_256(gpu_lib):
    # shape of the verify page's own head-dim-256 parity case
    inst = make_paged([4096] * 2, 4, 16, 2, 256, kv_dtype=BF16, seed=31, num_pages=600)
    _paged_check(gpu_lib, inst, label="verify D=256 [4096]x2")


@pytest.mark.parametrize("hq,hkv", [(32, 1), (16, 2), (8, 2)])
def test_verify_gqa_ratios(gpu_lib, hq, hkv):
    inst = make_paged([2048] * 2, 4, hq, hkv, 256, kv_dtype=BF16, seed=32 + hq, num_pages=300)
    _paged_check(gpu_lib, inst, label=f"verify GQA {hq}/{hkv}")


@pytest.mark.parametrize("prefix_len,lx,hq,hkv,d,kvdt", [
    (8192, 4, 4, 1, 128, BF16),    # 16 stacked rows: register streaming
    (32768, 2, 16, 1, 128, FP8),   # 32 stacked rows: wide streaming
])
def test_verify_sixty_four_splits(gpu_lib, prefix_len, lx, hq, hkv, d, kvdt):
    # one request and one kv head: the planner takes its largest split count,
    # 64, the most the merge holds (one split weight per lane)
    inst = make_paged([prefix_len], lx, hq, hkv, d, kv_dtype=kvdt, seed=95, num_pages=prefix_len // 16 + 8,
                      scales=kvdt == FP8, name=f"splits64_{kind_of(BF16, kvdt)}")
    fake = 256
    info = gpu_lib.plan_info(gpu_lib.paged_desc(1, lx, inst.page_size, inst.num_pages, fake, fake, fake, prefix_len,
                                                fake, fake), hq, hkv, d, inst.q_dtype, inst.kv_dtype)
    assert info.n_splits == 64
    _paged_check(gpu_lib, inst)


@pytest.mark.parametrize("prefix_lens,lx,hq,hkv,d,kvdt", [
    ([1000, 0, 17, 4096, 33], 3, 8, 2, 128, BF16),   # ragged, empty, partial pages
    ([300, 301], 1, 4, 4, 64, BF16),                  # Lx = 1, Hq = Hkv
    ([5000, 2500], 8, 16, 2, 256, FP8),               # fp8, partial last page
    ([777], 16, 8, 1, 128, FP8),                      # 128 stacked rows
    ([257, 1024], 4, 4, 2, 128, F32),                 # fp32
    ([2000], 2, 2, 1, 256, F32),                      # fp32, D = 256
    ([3000, 1500, 0], 2, 8, 2, 128, FP8),             # fp8, 8 stacked rows, empty prefix
    ([900, 2049], 16, 4, 4, 64, FP8),                 # fp8, D = 64, 16-token draft, G = 1
    ([4100], 4, 8, 2, 256, FP8),                      # fp8, D = 256, 16 stacked rows
    ([333, 16, 15], 16, 2, 2, 128, BF16),             # 16-token draft, one full / partial page
    ([3000, 70, 0], 8, 16, 4, 128, BF16),             # 32 stacked rows, short and empty prefixes
    ([1000, 4097], 6, 16, 2, 64, FP8),                # fp8, D = 64, 48 stacked rows
    ([2500, 63], 16, 8, 2, 128, FP8),                 # fp8, 64 stacked rows, 16-token draft
])
def test_verify_edge_cases(gpu_lib, prefix_lens, lx, hq, hkv, d, kvdt):
    n_pages = int(sum((x + 15) // 16 for x in prefix_lens)) + 7
    inst = make_paged(prefix_lens, lx, hq, hkv, d, kv_dtype=kvdt, seed=sum(prefix_lens) % 1000,
                      num_pages=n_pages, scales=(kvdt == FP8))
    _paged_check(gpu_lib, inst, label=f"verify {prefix_lens} Lx={lx} {hq}/{hkv} D={d}")


# Spike keys dominate every query that sees them by more than 128 ln 2, at
# positions spread over tiles, stages and lane groups: a row maximum that
# missed any lane's scores would overflow the softmax weights here.
@pytest.mark.parametrize("d", [64, 128, 256])
def test_flat_spike_keys(gpu_lib, d):
    inst = make_flat_spikes(300, [130, 70], 8, 2, d, spikes=[3, 21, 40, 62, 104, 126, 190, 250, 317, 345, 439],
                            seed=40 + d)
    _flat_check(gpu_lib, inst, label=f"flat spikes D={d}")


@pytest.mark.parametrize("lx,hq,hkv,d,kvdt", [
    (4, 8, 2, 128, BF16),    # 16 stacked rows
    (2, 8, 2, 256, FP8),     # 8 stacked rows, fp8
    (8, 16, 2, 128, BF16),   # 64 stacked rows
    (8, 8, 2, 256, FP8),     # 32 stacked rows, fp8
])
def test_verify_spike_keys(gpu_lib, lx, hq, hkv, d, kvdt):
    spikes = [5, 18, 31, 37, 58, 63, 700, 1023, 1500, 2047]
    inst = make_paged_spikes([2100, 900, 40], lx, hq, hkv, d, spikes=spikes, kv_dtype=kvdt, seed=50 + d,
                             num_pages=200)
    _paged_check(gpu_lib, inst, label=f"verify spikes Lx={lx} {hq}/{hkv} D={d}")


def test_verify_workspace_reused_across_calls(gpu_lib):
    """One workspace serves a series of calls of different shapes, split
    counts and kernels (register streaming, wide, fp8): nothing a call leaves
    in it may leak into the next result."""
    import torch

    def mk(plens, lx, hq, hkv, d, kvdt, seed):
        n_pages = int(sum((x + 15) // 16 for x in plens)) + 5
        return make_paged(plens, lx, hq, hkv, d, kv_dtype=kvdt, seed=seed, num_pages=n_pages,
                          scales=(kvdt == FP8))

    cases = [mk([1500] * 8, 4, 8, 4, 128, BF16, 61),
             mk([3000, 70, 0], 8, 16, 4, 128, BF16, 62),
             mk([900, 2000, 40, 600] * 4, 4, 16, 8, 128, FP8, 63),
             mk([5000, 33], 2, 8, 2, 256, FP8, 64),
             mk([1200, 800] * 6, 4, 4, 4, 64, BF16, 65),
             mk([1500] * 8, 4, 8, 4, 128, BF16, 66)]
    sizes = []
    for inst in cases:
        desc = gpu_lib.paged_desc(len(inst.prefix_lens), inst.draft_len, 16, inst.k_pool.shape[0], 1, 1, 1,
                                  inst.max_prefix_len, 1, 1)
        sizes.append(gpu_lib.psattn_workspace_size(desc, inst.hq, inst.hkv, inst.d, inst.q_dtype,
                                                   inst.kv_dtype))
    ws = torch.full((max(sizes),), 0x7F, dtype=torch.uint8, device="cuda")  # non-zero start
    for inst in cases:
        o, lse = run_paged(gpu_lib, inst, workspace=ws)
        ro, rl = attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr, inst.kv_indices,
                            inst.prefix_lens, inst.k_ext, inst.v_ext, inst.draft_len, inst.sm_scale,
                            k_scale=inst.k_scale, v_scale=inst.v_scale, q_dtype=inst.q_dtype,
                            kv_dtype=inst.kv_dtype, page_size=inst.page_size)
        compare(to_f64(o), to_f64(lse), ro, rl, kind_of(inst.q_dtype, inst.kv_dtype),
                f"reused workspace {list(inst.prefix_lens)[:4]} Lx={inst.draft_len} D={inst.d}")


@pytest.mark.parametrize("lx,hq,hkv,d,kvdt", [
    (4, 16, 4, 128, BF16),   # 16 stacked rows: the register split pass
    (8, 16, 2, 256, FP8),    # 64 stacked rows, fp8: the wide split pass
])
def test_verify_graph_replays(gpu_lib, lx, hq, hkv, d, kvdt):
    """A captured verify call (split pass and merge) replays to the eager
    result: three replays, each after an eager call with other inputs on the
    same workspace and then once more straight after, equal the eager call on
    the same inputs bit for bit."""
    import torch

    plens = [1500, 2300, 40, 800] * 2
    inst = make_paged(plens, lx, hq, hkv, d, kv_dtype=kvdt, seed=68, num_pages=600, scales=kvdt == FP8)
    other = make_paged(plens, lx, hq, hkv, d, kv_dtype=kvdt, seed=69, num_pages=600, scales=kvdt == FP8)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    def args_of(x):
        return (to_dev(x.q, x.q_dtype), to_dev(x.k_pool, x.kv_dtype), to_dev(x.v_pool, x.kv_dtype),
                i32(x.kv_indptr), i32(x.kv_indices), i32(x.prefix_lens), to_dev(x.k_ext, x.kv_dtype),
                to_dev(x.v_ext, x.kv_dtype), x.draft_len, x.max_prefix_len)

    a1, a2 = args_of(inst), args_of(other)
    kw = dict(sm_scale=inst.sm_scale, kv_dtype=kvdt, k_scale=inst.k_scale, v_scale=inst.v_scale)
    desc = gpu_lib.paged_desc(inst.batch, lx, 16, inst.num_pages, 1, 1, 1, inst.max_prefix_len, 1, 1)
    ws = torch.full((gpu_lib.psattn_workspace_size(desc, hq, hkv, d, BF16, kvdt),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    o_e, l_e = gpu_lib.fwd_paged(*a1, **kw, workspace=ws)
    torch.cuda.synchronize()
    compare(to_f64(o_e), to_f64(l_e), *attn_paged(inst.q, inst.k_pool, inst.v_pool, inst.kv_indptr,
                                                  inst.kv_indices, inst.prefix_lens, inst.k_ext, inst.v_ext,
                                                  inst.draft_len, inst.sm_scale, k_scale=inst.k_scale,
                                                  v_scale=inst.v_scale, q_dtype=BF16, kv_dtype=kvdt),
            kind_of(BF16, kvdt), f"graph replay case Lx={lx} D={d}, eager")
    o_g, l_g = torch.empty_like(o_e), torch.empty_like(l_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gpu_lib.fwd_paged(*a1, **kw, out=o_g, lse=l_g, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        gpu_lib.fwd_paged(*a2, **kw, workspace=ws)  # other partials left in the workspace
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {rep} differs from the eager call"
        graph.replay()  # straight after a replay
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"second replay {rep} differs"


def test_verify_zero_queries_closed_form(gpu_lib):
    inst = make_paged([100, 0, 63], 4, 8, 2, 128, kv_dtype=BF16, seed=7, num_pages=20)
    inst.q[:] = 0
    o, lse = run_paged(gpu_lib, inst)
    l64 = to_f64(lse)
    for b, pl in enumerate(inst.prefix_lens):
        for t in range(4):
            assert np.allclose(l64[b * 4 + t], math.log(int(pl) + t + 1), atol=1e-5)


# --------------------------------------------------------------------------- planner on device
def _dump(gpu_lib, desc, hq, hkv, d, qdt, kvdt):
    import torch

    ps = gpu_lib
    info = ps.PsattnPlanInfo()
    ps.check(ps.psattn_plan_dump(desc, hq, hkv, d, qdt, kvdt, 0, 0, info, 0))
    buf = torch.full((max(info.n_items, 1) * ps.ITEM_FIELDS,), -7, dtype=torch.int32, device="cuda")
    ps.check(ps.psattn_plan_dump(desc, hq, hkv, d, qdt, kvdt, buf.data_ptr(), info.n_items, info,
                                 torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return info, buf.cpu().numpy().reshape(-1, ps.ITEM_FIELDS)[:info.n_items]


@pytest.mark.parametrize("name", ["tiny", "grpo", "grpo_ragged"])
def test_device_planner_bit_exact_flat(gpu_lib, name):
    import torch
    from oracle.plan import enumerate_flat

    inst = make_config(name)
    seg = torch.from_numpy(inst.seg_offsets).cuda()
    desc = gpu_lib.flat_desc(inst.total_tokens, inst.prefix_len, inst.num_segments, seg.data_ptr(),
                             inst.max_seg_len)
    info, items = _dump(gpu_lib, desc, inst.hq, inst.hkv, inst.d, inst.dtype, inst.dtype)
    assert np.array_equal(items, enumerate_flat(inst.prefix_len, inst.seg_offsets, inst.hkv, info.tile_tokens))


@pytest.mark.parametrize("prefix_lens,lx,hq,hkv,d", [([16384] * 8, 4, 32, 8, 128), ([100, 0, 37], 3, 8, 2, 64)])
def test_device_planner_bit_exact_paged(gpu_lib, prefix_lens, lx, hq, hkv, d):
    import torch
    from oracle.plan import enumerate_paged

    pl = torch.tensor(prefix_lens, dtype=torch.int32, device="cuda")
    dummy = torch.zeros(4, dtype=torch.int32, device="cuda")
    n_pages = sum((x + 15) // 16 for x in prefix_lens) + 1
    desc = gpu_lib.paged_desc(len(prefix_lens), lx, 16, n_pages, pl.data_ptr(), dummy.data_ptr(),
                              dummy.data_ptr(), max(prefix_lens), dummy.data_ptr(), dummy.data_ptr())
    info, items = _dump(gpu_lib, desc, hq, hkv, d, BF16, BF16)
    assert np.array_equal(items, enumerate_paged(prefix_lens, hkv, lx, info.n_splits, info.split_len))
