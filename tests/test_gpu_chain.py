"""GPU parity of multi-level prefix sharing (psattn_desc.seg_parent) against
the float64 oracle's tree expansion (attn_flat_tree).

Every segment's rows see the prefix, all tokens of each ancestor segment and
their own segment causally.  Shapes cover ancestors shorter than one key tile,
ragged ancestor ends, empty segments in a chain, deep chains, the GRPO head
layout, and head dims 64 / 128 / 256.
"""
import numpy as np
import pytest

from gpu_util import compare, guarded_empty, guards_intact, to_dev, to_f64
from oracle.attention import attn_flat, attn_flat_tree
from psattn_inputs import BF16, make_flat, make_seg_parents

pytestmark = pytest.mark.gpu


def _run(ps, inst, parents):
    import torch

    q = to_dev(inst.q, BF16)
    k = to_dev(inst.k, BF16)
    v = to_dev(inst.v, BF16)
    seg = torch.from_numpy(inst.seg_offsets.astype(np.int32)).cuda()
    par = torch.from_numpy(np.asarray(parents, dtype=np.int32)).cuda()
    o, of = guarded_empty(q.shape, q.dtype)
    lse, lf = guarded_empty((q.shape[0], q.shape[1]), torch.float32)
    ps.fwd_flat(q, k, v, inst.prefix_len, seg, inst.max_seg_len, sm_scale=inst.sm_scale, out=o, lse=lse,
                seg_parent=par)
    torch.cuda.synchronize()
    assert guards_intact(of) and guards_intact(lf), "write outside the output tensors"
    return to_f64(o), to_f64(lse)


def _check(ps, inst, parents, label):
    o, lse = _run(ps, inst, parents)
    ro, rl = attn_flat_tree(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, parents, inst.sm_scale,
                            dtype=BF16)
    return compare(o, lse, ro, rl, "bf16", label)


@pytest.mark.parametrize("p,lens,parents,hq,hkv,d", [
    (100, [37, 50, 9], [-1, 0, 1], 8, 2, 128),                  # a chain of three, short ragged tiles
    (64, [5, 3, 70, 1, 2], [-1, 0, 1, 2, 3], 4, 1, 128),         # a deep chain, ancestors under one tile
    (130, [64, 0, 100, 33], [-1, 0, 1, 1], 12, 4, 128),          # an empty ancestor; G = 3
    (0, [40, 70, 20], [-1, 0, 0], 8, 2, 128),                    # no prefix: the root segment is the prefix
    (300, [200, 128, 1, 77], [-1, 0, 0, 2], 32, 8, 128),         # GRPO head layout, small
    (77, [19, 64, 90], [-1, 0, 1], 64, 1, 128),                  # G = 64
    (90, [33, 65, 70], [-1, 0, 1], 8, 2, 64),                    # head dim 64
    (90, [33, 65, 70], [-1, 0, 1], 8, 2, 256),                   # head dim 256
])
def test_chain_small_full(gpu_lib, p, lens, parents, hq, hkv, d):
    inst = make_flat(p, lens, hq, hkv, d, dtype=BF16, seed=p + len(lens) + d)
    _check(gpu_lib, inst, parents, f"P={p} lens={lens} parents={parents} hq={hq} hkv={hkv} d={d}")


@pytest.mark.parametrize("seed", [1, 2])
def test_chain_seeded_forest(gpu_lib, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 300, size=12).tolist()
    parents = make_seg_parents(12, seed)
    inst = make_flat(512, lens, 32, 8, 128, dtype=BF16, seed=100 + seed)
    _check(gpu_lib, inst, parents, f"forest seed={seed} parents={parents.tolist()}")


def test_all_roots_equal_one_level(gpu_lib):
    # every parent -1 takes the multi-level kernel through the one-level case
    inst = make_flat(200, [90, 140, 33], 16, 4, 128, dtype=BF16, seed=5)
    o, lse = _run(gpu_lib, inst, [-1, -1, -1])
    ro, rl = attn_flat(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, inst.sm_scale, dtype=BF16)
    compare(o, lse, ro, rl, "bf16", "all roots")


def test_malformed_parent_ends_the_walk(gpu_lib):
    # an entry outside [-1, i) stops the ancestor walk: segment 1 (parent 1,
    # itself) and segment 2 (parent 5, past the end) are read as one-level,
    # and nothing outside the outputs is written
    inst = make_flat(64, [30, 20, 10], 8, 2, 128, dtype=BF16, seed=6)
    o, lse = _run(gpu_lib, inst, [-1, 1, 5])
    ro, rl = attn_flat_tree(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, [-1, -1, -1],
                            inst.sm_scale, dtype=BF16)
    compare(o, lse, ro, rl, "bf16", "malformed parents")


def test_grpo_two_level_fullsize_sampled(gpu_lib):
    # the GRPO shape (P = 2048, Hq 32 / Hkv 8, D 128) with two shared
    # 512-token continuations, each continued by three 512-token rollouts
    lens = [512] * 8
    parents = [-1, -1, 0, 0, 0, 1, 1, 1]
    inst = make_flat(2048, lens, 32, 8, 128, dtype=BF16, seed=77)
    o, lse = _run(gpu_lib, inst, parents)
    rng = np.random.default_rng(3)
    offs = inst.seg_offsets
    rows = {0, 2047}
    for a, b in zip(offs[:-1], offs[1:]):
        rows.update({int(a), int(a) + 1, int(a) + 63, int(a) + 64, int(b) - 1})
    rows.update(int(x) for x in rng.integers(0, inst.total_tokens, size=24))
    rows = np.array(sorted(rows))
    ro, rl = attn_flat_tree(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, parents, inst.sm_scale,
                            dtype=BF16)
    compare(o[rows], lse[rows], ro[rows], rl[rows], "bf16", "grpo two-level sampled")
