"""GPU parity of the multi-level backward (psattn_bwd with seg_parent)
against the float64 oracle's tree expansion (attn_flat_tree_bwd).

The forward runs on the GPU first (its bf16 O and fp32 LSE are the
backward's inputs); the oracle differentiates the tree definition from the
same stored bf16 Q, K, V and dO.  A segment's keys collect gradient from its
own later rows and from every row of each descendant; dQ of a row walks the
prefix, its own segment and every ancestor segment.  Shapes cover chains
with ancestors shorter than a key tile, empty segments in a chain, deep
chains, sibling subtrees, GQA groups 1 to 64, a seeded forest, the GRPO head
layout with two shared continuations at full size (sampled rows and keys),
and a max_seg_len below the longest segment.
"""
import numpy as np
import pytest

from gpu_util import guarded_empty, guards_intact, to_dev, to_f64
from oracle.backward import attn_flat_tree_bwd
from psattn_inputs import BF16, f32_to_bf16_bits, make_flat, make_seg_parents

pytestmark = pytest.mark.gpu

# as for the one-level backward: bf16 P and dS in the products, bf16 outputs
TOL_MAX_REL = 2e-2
TOL_MEAN_REL = 5e-3


def _dout(inst, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(inst.q.shape).astype(np.float32))


def _run(ps, inst, parents, do_bits, max_seg_len=None):
    import torch

    msl = inst.max_seg_len if max_seg_len is None else max_seg_len
    q, k, v = to_dev(inst.q, BF16), to_dev(inst.k, BF16), to_dev(inst.v, BF16)
    seg = torch.from_numpy(inst.seg_offsets.astype(np.int32)).cuda()
    par = torch.from_numpy(np.asarray(parents, dtype=np.int32)).cuda()
    o, lse = ps.fwd_flat(q, k, v, inst.prefix_len, seg, msl, sm_scale=inst.sm_scale, seg_parent=par)
    do = to_dev(do_bits, BF16)
    dq, dqf = guarded_empty(q.shape, torch.bfloat16)
    dk, dkf = guarded_empty(k.shape, torch.bfloat16)
    dv, dvf = guarded_empty(v.shape, torch.bfloat16)
    ps.bwd_flat(q, k, v, o, lse, do, inst.prefix_len, seg, msl, sm_scale=inst.sm_scale, dq=dq, dk=dk, dv=dv,
                seg_parent=par)
    torch.cuda.synchronize()
    assert guards_intact(dqf) and guards_intact(dkf) and guards_intact(dvf), "write outside an output"
    return to_f64(dq), to_f64(dk), to_f64(dv)


def _compare(got, ref, label):
    top_max = max(np.max(np.abs(r)) for r in ref)
    top_mean = max(np.mean(np.abs(r)) for r in ref)
    errs = {}
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), name
        dmax = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-2 * top_max)
        dmean = np.mean(np.abs(g - r)) / max(np.mean(np.abs(r)), 1e-2 * top_mean)
        errs[name] = (float(dmax), float(dmean))
    print(f"[tree bwd parity] {label}: " + ", ".join(f"{n} max {a:.2e} mean {b:.2e}" for n, (a, b) in errs.items()),
          flush=True)
    for name, (dmax, dmean) in errs.items():
        assert dmax <= TOL_MAX_REL and dmean <= TOL_MEAN_REL, (name, dmax, dmean)


def _check(ps, inst, parents, label, seed=7, max_seg_len=None):
    do_bits = _dout(inst, seed)
    got = _run(ps, inst, parents, do_bits, max_seg_len=max_seg_len)
    ref = attn_flat_tree_bwd(inst.q, inst.k, inst.v, do_bits, inst.prefix_len, inst.seg_offsets, parents,
                             inst.sm_scale, dtype=BF16)
    _compare(got, ref, label)


@pytest.mark.parametrize("p,lens,parents,hq,hkv", [
    (100, [37, 50, 9], [-1, 0, 1], 8, 2),               # a chain of three, short ragged tiles
    (64, [5, 3, 70, 1, 2], [-1, 0, 1, 2, 3], 4, 1),      # a deep chain, ancestors under one key tile
    (130, [64, 0, 100, 33], [-1, 0, 1, 1], 12, 4),       # an empty ancestor; G = 3 (every row tile masked)
    (0, [40, 70, 20], [-1, 0, 0], 8, 2),                 # no prefix: the root segment plays its part
    (300, [200, 128, 1, 77], [-1, 0, 0, 2], 32, 8),      # GRPO head layout, small
    (77, [19, 64, 90], [-1, 0, 1], 64, 1),               # G = 64
    (200, [300, 150, 700], [-1, 0, 0], 8, 2),            # a key tile's descendant rows span 512-token chunks
])
def test_tree_bwd_small_full(gpu_lib, p, lens, parents, hq, hkv):
    inst = make_flat(p, lens, hq, hkv, 128, dtype=BF16, seed=p + len(lens) + hq)
    _check(gpu_lib, inst, parents, f"P={p} lens={lens} parents={parents} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("seed", [1, 2])
def test_tree_bwd_seeded_forest(gpu_lib, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 200, size=10).tolist()
    parents = make_seg_parents(10, seed)
    inst = make_flat(256, lens, 16, 4, 128, dtype=BF16, seed=200 + seed)
    _check(gpu_lib, inst, parents, f"forest seed={seed} parents={parents.tolist()}")


@pytest.mark.parametrize("d", [64, 256])
def test_tree_bwd_head_dims_64_and_256(gpu_lib, d):
    inst = make_flat(90, [33, 65, 70, 20], 8, 2, d, dtype=BF16, seed=d)
    _check(gpu_lib, inst, [-1, 0, 1, 0], f"D={d} chain")


def test_tree_bwd_all_roots_is_one_level(gpu_lib):
    inst = make_flat(200, [90, 140, 33], 16, 4, 128, dtype=BF16, seed=5)
    _check(gpu_lib, inst, [-1, -1, -1], "all roots")


def test_tree_bwd_underestimated_max_seg_len(gpu_lib):
    # max_seg_len below the longest segment passes the host check; the dK/dV
    # items past the launch the bound sizes are walked by the second launch
    lens, parents, msl = [1000, 24, 300], [-1, 0, 0], 448
    assert len(lens) * msl >= sum(lens) and max(lens) > msl
    inst = make_flat(100, lens, 8, 2, 128, dtype=BF16, seed=17)
    _check(gpu_lib, inst, parents, f"lens={lens} max_seg_len={msl}", max_seg_len=msl)


def test_tree_bwd_grpo_two_level_fullsize_sampled(gpu_lib):
    # the GRPO shape (P = 2048, Hq 32 / Hkv 8, D 128) with two shared
    # 512-token continuations, each continued by three 512-token rollouts;
    # dQ rows and dK / dV rows sampled at segment boundaries, tile edges and
    # seeded random positions
    lens = [512] * 8
    parents = [-1, -1, 0, 0, 0, 1, 1, 1]
    inst = make_flat(2048, lens, 32, 8, 128, dtype=BF16, seed=77)
    do_bits = _dout(inst, 8)
    dq, dk, dv = _run(gpu_lib, inst, parents, do_bits)
    rng = np.random.default_rng(4)
    offs = inst.seg_offsets
    edges = {0, 1, 63, 64, 2047}
    for a, b in zip(offs[:-1], offs[1:]):
        edges.update({int(a), int(a) + 1, int(a) + 127, int(a) + 128, int(b) - 1})
    rows = np.array(sorted(edges | {int(x) for x in rng.integers(0, inst.total_tokens, size=8)}))
    keys = np.array(sorted(edges | {int(x) for x in rng.integers(0, inst.total_tokens, size=6)}))
    ref = attn_flat_tree_bwd(inst.q, inst.k, inst.v, do_bits, inst.prefix_len, offs, parents, inst.sm_scale,
                             dtype=BF16, rows=rows, keys=keys)
    _compare((dq[rows], dk[keys], dv[keys]), ref, "grpo two-level sampled")
