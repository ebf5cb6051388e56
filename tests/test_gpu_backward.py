"""GPU parity of the flat backward (psattn_bwd) against the float64 oracle.

The forward runs on the GPU first (its bf16 O and fp32 LSE are the backward's
inputs, as in training); the oracle differentiates the exact definition from
the same stored bf16 Q, K, V and dO.  Errors are relative to the reference's
scale: max |g - r| / max |r| and mean |g - r| / mean |r| per gradient.
"""
import numpy as np
import pytest

from gpu_util import guarded_empty, guards_intact, to_dev, to_f64
from oracle.backward import attn_flat_bwd
from psattn_inputs import BF16, f32_to_bf16_bits, make_flat

pytestmark = pytest.mark.gpu

# bf16 P and dS enter the MFMAs, the outputs are rounded to bf16, and delta is
# formed from the bf16 forward output: each a relative 2^-9 per element
TOL_MAX_REL = 2e-2
TOL_MEAN_REL = 5e-3


def _dout(inst, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(inst.q.shape).astype(np.float32))


def _run(ps, inst, do_bits, ws_fill=None, repeat=1, max_seg_len=None):
    import torch

    msl = inst.max_seg_len if max_seg_len is None else max_seg_len

    q = to_dev(inst.q, BF16)
    k = to_dev(inst.k, BF16)
    v = to_dev(inst.v, BF16)
    seg = torch.from_numpy(inst.seg_offsets.astype(np.int32)).cuda() if inst.num_segments > 0 else None
    o, lse = ps.fwd_flat(q, k, v, inst.prefix_len, seg, msl, sm_scale=inst.sm_scale)
    do = to_dev(do_bits, BF16)
    dq, dqf = guarded_empty(q.shape, torch.bfloat16)
    dk, dkf = guarded_empty(k.shape, torch.bfloat16)
    dv, dvf = guarded_empty(v.shape, torch.bfloat16)
    ws = None
    if ws_fill is not None:
        n = int(inst.num_segments)
        desc = ps.flat_desc(inst.total_tokens, inst.prefix_len, n, 0 if seg is None else seg.data_ptr(), msl)
        nb = ps.psattn_bwd_workspace_size(desc, inst.hq, inst.hkv, inst.d, BF16)
        ws = torch.full((nb,), ws_fill, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(repeat):
        ps.bwd_flat(q, k, v, o, lse, do, inst.prefix_len, seg, msl, sm_scale=inst.sm_scale,
                    dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        outs.append((dq.clone(), dk.clone(), dv.clone()))
    assert guards_intact(dqf) and guards_intact(dkf) and guards_intact(dvf), "write outside an output"
    return outs


def _check(ps, inst, seed=7, label="", max_seg_len=None):
    do_bits = _dout(inst, seed)
    (dq, dk, dv), = _run(ps, inst, do_bits, max_seg_len=max_seg_len)
    ref = attn_flat_bwd(inst.q, inst.k, inst.v, do_bits, inst.prefix_len, inst.seg_offsets, inst.sm_scale,
                        dtype=BF16)
    errs = {}
    if inst.total_tokens == 0:
        return
    # a gradient can vanish exactly (one visible key: P = 1, so dQ = dK = 0);
    # its scale is then floored at 1% of the largest gradient's
    top_max = max(np.max(np.abs(r)) for r in ref)
    top_mean = max(np.mean(np.abs(r)) for r in ref)
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        g = to_f64(g)
        assert np.all(np.isfinite(g)), name
        dmax = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-2 * top_max)
        dmean = np.mean(np.abs(g - r)) / max(np.mean(np.abs(r)), 1e-2 * top_mean)
        errs[name] = (float(dmax), float(dmean))
    print(f"[bwd parity] {label or inst.name}: " + ", ".join(f"{n} max {a:.2e} mean {b:.2e}" for n, (a, b) in errs.items()),
          flush=True)
    for name, (dmax, dmean) in errs.items():
        assert dmax <= TOL_MAX_REL and dmean <= TOL_MEAN_REL, (name, dmax, dmean)


@pytest.mark.parametrize("p,lens,hq,hkv", [
    (100, [37], 8, 2),              # N = 1
    (0, [33, 5, 70], 8, 2),         # no prefix
    (64, [1, 1, 1, 1], 4, 4),       # one-token rollouts, G = 1
    (50, [0, 20, 0, 9], 16, 4),     # empty rollouts
    (130, [3, 200], 12, 4),         # G = 3: 21-token row tiles, every tile masked
    (77, [19, 64], 64, 1),          # G = 64: one token per row tile
    (1, [], 2, 1),                  # a one-token prefix only
    (0, [1], 1, 1),                 # a single token in total
    (600, [700, 513], 8, 2),        # rows of a key tile span several 512-token chunks
    (300, [200, 128, 1, 77], 32, 8),  # GRPO head layout, small
])
def test_bwd_small_full(gpu_lib, p, lens, hq, hkv):
    inst = make_flat(p, lens, hq, hkv, 128, dtype=BF16, seed=p + len(lens) + hq)
    _check(gpu_lib, inst, label=f"P={p} lens={lens} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("p,lens,hq,hkv", [
    (100, [37], 8, 2),              # N = 1
    (0, [33, 5, 70], 8, 2),         # no prefix
    (130, [3, 200], 12, 4),         # G = 3: every row tile masked
    (600, [700, 513], 8, 2),        # rows of a key tile span several 512-token chunks
    (300, [200, 128, 1, 77], 32, 8),  # GRPO head layout, small
])
@pytest.mark.parametrize("d", [64, 256])
def test_bwd_head_dims_64_and_256(gpu_lib, p, lens, hq, hkv, d):
    inst = make_flat(p, lens, hq, hkv, d, dtype=BF16, seed=p + len(lens) + hq + d)
    _check(gpu_lib, inst, label=f"D={d} P={p} lens={lens} hq={hq} hkv={hkv}")


def test_bwd_grpo_block(gpu_lib):
    # the GRPO head layout at a quarter of its length
    inst = make_flat(512, [128] * 8, 32, 8, 128, dtype=BF16, seed=41, name="grpo_quarter")
    _check(gpu_lib, inst)


def test_bwd_grpo_fullsize_sampled(gpu_lib):
    # the full GRPO shape in the benchmark's launch configuration; dQ rows and
    # dK / dV rows sampled at the prefix and rollout boundaries, at tile edges
    # and at seeded random positions
    from psattn_inputs import make_config

    inst = make_config("grpo")
    do_bits = _dout(inst, 7)
    (dq, dk, dv), = _run(gpu_lib, inst, do_bits)
    t, p = inst.total_tokens, inst.prefix_len
    rng = np.random.default_rng(9)
    edges = [0, 1, 63, 64, 127, 128, p - 1, p, p + 1, p + 511, p + 512, t - 1]
    rows = np.unique(np.concatenate([edges, rng.choice(t, 8, replace=False)]))
    keys = np.unique(np.concatenate([edges, rng.choice(t, 6, replace=False)]))
    ref = attn_flat_bwd(inst.q, inst.k, inst.v, do_bits, p, inst.seg_offsets, inst.sm_scale, dtype=BF16,
                        rows=rows, keys=keys)
    got = (to_f64(dq)[rows], to_f64(dk)[keys], to_f64(dv)[keys])
    top_max = max(np.max(np.abs(r)) for r in ref)
    top_mean = max(np.mean(np.abs(r)) for r in ref)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(g)), name
        dmax = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-2 * top_max)
        dmean = np.mean(np.abs(g - r)) / max(np.mean(np.abs(r)), 1e-2 * top_mean)
        print(f"[bwd parity] grpo sampled {name}: max {dmax:.2e} mean {dmean:.2e}", flush=True)
        assert dmax <= TOL_MAX_REL and dmean <= TOL_MEAN_REL, (name, dmax, dmean)


def test_bwd_workspace_contents_do_not_matter_and_dq_is_deterministic(gpu_lib):
    inst = make_flat(200, [90, 140, 33], 16, 4, 128, dtype=BF16, seed=43)
    do_bits = _dout(inst, 3)
    a = _run(gpu_lib, inst, do_bits, ws_fill=0x7F, repeat=2)
    b = _run(gpu_lib, inst, do_bits, ws_fill=0x00)
    import torch

    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][0], b[0][0]), "dQ must not depend on the call"
    for j in (1, 2):  # dK, dV sum partials with atomics: equal up to the order of the additions
        x, y = to_f64(a[0][j]), to_f64(b[0][j])
        assert np.max(np.abs(x - y)) <= 1e-2 * max(np.max(np.abs(y)), 1e-30)


@pytest.mark.parametrize("p,lens,msl", [
    (100, [1000, 24], 512),           # passes the host check (2 x 512 >= 1024), true longest 1000
    (64, [2000, 10, 10, 10], 508),    # 4 x 508 >= 2030, true longest 2000
])
def test_bwd_underestimated_max_seg_len(gpu_lib, p, lens, msl):
    """max_seg_len below the longest rollout still passes the host check
    (N * max_seg_len >= T - P); the dK/dV launch sized from it walks the
    surplus items, so the gradients stay exact."""
    assert len(lens) * msl >= sum(lens) and max(lens) > msl
    inst = make_flat(p, lens, 8, 2, 128, dtype=BF16, seed=p + sum(lens))
    _check(gpu_lib, inst, label=f"P={p} lens={lens} max_seg_len={msl}", max_seg_len=msl)
