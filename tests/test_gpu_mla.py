"""GPU parity of the sparse shared-latent MLA forward (psattn_mla_fwd)
against the float64 oracle (oracle.mla.mla_sparse).

Cases: lists shorter than one tile, ragged tails, scattered padding,
duplicate and out-of-range entries, empty lists, sinks, a latent cache whose
rows are wider than the 512 values used, 32 / 64 / 128 heads, the largest list
(2048 entries), and the DSA prefill shape (16384 tokens, 64 heads, top-2048)
on sampled tokens in the benchmark's launch configuration.
"""
import numpy as np
import pytest

from gpu_util import compare, guarded_empty, guards_intact, to_f64
from oracle.mla import mla_sparse
from psattn_inputs import BF16, make_mla

pytestmark = pytest.mark.gpu


def _dev(inst, kv_stride=None):
    import torch

    q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
    c = inst.ckv
    if kv_stride is not None and kv_stride != c.shape[1]:
        wide = np.zeros((c.shape[0], kv_stride), dtype=np.uint16)
        wide[:, :c.shape[1]] = c
        wide[:, c.shape[1]:] = 0x7FC0  # NaN in the unused part of a row
        c = wide
    ckv = torch.from_numpy(np.ascontiguousarray(c).view(np.int16)).view(torch.bfloat16).cuda()
    idx = torch.from_numpy(np.ascontiguousarray(inst.indices, dtype=np.int32)).cuda()
    sink = None if inst.sink is None else torch.from_numpy(inst.sink.astype(np.float32)).cuda()
    return q, ckv, idx, sink


def _run(ps, inst, kv_stride=None):
    import torch

    q, ckv, idx, sink = _dev(inst, kv_stride)
    o, of = guarded_empty(q.shape, torch.bfloat16)
    lse, lf = guarded_empty(q.shape[:2], torch.float32)
    ps.fwd_mla(q, ckv, idx, sm_scale=inst.sm_scale, sink=sink, out=o, lse=lse)
    torch.cuda.synchronize()
    assert guards_intact(of) and guards_intact(lf), "write outside the outputs"
    return o, lse


def _check(ps, inst, label, tokens=None, kv_stride=None):
    o, lse = _run(ps, inst, kv_stride)
    ro, rl = mla_sparse(inst.q, inst.ckv, inst.indices, inst.sm_scale, sink=inst.sink, dtype=BF16, tokens=tokens)
    go, gl = to_f64(o), to_f64(lse)
    if tokens is not None:
        go, gl = go[tokens], gl[tokens]
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{label}: -inf LSE rows differ"
    assert np.all(go[empty] == 0), f"{label}: rows without keys must be zero"
    gl = np.where(empty, 0.0, gl)
    rl = np.where(empty, 0.0, rl)
    return compare(go, gl, ro, rl, "bf16", label)


@pytest.mark.parametrize("t,h,topk,sink,scatter", [
    (40, 64, 16, False, False),     # lists shorter than one 32-key tile
    (300, 64, 64, False, False),    # two tiles per token once t >= 63
    (300, 64, 50, True, True),      # ragged tail tile, scattered padding, sinks
    (200, 32, 96, False, True),     # 32 heads
    (150, 128, 40, True, False),    # 128 heads
    (64, 64, 1, False, False),      # one entry per token
])
def test_mla_small_full(gpu_lib, t, h, topk, sink, scatter):
    inst = make_mla(t, h, 512, topk, seed=t + h + topk, sink=sink, scatter_pad=scatter)
    _check(gpu_lib, inst, f"T={t} H={h} topk={topk} sink={sink} scatter={scatter}")


def test_mla_duplicates_out_of_range_and_empty_lists(gpu_lib):
    inst = make_mla(48, 64, 512, 40, seed=3, sink=False, num_kv=70)
    rng = np.random.default_rng(5)
    idx = inst.indices
    idx[:, 5] = idx[:, 4]                                 # a duplicate counts twice
    idx[::3, 7] = 70 + rng.integers(0, 1000, size=idx[::3].shape[0])  # past the cache: skipped
    idx[::5, 9] = -7
    idx[10] = -1                                          # no key at all
    idx[11] = np.array([3] * 40)                          # one row listed 40 times
    _check(gpu_lib, inst, "duplicates / out of range / empty")


def test_mla_empty_lists_with_sinks(gpu_lib):
    inst = make_mla(20, 64, 512, 32, seed=4, sink=True)
    inst.indices[:] = -1
    inst.indices[3, :5] = [0, 1, 2, 3, 3]
    _check(gpu_lib, inst, "empty lists with sinks")


def test_mla_wide_cache_rows(gpu_lib):
    # latent rows of 576 values (a rope part after the 512 used): the extra
    # values are NaN and must not be read
    inst = make_mla(100, 64, 512, 48, seed=6, sink=True, scatter_pad=True)
    _check(gpu_lib, inst, "kv_stride 576", kv_stride=576)


def test_mla_largest_list_sampled(gpu_lib):
    # 2048-entry lists (the largest staged in LDS) over a 3000-row cache
    inst = make_mla(64, 64, 512, 2048, seed=7, num_kv=3000, scatter_pad=True)
    _check(gpu_lib, inst, "topk 2048 sampled", tokens=[0, 1, 17, 40, 63])


def test_mla_deterministic(gpu_lib):
    import torch

    inst = make_mla(120, 64, 512, 80, seed=8, sink=True)
    a = _run(gpu_lib, inst)
    b = _run(gpu_lib, inst)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_mla_dsa_fullsize_sampled(gpu_lib):
    # the DSA prefill shape: 16384 tokens, 64 heads, top-2048 lists
    from psattn_inputs import make_config

    inst = make_config("mla_dsa")
    rng = np.random.default_rng(11)
    tokens = sorted({0, 1, 31, 32, 33, 2046, 2047, 2048, 8191, 16383} |
                    {int(x) for x in rng.integers(0, inst.num_tokens, size=10)})
    _check(gpu_lib, inst, "mla_dsa sampled", tokens=tokens)


def test_mla_empty_cache(gpu_lib):
    # no cached rows: every entry is out of range, every token has no key
    import torch

    inst = make_mla(16, 64, 512, 8, seed=9, sink=True)
    q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
    ckv = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(inst.indices).cuda()
    sink = torch.from_numpy(inst.sink.astype(np.float32)).cuda()
    o, lse = gpu_lib.fwd_mla(q, ckv, idx, sm_scale=inst.sm_scale, sink=sink)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert np.allclose(to_f64(lse), np.broadcast_to(inst.sink.astype(np.float64), (16, 64)), rtol=0, atol=1e-6)


def test_mla_zero_length_lists(gpu_lib):
    # topk = 0: no entries at all; without sinks every row is zero with LSE -inf
    import torch

    inst = make_mla(12, 32, 512, 4, seed=10)
    q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
    ckv = torch.from_numpy(inst.ckv.view(np.int16)).view(torch.bfloat16).cuda()
    idx = torch.empty((12, 0), dtype=torch.int32, device="cuda")
    o, lse = gpu_lib.fwd_mla(q, ckv, idx, sm_scale=inst.sm_scale)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    assert bool(torch.all(torch.isneginf(lse)))
