"""GPU parity of the dense causal shared-latent MLA prefill
(psattn_mla_dense_fwd) against the float64 oracle (oracle.mla.mla_dense).

The query tokens are the cache's last rows; token t attends to rows
0 .. S - T + t.  Cases: a cache holding only the queries (S = T) and longer
ones (S > T), one query token, counts that end inside a 16-key tile, sinks,
latent rows wider than the 512 values used, 32 / 64 / 128 heads, and a
4096-token prefill with 64 heads on sampled tokens.
"""
import numpy as np
import pytest

from gpu_util import compare, guarded_empty, guards_intact, to_f64
from oracle.mla import mla_dense
from psattn_inputs import make_mla

pytestmark = pytest.mark.gpu


def _run(ps, inst, kv_stride=None):
    import torch

    q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
    c = inst.ckv
    if kv_stride is not None and kv_stride != c.shape[1]:
        wide = np.zeros((c.shape[0], kv_stride), dtype=np.uint16)
        wide[:, :c.shape[1]] = c
        wide[:, c.shape[1]:] = 0x7FC0  # NaN in the unused part of a row
        c = wide
    ckv = torch.from_numpy(np.ascontiguousarray(c).view(np.int16)).view(torch.bfloat16).cuda()
    sink = None if inst.sink is None else torch.from_numpy(inst.sink.astype(np.float32)).cuda()
    o, of = guarded_empty(q.shape, torch.bfloat16)
    lse, lf = guarded_empty(q.shape[:2], torch.float32)
    ps.fwd_mla_dense(q, ckv, sm_scale=inst.sm_scale, sink=sink, out=o, lse=lse)
    torch.cuda.synchronize()
    assert guards_intact(of) and guards_intact(lf), "write outside the outputs"
    return to_f64(o), to_f64(lse)


def _check(ps, inst, label, tokens=None, kv_stride=None):
    o, lse = _run(ps, inst, kv_stride)
    ro, rl = mla_dense(inst.q, inst.ckv, inst.sm_scale, sink=inst.sink, dtype=1, tokens=tokens)
    if tokens is not None:
        o, lse = o[tokens], lse[tokens]
    return compare(o, lse, ro, rl, "bf16", label)


@pytest.mark.parametrize("t,s,h,sink", [
    (50, 50, 64, False),     # the cache holds only the queries
    (37, 120, 32, True),     # a longer cache, 32 heads, sinks
    (16, 16, 128, False),    # 128 heads; the first token sees one row
    (1, 300, 64, True),      # one query token
    (200, 233, 64, False),   # counts ending inside a tile
])
def test_mla_dense_small_full(gpu_lib, t, s, h, sink):
    inst = make_mla(t, h, 512, 1, seed=t + s + h, sink=sink, num_kv=s)
    _check(gpu_lib, inst, f"dense T={t} S={s} H={h} sink={sink}")


def test_mla_dense_wide_rows(gpu_lib):
    inst = make_mla(40, 64, 512, 1, seed=9, num_kv=90)
    _check(gpu_lib, inst, "dense kv_stride 576", kv_stride=576)


def test_mla_dense_prefill_4096_sampled(gpu_lib):
    inst = make_mla(4096, 64, 512, 1, seed=11, num_kv=4096)
    rng = np.random.default_rng(12)
    tokens = np.unique(np.concatenate([[0, 1, 15, 16, 17, 2047, 4095], rng.integers(0, 4096, size=9)]))
    _check(gpu_lib, inst, "dense 4096 x 64 heads sampled", tokens=tokens)
