"""Host-side tests of the C ABI (no GPU needed).

* the shared library loads and exports every function include/psattn.h declares;
* argument validation returns the documented status before any HIP call;
* the planner (same header code the kernels run) matches the independent
  enumeration in oracle/plan.py bit-exactly, and its items cover exactly the
  visible (row, key) pairs.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle.plan import coverage_flat, enumerate_flat, enumerate_paged
from oracle.brute import visible
from prefix_shared_block_amd import psattn as ps
from psattn_inputs import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ps.LIB_PATH):
        from prefix_shared_block_amd.build import build

        build()
    return ps.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "psattn.h")).read()
    names = set(re.findall(r"\b(psattn_[a-z_]+)\s*\(", hdr))
    assert {"psattn_fwd", "psattn_workspace_size", "psattn_plan_dump", "psattn_plan_host",
            "psattn_status_string", "psattn_last_error"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(lib):
    # offsets of the C struct (x86-64 SysV): int64 after int32 is 8-aligned
    assert ctypes.sizeof(ps.PsattnDesc) == 128
    assert ps.PsattnDesc.seg_offsets.offset == 24
    assert ps.PsattnDesc.k_ext.offset == 88
    assert ps.PsattnDesc.draft_mask.offset == 104
    assert ps.PsattnDesc.qo_indptr.offset == 112
    assert ps.PsattnDesc.seg_parent.offset == 120
    assert ctypes.sizeof(ps.PsattnPlanInfo) == 32


def test_status_strings(lib):
    for st in range(5):
        assert ps.psattn_status_string(st)
    assert "unknown" in ps.psattn_status_string(99)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _flat(t=96, p=64, n=2, offs=FAKE, mx=16):
    return ps.flat_desc(t, p, n, offs, mx)


def _call(desc, hq=2, hkv=2, d=64, qdt=ps.F32, kvdt=ps.F32, sm=0.125, ks=1.0, vs=1.0,
          q=FAKE, o=FAKE, lse=FAKE, ws=0, wsb=0):
    return ps.psattn_fwd(q, FAKE, FAKE, o, lse, desc, hq, hkv, d, sm, qdt, kvdt, ks, vs, ws, wsb, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), ps.E_INVAL),
    (dict(hq=0), ps.E_INVAL),
    (dict(d=96), ps.E_UNSUPPORTED),
    (dict(qdt=ps.BF16, kvdt=ps.F32), ps.E_UNSUPPORTED),
    (dict(qdt=ps.BF16, kvdt=ps.FP8), ps.E_UNSUPPORTED),  # fp8 K/V only in paged mode
    (dict(qdt=7), ps.E_INVAL),
    (dict(sm=0.0), ps.E_INVAL),
    (dict(sm=float("nan")), ps.E_INVAL),
    (dict(ks=2.0), ps.E_UNSUPPORTED),
    (dict(q=0), ps.E_INVAL),
    (dict(o=FAKE + 8), ps.E_INVAL),
    (dict(lse=FAKE + 2), ps.E_INVAL),
])
def test_flat_validation(lib, kw, status):
    assert _call(_flat(), **kw) == status
    assert ps.psattn_last_error()


@pytest.mark.parametrize("desc_kw,status", [
    (dict(t=96, p=97), ps.E_INVAL),
    (dict(t=-1), ps.E_INVAL),
    (dict(n=-1), ps.E_INVAL),
    (dict(n=0), ps.E_INVAL),           # T != P with no segments
    (dict(offs=0), ps.E_INVAL),        # seg_offsets NULL
    (dict(mx=8), ps.E_INVAL),          # N * max_seg_len < T - P
])
def test_flat_descriptor_validation(lib, desc_kw, status):
    assert _call(_flat(**desc_kw)) == status


def test_seg_parent_takes_bf16_only(lib):
    # multi-level sharing: the bf16 kernels only; the fp32 forward refuses it,
    # the bf16 backward takes it with the one-level workspace (its scratch
    # does not depend on the tree)
    d = ps.flat_desc(96, 64, 2, FAKE, 16, seg_parent_ptr=FAKE)
    assert _call(d, qdt=ps.F32, kvdt=ps.F32) == ps.E_UNSUPPORTED
    assert "seg_parent" in ps.psattn_last_error()
    one = ps.flat_desc(96, 64, 2, FAKE, 16)
    assert ps.psattn_bwd_workspace_size(d, 8, 2, 128, ps.BF16) == ps.psattn_bwd_workspace_size(one, 8, 2, 128,
                                                                                               ps.BF16) > 0
    assert _bwd(d, dt=ps.F32) == ps.E_UNSUPPORTED


def test_flat_gqa_group_too_large(lib):
    assert _call(_flat(), hq=256, hkv=1) == ps.E_UNSUPPORTED


def test_empty_inputs_enqueue_nothing(lib):
    # T = 0 (and P = 0, N = 0): valid, nothing to do, no pointer is touched
    assert _call(ps.flat_desc(0, 0, 0, 0, 0), q=0, o=0, lse=0) == ps.OK
    d = ps.paged_desc(0, 4, 16, 0, 0, 0, 0, 0, 0, 0)
    assert _call(d, qdt=ps.BF16, kvdt=ps.BF16, q=0, o=0, lse=0) == ps.OK


def _paged(batch=2, lx=4, page=16, pages=64, mx=100, arrays=FAKE, ext=FAKE):
    return ps.paged_desc(batch, lx, page, pages, arrays, arrays, arrays, mx, ext, ext)


@pytest.mark.parametrize("desc_kw,kw,status", [
    (dict(lx=0), {}, ps.E_INVAL),
    (dict(page=0), {}, ps.E_INVAL),
    (dict(mx=64 * 16 + 1), {}, ps.E_INVAL),
    (dict(arrays=0), {}, ps.E_INVAL),
    (dict(ext=0), {}, ps.E_INVAL),
    (dict(lx=40), dict(hq=8, hkv=2), ps.E_UNSUPPORTED),   # 40 * 4 rows > 128
    ({}, dict(ks=-1.0), ps.E_INVAL),
    ({}, dict(vs=float("inf")), ps.E_INVAL),
    ({}, {}, ps.E_WORKSPACE),                             # workspace missing
    ({}, dict(ws=FAKE, wsb=16), ps.E_WORKSPACE),          # workspace too small
])
def test_paged_validation(lib, desc_kw, kw, status):
    args = dict(hq=8, hkv=2, d=128, qdt=ps.BF16, kvdt=ps.FP8)
    args.update(kw)
    assert _call(_paged(**desc_kw), **args) == status


def test_workspace_misaligned(lib):
    desc = _paged()
    need = ps.psattn_workspace_size(desc, 8, 2, 128, ps.BF16, ps.FP8)
    assert need > 0
    assert _call(desc, hq=8, hkv=2, d=128, qdt=ps.BF16, kvdt=ps.FP8, ws=FAKE + 16, wsb=need) == ps.E_INVAL


def test_workspace_size_formula(lib):
    desc = _paged(batch=3, lx=4, mx=1000)
    info = ps.plan_info(desc, 8, 2, 128, ps.BF16, ps.BF16)
    rows = 4 * 4
    prow = 3 * 2 * info.n_splits * rows
    r256 = lambda x: (x + 255) // 256 * 256
    # 16 stacked rows in 16-slot pages: the register-streaming pass, whose partial O is bf16
    assert ps.psattn_workspace_size(desc, 8, 2, 128, ps.BF16, ps.BF16) == r256(prow * 128 * 2) + r256(prow * 4)
    assert ps.psattn_workspace_size(_flat(), 2, 2, 64, ps.F32, ps.F32) == 0
    assert ps.psattn_workspace_size(None, 2, 2, 64, ps.F32, ps.F32) == 0


# ---------------------------------------------------------------------------
# planner (host copy of the device code) vs the oracle enumeration
# ---------------------------------------------------------------------------
def _plan_host(desc, hq, hkv, d, qdt, kvdt):
    info = ps.PsattnPlanInfo()
    ps.check(ps.psattn_plan_host(desc, hq, hkv, d, qdt, kvdt, 0, 0, info))
    items = np.zeros((max(info.n_items, 1), ps.ITEM_FIELDS), dtype=np.int32)
    ps.check(ps.psattn_plan_host(desc, hq, hkv, d, qdt, kvdt, items.ctypes.data, info.n_items, info))
    return info, items[:info.n_items]


def _flat_plan(p, lens, hq, hkv, d=128, dt=ps.BF16):
    offs = np.concatenate([[p], p + np.cumsum(lens)]).astype(np.int32) if len(lens) else np.array([p], np.int32)
    desc = ps.flat_desc(int(offs[-1]), p, len(lens), offs.ctypes.data if len(lens) else 0,
                        max(lens) if len(lens) else 0)
    info, items = _plan_host(desc, hq, hkv, d, dt, dt)
    return offs, info, items


@pytest.mark.parametrize("case", range(30))
def test_flat_planner_matches_enumeration(lib, case):
    rng = np.random.default_rng(case)
    p = int(rng.integers(0, 300))
    n = int(rng.integers(0, 6))
    lens = [int(x) for x in rng.integers(0, 200, size=n)]
    if n == 0 and p == 0:
        p = 5
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    offs, info, items = _flat_plan(p, lens, g * hkv, hkv, d=int(rng.choice([64, 128, 256])))
    assert info.tile_tokens == 128 // g
    ref = enumerate_flat(p, offs, hkv, info.tile_tokens)
    assert np.array_equal(items, ref)


@pytest.mark.parametrize("case", range(12))
def test_flat_planner_items_cover_visible_pairs_once(lib, case):
    rng = np.random.default_rng(100 + case)
    p = int(rng.integers(0, 70))
    lens = [int(x) for x in rng.integers(0, 60, size=int(rng.integers(1, 4)))]
    hkv = 2
    g = int(rng.choice([4, 8, 16, 32]))   # small tiles so that tiles are ragged
    offs, info, items = _flat_plan(p, lens, g * hkv, hkv)
    cnt = coverage_flat(items, p, offs, hkv)
    t_n = int(offs[-1])
    vis = np.array([[visible(r, c, p, offs) for c in range(t_n)] for r in range(t_n)], dtype=np.int64)
    for h in range(hkv):
        assert np.array_equal(cnt[h], vis)


@pytest.mark.parametrize("name", ["tiny", "grpo", "grpo_ragged"])
def test_flat_planner_on_named_workloads(lib, name):
    inst = make_config(name)
    offs = inst.seg_offsets
    desc = ps.flat_desc(inst.total_tokens, inst.prefix_len, inst.num_segments, offs.ctypes.data,
                        inst.max_seg_len)
    info, items = _plan_host(desc, inst.hq, inst.hkv, inst.d, inst.dtype, inst.dtype)
    assert np.array_equal(items, enumerate_flat(inst.prefix_len, offs, inst.hkv, info.tile_tokens))


@pytest.mark.parametrize("prefix_lens,lx,hq,hkv,d,kvdt", [
    ([16384] * 8, 4, 32, 8, 128, ps.BF16),
    ([32768] * 4, 8, 16, 2, 256, ps.FP8),
    ([100, 0, 5000, 17], 3, 8, 2, 64, ps.BF16),
    ([0], 1, 4, 4, 128, ps.F32),
    ([4096] * 2, 4, 16, 2, 256, ps.BF16),
])
def test_paged_planner_matches_enumeration(lib, prefix_lens, lx, hq, hkv, d, kvdt):
    pl = np.asarray(prefix_lens, dtype=np.int32)
    n_pages = int(sum((x + 15) // 16 for x in prefix_lens)) + 1
    desc = ps.paged_desc(len(pl), lx, 16, n_pages, pl.ctypes.data, FAKE, FAKE, int(pl.max()), FAKE, FAKE)
    qdt = ps.F32 if kvdt == ps.F32 else ps.BF16
    info, items = _plan_host(desc, hq, hkv, d, qdt, kvdt)
    assert info.split_len % 16 == 0 and info.split_len % info.kv_tile == 0
    assert info.n_splits * info.split_len >= pl.max()
    ref = enumerate_paged(pl, hkv, lx, info.n_splits, info.split_len)
    assert np.array_equal(items, ref)


# ------------------------------------------------------------------ backward
def _bwd(desc, hq=8, hkv=2, d=128, dt=ps.BF16, sm=0.088, ptr=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40):
    return ps.psattn_bwd(ptr, ptr, ptr, ptr, lse, ptr, ptr, ptr, ptr, desc, hq, hkv, d, sm, dt, ws, wsb, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=ps.F32), ps.E_UNSUPPORTED),
    (dict(dt=ps.FP8), ps.E_UNSUPPORTED),
    (dict(hq=128, hkv=1), ps.E_UNSUPPORTED),   # G = 128 > 64
    (dict(hq=7, hkv=2), ps.E_INVAL),
    (dict(sm=-1.0), ps.E_INVAL),
    (dict(ptr=0), ps.E_INVAL),
    (dict(ptr=FAKE + 4), ps.E_INVAL),
    (dict(lse=FAKE + 1), ps.E_INVAL),
    (dict(ws=0), ps.E_WORKSPACE),
    (dict(wsb=1024), ps.E_WORKSPACE),
    (dict(ws=FAKE + 16), ps.E_INVAL),          # workspace not 256-byte aligned
])
def test_bwd_validation(lib, kw, status):
    assert _bwd(_flat(t=96, p=64, n=2, mx=16), **kw) == status
    assert ps.psattn_last_error()


def test_bwd_paged_mode_unsupported(lib):
    assert _bwd(_paged()) == ps.E_UNSUPPORTED
    assert ps.psattn_bwd_workspace_size(_paged(), 8, 2, 128, ps.BF16) == 0


def test_bwd_takes_head_dims_64_128_and_256(lib):
    desc = _flat(t=96, p=64, n=2, mx=16)
    up = lambda x: (x + 255) // 256 * 256
    for d in (64, 128, 256):
        assert ps.psattn_bwd_workspace_size(desc, 8, 2, d, ps.BF16) == 2 * up(96 * 8 * 4) + 2 * up(96 * 2 * d * 4) + up(16 * (5 + 1))


def test_bwd_workspace_size(lib):
    # lse2 and delta [T, Hq] fp32, then the dK / dV accumulators [T, Hkv, D] fp32, then the table of
    # one kv head's dK/dV items (16 bytes each, plus one entry for the first item past them), each
    # 256-byte aligned.  Items: P = 64, two
    # rollouts of 32 tokens, max_seg_len 16: one prefix key tile with one prefix chunk and
    # 32 / 512 + 2 rollout chunks (bound), and 32 / 128 + 2 rollout key tiles with one chunk each
    t, hq, hkv, d = 96, 8, 2, 128
    up = lambda x: (x + 255) // 256 * 256
    n_items = 1 * (1 + (0 + 2)) + (0 + 2) * 1
    want = 2 * up(t * hq * 4) + 2 * up(t * hkv * d * 4) + up(16 * (n_items + 1))
    assert ps.psattn_bwd_workspace_size(_flat(t=t, p=64, n=2, mx=16), hq, hkv, d, ps.BF16) == want
    assert ps.psattn_bwd_workspace_size(ps.flat_desc(0, 0, 0, 0, 0), hq, hkv, d, ps.BF16) == 0


def test_bwd_empty_enqueues_nothing(lib):
    assert _bwd(ps.flat_desc(0, 0, 0, 0, 0), ptr=0, lse=0, ws=0, wsb=0) == ps.OK


# ------------------------------------------------------------------ sparse MLA
def _mla(q=FAKE, ckv=FAKE, idx=FAKE, sink=0, o=FAKE, lse=FAKE, t=16, h=64, d=512, s=100, stride=512, topk=32,
         sm=0.04, dt=ps.BF16):
    return ps.psattn_mla_fwd(q, ckv, idx, sink, o, lse, t, h, d, s, stride, topk, sm, dt, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=ps.F32), ps.E_UNSUPPORTED),
    (dict(dt=9), ps.E_INVAL),
    (dict(d=256), ps.E_UNSUPPORTED),
    (dict(h=48), ps.E_UNSUPPORTED),
    (dict(h=16), ps.E_UNSUPPORTED),
    (dict(topk=2049), ps.E_UNSUPPORTED),
    (dict(topk=-1), ps.E_INVAL),
    (dict(t=-1), ps.E_INVAL),
    (dict(s=-5), ps.E_INVAL),
    (dict(stride=500), ps.E_INVAL),
    (dict(stride=516), ps.E_INVAL),
    (dict(sm=0.0), ps.E_INVAL),
    (dict(q=0), ps.E_INVAL),
    (dict(idx=0), ps.E_INVAL),
    (dict(ckv=0), ps.E_INVAL),
    (dict(o=FAKE + 8), ps.E_INVAL),
    (dict(lse=FAKE + 2), ps.E_INVAL),
    (dict(sink=FAKE + 1), ps.E_INVAL),
])
def test_mla_validation(lib, kw, status):
    assert _mla(**kw) == status
    assert ps.psattn_last_error()


def _mla_dense(q=FAKE, ckv=FAKE, sink=0, o=FAKE, lse=FAKE, t=16, h=64, d=512, s=100, stride=512, sm=0.04,
               dt=ps.BF16):
    return ps.psattn_mla_dense_fwd(q, ckv, sink, o, lse, t, h, d, s, stride, sm, dt, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=ps.F32), ps.E_UNSUPPORTED),
    (dict(d=256), ps.E_UNSUPPORTED),
    (dict(h=48), ps.E_UNSUPPORTED),
    (dict(s=15), ps.E_INVAL),          # the cache must hold the 16 query tokens
    (dict(t=-1), ps.E_INVAL),
    (dict(stride=500), ps.E_INVAL),
    (dict(sm=float("nan")), ps.E_INVAL),
    (dict(ckv=0), ps.E_INVAL),
    (dict(q=FAKE + 4), ps.E_INVAL),
    (dict(sink=FAKE + 2), ps.E_INVAL),
])
def test_mla_dense_validation(lib, kw, status):
    assert _mla_dense(**kw) == status
    assert ps.psattn_last_error()


def test_mla_dense_empty_enqueues_nothing(lib):
    assert _mla_dense(t=0, s=0, q=0, o=0, lse=0, ckv=0) == ps.OK


def test_mla_no_tokens_enqueues_nothing(lib):
    assert _mla(q=0, ckv=0, idx=0, o=0, lse=0, t=0) == ps.OK


def test_mla_binding_checks_argument_types(lib):
    # the binding refuses malformed tensors before any device work
    import torch

    q = torch.zeros(4, 32, 512, dtype=torch.bfloat16)
    ckv = torch.zeros(10, 512, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ps.fwd_mla(q, ckv, torch.zeros(4, 8, dtype=torch.int64))
    with pytest.raises(ValueError):
        ps.fwd_mla(q, ckv, torch.zeros(3, 8, dtype=torch.int32))
    with pytest.raises(ValueError):
        ps.fwd_mla(q, ckv, torch.zeros(4, 8, dtype=torch.int32), sink=torch.zeros(31))


# ---------------------------------------------------------- allocation-free entry point
def _call_noalloc(desc, hq=2, hkv=2, d=64, qdt=ps.F32, kvdt=ps.F32, q=FAKE, o=FAKE, lse=FAKE, ks=1.0, vs=1.0):
    return ps.psattn_fwd_noalloc(q, FAKE, FAKE, o, lse, desc, hq, hkv, d, 0.125, qdt, kvdt, ks, vs, 0)


def test_noalloc_rejects_scratch_beyond_its_array(lib):
    # 256 requests x 8 kv heads x (splits) x 64 stacked rows of partials: far above the array
    desc = _paged(batch=256, lx=8, pages=256 * 2048, mx=32768)
    need = ps.psattn_workspace_size(desc, 64, 8, 256, ps.BF16, ps.FP8)
    limit = 32 << 20
    assert need > limit
    assert _call_noalloc(desc, hq=64, hkv=8, d=256, qdt=ps.BF16, kvdt=ps.FP8) == ps.E_UNSUPPORTED
    msg = ps.psattn_last_error()
    assert str(need) in msg and str(limit) in msg


@pytest.mark.parametrize("desc_kw,kw,status", [
    (dict(lx=0), {}, ps.E_INVAL),
    (dict(arrays=0), {}, ps.E_INVAL),
    ({}, dict(ks=-1.0), ps.E_INVAL),
    (dict(lx=40), dict(hq=8, hkv=2), ps.E_UNSUPPORTED),
])
def test_noalloc_validates_like_psattn_fwd(lib, desc_kw, kw, status):
    args = dict(hq=8, hkv=2, d=128, qdt=ps.BF16, kvdt=ps.FP8)
    args.update(kw)
    assert _call_noalloc(_paged(**desc_kw), **args) == status


def test_noalloc_empty_inputs_enqueue_nothing(lib):
    assert _call_noalloc(ps.flat_desc(0, 0, 0, 0, 0), q=0, o=0, lse=0) == ps.OK
    assert _call_noalloc(ps.paged_desc(0, 4, 16, 0, 0, 0, 0, 0, 0, 0), qdt=ps.BF16, kvdt=ps.BF16, q=0, o=0,
                         lse=0) == ps.OK
