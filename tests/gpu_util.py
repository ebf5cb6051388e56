"""Helpers for the GPU tests: move seeded instances to the device, run the
library through its C ABI (via the ctypes binding), bring results back as
float64, and compare with the oracle to the stated tolerances."""
from __future__ import annotations

import numpy as np

from psattn_inputs import BF16, F32, FP8

# Tolerances (O absolute error; LSE absolute error, natural log)
TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3),
    "fp8": dict(max_abs=6e-2, mean_abs=2e-3, lse=1e-3),
    # fp32 inputs are held to the bf16 contract and, additionally, to a bar
    # derived from fp32 accumulation over at most a few thousand keys
    "f32": dict(max_abs=1e-4, mean_abs=1e-5, lse=1e-4),
}

GUARD = 64  # elements of NaN guard band before and after every output


def to_dev(arr: np.ndarray, code: int, dev="cuda"):
    import torch

    if code == F32:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)
    if code == BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
    if code == FP8:
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to(dev)
    raise ValueError(code)


def guarded_empty(shape, torch_dtype, dev="cuda"):
    """Output buffer surrounded by NaN guard bands; returns (view, full)."""
    import torch

    n = int(np.prod(shape))
    full = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch_dtype, device=dev)
    return full[GUARD:GUARD + n].view(*shape), full


def guards_intact(full) -> bool:
    import torch

    g = torch.cat([full[:GUARD], full[-GUARD:]]).float()
    return bool(torch.isnan(g).all().item())


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_flat(lib, inst, dev="cuda"):
    import torch

    q = to_dev(inst.q, inst.dtype, dev)
    k = to_dev(inst.k, inst.dtype, dev)
    v = to_dev(inst.v, inst.dtype, dev)
    seg = torch.from_numpy(inst.seg_offsets.astype(np.int32)).to(dev) if inst.num_segments > 0 else None
    o, of = guarded_empty(q.shape, q.dtype, dev)
    lse, lf = guarded_empty((q.shape[0], q.shape[1]), torch.float32, dev)
    lib.fwd_flat(q, k, v, inst.prefix_len, seg, inst.max_seg_len, sm_scale=inst.sm_scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert guards_intact(of) and guards_intact(lf), "write outside the output tensors"
    return o, lse


def run_paged(lib, inst, dev="cuda", workspace=None, draft_mask=None):
    import torch

    q = to_dev(inst.q, inst.q_dtype, dev)
    kp = to_dev(inst.k_pool, inst.kv_dtype, dev)
    vp = to_dev(inst.v_pool, inst.kv_dtype, dev)
    kx = to_dev(inst.k_ext, inst.kv_dtype, dev)
    vx = to_dev(inst.v_ext, inst.kv_dtype, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    indptr, indices, plens = i32(inst.kv_indptr), i32(inst.kv_indices), i32(inst.prefix_lens)
    if indices.numel() == 0:
        indices = torch.zeros(1, dtype=torch.int32, device=dev)
    o, of = guarded_empty(q.shape, q.dtype, dev)
    lse, lf = guarded_empty((q.shape[0], q.shape[1]), torch.float32, dev)
    dm = None if draft_mask is None else torch.from_numpy(np.ascontiguousarray(draft_mask, dtype=np.uint8)).to(dev)
    qo = None if getattr(inst, "qo_indptr", None) is None else i32(inst.qo_indptr)
    lib.fwd_paged(q, kp, vp, indptr, indices, plens, kx, vx, inst.draft_len, inst.max_prefix_len,
                  sm_scale=inst.sm_scale, k_scale=inst.k_scale, v_scale=inst.v_scale,
                  kv_dtype=inst.kv_dtype, out=o, lse=lse, workspace=workspace, draft_mask=dm, qo_indptr=qo)
    torch.cuda.synchronize()
    assert guards_intact(of) and guards_intact(lf), "write outside the output tensors"
    return o, lse


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, kind: str,
            label: str = ""):
    tol = TOL[kind]
    assert np.isfinite(o_gpu).all(), f"{label}: non-finite output"
    assert np.isfinite(lse_gpu).all(), f"{label}: non-finite lse"
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    stats = dict(max_abs=float(err.max(initial=0.0)), mean_abs=float(err.mean()) if err.size else 0.0,
                 lse=float(lerr.max(initial=0.0)))
    print(f"[parity] {label} {kind}: {stats}", flush=True)
    assert stats["max_abs"] <= tol["max_abs"], (label, stats)
    assert stats["mean_abs"] <= tol["mean_abs"], (label, stats)
    assert stats["lse"] <= tol["lse"], (label, stats)
    return stats


def kind_of(code: int, kv_code: int = None) -> str:
    kv = code if kv_code is None else kv_code
    if kv == FP8:
        return "fp8"
    return "f32" if code == F32 else "bf16"


def sample_rows(inst, n_random=48, seed=0):
    """Rows of a flat instance to compare at full size: both ends of the
    prefix, tile boundaries, both ends and the 16/17 boundary of every rollout,
    plus seeded random rows."""
    p = inst.prefix_len
    offs = inst.seg_offsets
    rows = {0, max(p - 1, 0)}
    for t in (31, 32, 63, 64, 127, 128):
        if t < p:
            rows.add(t)
    for a, b in zip(offs[:-1], offs[1:]):
        if b > a:
            rows.update({int(a), int(b) - 1, int(min(a + 16, b - 1)), int(min(a + 17, b - 1))})
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, inst.total_tokens, size=n_random))
    return sorted(r for r in rows if 0 <= r < inst.total_tokens)
