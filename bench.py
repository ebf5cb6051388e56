"""Benchmark of prefix-shared attention forward on one MI355X.

Every timed call is one ``psattn_fwd`` over one whole workload: the planner,
the prefix pass, the own-rollout (or draft) diagonal, the split merge and
the epilogue, all in the library's kernels.  The default run times all five
workloads:

* ``tiny``        P=64 + 2 x 16, Hq=Hkv=2, D=64, fp32 (latency only);
* ``grpo``        P=2048 + 8 rollouts x 512, Hq=32, Hkv=8, D=128, bf16;
* ``verify16k``   8 requests x 16384 paged prefix tokens, 4 draft tokens,
                  Hq=32, Hkv=8, D=128, bf16 ("verify us @16k");
* ``verify_fp8``  4 x 32768 paged prefix, 8 drafts, Hq=16, Hkv=2, D=256,
                  fp8 e4m3 K/V with per-tensor scales;
* ``grpo_ragged`` P=8192 + 16 rollouts of U{256..1024} tokens, Hq=64, Hkv=8,
                  D=128, bf16, 1% of key rows x8 -- the headline: ``value`` is
                  its useful TFLOP/s (4 D Hq per visible (query row, key)
                  pair; masked pairs and the softmax excluded).

Each workload reports its time distribution (mean, p10, p50, p90 over the
timed calls), useful TFLOP/s, HBM GB/s against its algorithmic bytes (every
K/V byte counted once), and the fraction of the roof that binds it: dense
bf16 MFMA (2500 TFLOP/s) for the GRPO shapes, HBM (8000 GB/s) for the verify
shapes.  The GRPO backward is timed too; with --all, the two-level sharing
and sparse-MLA workloads as well.

Every timed call is preceded (outside its events) by a 1 GiB read that
evicts L2 and the 256 MiB MALL, so every K/V byte comes from HBM; a read, so
that no dirty lines are written back during the timed call.  The events are
recorded on the stream the kernels are launched on.  Before timing, each
workload's first call is checked for finite outputs; parity with the float64
oracle at these shapes and launch configurations is the GPU tests' job (the
full-size tests), and the oracle runs here only as the host baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "useful TFLOP/s + HBM GB/s (% roofline) of prefix-shared attn fwd; verify µs @16k"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 (vector and matrix)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 1 << 30
HEADLINE = "grpo_ragged"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ work counts
def flat_visible_pairs(inst) -> int:
    p = inst.prefix_len
    s = inst.seg_lens.astype(np.int64)
    return int(p * (p + 1) // 2 + np.sum(s * p + s * (s + 1) // 2))


def flat_useful_flops(inst) -> float:
    return 4.0 * inst.d * inst.hq * flat_visible_pairs(inst)


def flat_rows_useful_flops(inst, rows) -> float:
    """Useful flop of the given flat rows only (the host-baseline sample)."""
    p = inst.prefix_len
    offs = inst.seg_offsets.astype(np.int64)
    pairs = 0
    for r in rows:
        if r < p:
            pairs += r + 1
        else:
            i = int(np.searchsorted(offs, r, side="right")) - 1
            pairs += p + (r - int(offs[i])) + 1
    return 4.0 * inst.d * inst.hq * float(pairs)


def flat_tree_useful_flops(inst, parents) -> float:
    """Multi-level sharing: a segment's rows also see every ancestor token."""
    p = inst.prefix_len
    s = inst.seg_lens.astype(np.int64)
    pairs = p * (p + 1) // 2
    for i in range(len(s)):
        anc, j = 0, int(parents[i])
        while j >= 0:
            anc += int(s[j])
            j = int(parents[j])
        pairs += int(s[i]) * (p + anc) + int(s[i]) * (int(s[i]) + 1) // 2
    return 4.0 * inst.d * inst.hq * float(pairs)


def flat_alg_bytes(inst) -> float:
    es = 4 if inst.dtype == 0 else 2
    t = inst.total_tokens
    return float(t * inst.hq * inst.d * 2 * es + 2 * t * inst.hkv * inst.d * es + 4 * t * inst.hq
                 + 4 * (inst.num_segments + 1))


def paged_useful_flops(inst) -> float:
    lx = inst.draft_len
    pl = inst.prefix_lens.astype(np.int64)
    return 4.0 * inst.d * inst.hq * float(np.sum(lx * pl + lx * (lx + 1) // 2))


def paged_alg_bytes(inst) -> float:
    bkv = {0: 4, 1: 2, 2: 1}[inst.kv_dtype]
    bq = 4 if inst.q_dtype == 0 else 2
    b, lx = inst.batch, inst.draft_len
    pl = inst.prefix_lens.astype(np.int64)
    n_pages = int(inst.kv_indptr[-1])
    return float(np.sum(2 * pl * inst.hkv * inst.d * bkv) + b * lx * inst.hq * inst.d * 2 * bq
                 + 2 * b * lx * inst.hkv * inst.d * bkv + 4 * b * lx * inst.hq
                 + 4 * (n_pages + 2 * b + 1))


# ------------------------------------------------------------------ runners
class FlatRunner:
    def __init__(self, ps, inst, seg_parent=None):
        import torch
        from gpu_util import to_dev

        self.ps, self.inst = ps, inst
        self.parents = None if seg_parent is None else np.asarray(seg_parent, dtype=np.int32)
        self.par = None if seg_parent is None else torch.from_numpy(self.parents).cuda()
        self.q = to_dev(inst.q, inst.dtype)
        self.k = to_dev(inst.k, inst.dtype)
        self.v = to_dev(inst.v, inst.dtype)
        self.seg = torch.from_numpy(inst.seg_offsets).cuda()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")

    def grid_threads(self) -> int:
        d = self.ps.flat_desc(self.inst.total_tokens, self.inst.prefix_len, self.inst.num_segments,
                              self.seg.data_ptr(), self.inst.max_seg_len)
        info = self.ps.plan_info(d, self.inst.hq, self.inst.hkv, self.inst.d, self.inst.dtype, self.inst.dtype)
        return int(info.n_items) * (int(info.rows_per_tile) // 32) * 64

    def __call__(self):
        self.ps.fwd_flat(self.q, self.k, self.v, self.inst.prefix_len, self.seg, self.inst.max_seg_len,
                         sm_scale=self.inst.sm_scale, out=self.o, lse=self.lse, seg_parent=self.par)

    def outputs(self):
        return self.o, self.lse


class PagedRunner:
    def __init__(self, ps, inst):
        import torch
        from gpu_util import to_dev

        self.ps, self.inst = ps, inst
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        self.q = to_dev(inst.q, inst.q_dtype)
        self.kp = to_dev(inst.k_pool, inst.kv_dtype)
        self.vp = to_dev(inst.v_pool, inst.kv_dtype)
        self.kx = to_dev(inst.k_ext, inst.kv_dtype)
        self.vx = to_dev(inst.v_ext, inst.kv_dtype)
        self.indptr, self.indices, self.plens = i32(inst.kv_indptr), i32(inst.kv_indices), i32(inst.prefix_lens)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
        desc = ps.paged_desc(inst.batch, inst.draft_len, inst.page_size, inst.num_pages, self.plens.data_ptr(),
                             self.indptr.data_ptr(), self.indices.data_ptr(), inst.max_prefix_len,
                             self.kx.data_ptr(), self.vx.data_ptr())
        nbytes = ps.psattn_workspace_size(desc, inst.hq, inst.hkv, inst.d, inst.q_dtype, inst.kv_dtype)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        self.info = ps.plan_info(desc, inst.hq, inst.hkv, inst.d, inst.q_dtype, inst.kv_dtype)

    def __call__(self):
        i = self.inst
        self.ps.fwd_paged(self.q, self.kp, self.vp, self.indptr, self.indices, self.plens, self.kx, self.vx,
                          i.draft_len, i.max_prefix_len, sm_scale=i.sm_scale, k_scale=i.k_scale,
                          v_scale=i.v_scale, kv_dtype=i.kv_dtype, out=self.o, lse=self.lse, workspace=self.ws)

    def outputs(self):
        return self.o, self.lse


class MlaRunner:
    """The shared-latent MLA forward at one instance: the sparse top-k form,
    or with dense=True the causal prefill over the whole cache (the index
    lists unused)."""

    def __init__(self, ps, inst, dense=False):
        import torch

        self.ps, self.inst, self.dense = ps, inst, dense
        self.q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
        self.ckv = torch.from_numpy(inst.ckv.view(np.int16)).view(torch.bfloat16).cuda()
        self.idx = torch.from_numpy(inst.indices).cuda()
        self.sink = None if inst.sink is None else torch.from_numpy(inst.sink.astype(np.float32)).cuda()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
        if dense:
            t_n, s_n = inst.q.shape[0], inst.ckv.shape[0]
            self.n_keys = sum(s_n - t_n + t + 1 for t in range(t_n))
        else:
            self.n_keys = int(((inst.indices >= 0) & (inst.indices < inst.ckv.shape[0])).sum())

    def __call__(self):
        if self.dense:
            self.ps.fwd_mla_dense(self.q, self.ckv, sm_scale=self.inst.sm_scale, sink=self.sink, out=self.o,
                                  lse=self.lse)
        else:
            self.ps.fwd_mla(self.q, self.ckv, self.idx, sm_scale=self.inst.sm_scale, sink=self.sink, out=self.o,
                            lse=self.lse)

    def outputs(self):
        return self.o, self.lse

    def useful_flops(self) -> float:
        # 4 * D per (token, head, listed key): the score and value products
        return 4.0 * self.inst.dim * self.inst.num_heads * self.n_keys

    def gathered_bytes(self) -> float:
        # every listed latent row once per token (2 * D bytes), plus Q and O
        return float(self.n_keys * 2 * self.inst.dim + 2 * self.q.numel() * 2)


class BwdRunner:
    """The flat backward at one instance: forward outputs computed once, then
    each call runs psattn_bwd (row terms, dQ, dK/dV, conversion)."""

    def __init__(self, ps, inst, seg_parent=None):
        import torch
        from gpu_util import to_dev
        from psattn_inputs import f32_to_bf16_bits

        self.ps, self.inst = ps, inst
        self.q = to_dev(inst.q, inst.dtype)
        self.k = to_dev(inst.k, inst.dtype)
        self.v = to_dev(inst.v, inst.dtype)
        self.seg = torch.from_numpy(inst.seg_offsets).cuda()
        self.par = None if seg_parent is None else torch.from_numpy(np.asarray(seg_parent, dtype=np.int32)).cuda()
        self.o, self.lse = ps.fwd_flat(self.q, self.k, self.v, inst.prefix_len, self.seg, inst.max_seg_len,
                                       sm_scale=inst.sm_scale, seg_parent=self.par)
        rng = np.random.default_rng(inst.seed + 1000)
        self.do = to_dev(f32_to_bf16_bits(rng.standard_normal(inst.q.shape).astype(np.float32)), inst.dtype)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        desc = ps.flat_desc(inst.total_tokens, inst.prefix_len, inst.num_segments, self.seg.data_ptr(),
                            inst.max_seg_len, 0 if self.par is None else self.par.data_ptr())
        nb = ps.psattn_bwd_workspace_size(desc, inst.hq, inst.hkv, inst.d, inst.dtype)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def __call__(self):
        i = self.inst
        self.ps.bwd_flat(self.q, self.k, self.v, self.o, self.lse, self.do, i.prefix_len, self.seg, i.max_seg_len,
                         sm_scale=i.sm_scale, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws,
                         seg_parent=self.par)

    def outputs(self):
        return self.dq, self.dk, self.dv


def check_finite(run, name):
    import torch

    run()
    torch.cuda.synchronize()
    ok = all(bool(torch.isfinite(t.float()).all().item()) for t in run.outputs())
    log(f"{name}: outputs finite: {ok}")
    if not ok:
        raise RuntimeError(f"{name}: non-finite output")


def evict(flush):
    """Read 1 GiB so that L2 and the MALL hold none of the workload's bytes."""
    return flush.sum()


def time_calls(fn, flush, steps: int, warmup: int):
    """Per-call event times (ms) of `steps` calls after `warmup` untimed ones,
    each call preceded by a cache-evicting read outside its events.  The
    events go on the current stream, the one the library launches on."""
    import torch

    for _ in range(warmup):
        evict(flush)
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evict(flush)
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    return dict(mean=float(ms.mean()), min=float(ms.min()), p10=float(np.percentile(ms, 10)),
                p50=float(np.median(ms)), p90=float(np.percentile(ms, 90)), wall_s=wall)


def time_record(t, unit="us"):
    f = 1e3 if unit == "us" else 1.0
    return {f"{k}_{unit}": round(t[k] * f, 3) for k in ("mean", "p10", "p50", "p90", "min")}


# ------------------------------------------------------------------ host baseline
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(inst, n_rows: int):
    """The float64 oracle (build_kv expansion + causal softmax attention) on a
    bounded, seeded sample of the headline workload's query rows, on every
    core this process may run on (BLAS threads set to that count)."""
    from oracle.attention import attn_flat

    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    rows = np.sort(np.random.default_rng(12345).choice(inst.total_tokens, size=n_rows, replace=False))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        attn_flat(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, inst.sm_scale, dtype=inst.dtype,
                  rows=rows)
        dt = time.perf_counter() - t0
    flops = flat_rows_useful_flops(inst, rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n_rows} seeded query rows (all {inst.hq} heads) of the {inst.name} workload "
                      f"({inst.total_tokens} rows), float64 build_kv expansion per rollout, {dt:.2f} s "
                      f"for {flops:.3e} useful flop"}


# ------------------------------------------------------------------ counters
# the sources the headline kernel (flat2_kernel) is compiled from; of
# launch.h only the argument struct it takes (the file also declares the
# paged and backward interfaces)
HEADLINE_SOURCES = ("device_common.h", "launch.h", "plan.h", "psattn_flat.hip")


def _headline_text(name: str, text: bytes) -> bytes:
    """The code of one source: comments dropped and whitespace collapsed,
    launch.h reduced to FlatArgs."""
    import re

    if name == "launch.h":
        i = text.index(b"struct FlatArgs {")
        text = text[i:text.index(b"};", i) + 2]
    text = re.sub(rb"/\*.*?\*/", b" ", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b" ", text)
    return b" ".join(text.split())


def kernel_source_digest() -> str:
    """sha256 over the code of the headline kernel's sources (sorted by name;
    comments and whitespace ignored, launch.h reduced to FlatArgs): profiler
    counters are only reused while this digest is unchanged."""
    import hashlib

    csrc = os.path.join(ROOT, "prefix_shared_block_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(HEADLINE_SOURCES):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(_headline_text(name, f.read()))
    return h.hexdigest()


def traffic_from_profile(kernel_prefix: str, grid: int):
    """HBM bytes (read + written) per launch of a kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the factors that a
    plain copy of known size gave in the same runs.  None when the counters
    were taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "all_workloads_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("kernel_source_sha256") != kernel_source_digest():
        return None
    for key, v in prof.get("per_kernel", {}).items():
        name, g = key.rsplit("|", 1)
        if kernel_prefix in name and int(g) == grid:
            return round(v["read_bytes"] + v["write_bytes"])
    return None


# ------------------------------------------------------------------ sweeps
def prefix_sweep(ps, flush, calls: int, copy_calib: bool, json_out=None):
    """The GRPO head layouts with N = 1, 2, 4, 8, 16 rollouts of 512 tokens,
    at P = 2048 (Hq=32, Hkv=8) and at P = 8192 (Hq=64, Hkv=8, the ragged
    workload's), D = 128, bf16: a few evicted calls each, for a counter run
    that checks that the prefix K/V is read about once per call whatever N
    is.  Prints one JSON line with, per case, the launch grid (to match the
    counter rows) and the algorithmic bytes split into Q, prefix K/V and
    rollout K/V."""
    import torch
    from psattn_inputs import BF16, make_flat

    rows = []
    for p, hq in ((2048, 32), (8192, 64)):
        for n in (1, 2, 4, 8, 16):
            inst = make_flat(p, [512] * n, hq, 8, 128, dtype=BF16, seed=200 + n + p, name=f"p{p}_n{n}")
            run = FlatRunner(ps, inst)
            t = time_calls(run, flush, calls, 1)
            tok = inst.total_tokens
            rows.append({"p": p, "hq": hq, "n": n, "grid_threads": run.grid_threads(), "calls": calls + 1,
                         "us": round(t["mean"] * 1e3, 2), "q_bytes": tok * hq * 128 * 2,
                         "o_bytes": tok * hq * 128 * 2, "prefix_kv_bytes": 2 * p * 8 * 128 * 2,
                         "rollout_kv_bytes": 2 * (tok - p) * 8 * 128 * 2})
            del run, inst
    out = {"prefix_sweep": rows}
    if copy_calib:
        out["copy_calib_bytes"] = copy_calibration()
    print(json.dumps(out), file=json_out or sys.stdout, flush=True)


def verify_sweep(ps, flush, calls: int, json_out=None):
    """The fp8 verify head layout (4 requests, 8 drafts, Hq=16, Hkv=2,
    D=256, fp8 K/V, pages of 16) at prefix lengths 4096 .. 65536: time per
    call against K/V bytes, whose straight-line fit splits a call into a
    fixed part (launch ramp, epilogue, tail, merge launch) and a streaming
    part.  Prints one JSON line with, per length, the call's mean time and
    its algorithmic bytes; a kernel trace of the same run gives the split
    and merge launches of each length by their grids."""
    from psattn_inputs import FP8, make_paged

    rows = []
    for plen in (4096, 8192, 16384, 32768, 65536):
        pages = max(16384, 4 * plen // 16)
        inst = make_paged([plen] * 4, 8, 16, 2, 256, kv_dtype=FP8, seed=400 + plen // 4096,
                          num_pages=pages, scales=True, name=f"fp8_{plen}")
        run = PagedRunner(ps, inst)
        t = time_calls(run, flush, calls, 2)
        rows.append({"prefix": plen, "n_splits": int(run.info.n_splits), "us": round(t["mean"] * 1e3, 2),
                     "p50_us": round(t["p50"] * 1e3, 2), "alg_bytes": paged_alg_bytes(inst)})
        del run, inst
    xs = np.array([r["alg_bytes"] for r in rows], dtype=np.float64)
    ys = np.array([r["us"] for r in rows], dtype=np.float64)
    slope, icpt = np.polyfit(xs, ys, 1)
    print(json.dumps({"verify_sweep": rows, "fit_fixed_us": round(float(icpt), 2),
                      "fit_stream_tbs": round(float(1e-6 / slope), 3)}),
          file=json_out or sys.stdout, flush=True)


def copy_calibration():
    """A plain 256 MiB device copy (known bytes), to scale the profiler's
    byte counters."""
    import torch

    n = (256 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"read": n * 4, "write": n * 4}


# ------------------------------------------------------------------ main
def flat_record(inst, t, bound_peak, bound="mfma"):
    flops = flat_useful_flops(inst)
    ab = flat_alg_bytes(inst)
    tf = flops / (t["mean"] * 1e-3) / 1e12
    gbs = ab / (t["mean"] * 1e-3) / 1e9
    rec = {"useful_flop": flops, "alg_bytes": ab, "useful_tflops": round(tf, 2), "hbm_gbs": round(gbs, 1),
           "bound": bound, "peak": bound_peak, "frac": round((tf if bound != "hbm" else gbs) / bound_peak, 4)}
    rec.update(time_record(t))
    return rec


def paged_record(inst, t, runner):
    flops = paged_useful_flops(inst)
    ab = paged_alg_bytes(inst)
    gbs = ab / (t["mean"] * 1e-3) / 1e9
    rec = {"useful_flop": flops, "alg_bytes": ab, "useful_tflops": round(flops / (t["mean"] * 1e-3) / 1e12, 2),
           "hbm_gbs": round(gbs, 1), "bound": "hbm", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
           "n_splits": runner.info.n_splits, "split_len": runner.info.split_len}
    rec.update(time_record(t))
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--all", action="store_true", help="also time the two-level sharing and sparse-MLA workloads")
    ap.add_argument("--only", default=None, help="comma-separated workload names to time (no headline line)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) to scale profiler byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6000, help="query rows of the host-baseline sample")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--prefix-sweep", action="store_true",
                    help="instead of the benchmark: GRPO shapes with 1..16 rollouts at P=2048 and P=8192, "
                         "for the prefix-K/V-read-once counter check")
    ap.add_argument("--verify-sweep", action="store_true",
                    help="instead of the benchmark: the fp8 verify shape at prefix lengths 4096..65536, "
                         "for a fixed-cost / streaming split of its call time")
    args = ap.parse_args()
    # the one JSON line is the only thing on stdout; progress goes to stderr
    json_out = sys.stdout
    sys.stdout = sys.stderr
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from prefix_shared_block_amd import psattn as ps
    from psattn_inputs import BF16, make_config, make_flat

    ps.load()
    torch.cuda.set_device(0)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    if args.prefix_sweep:
        prefix_sweep(ps, flush, max(1, args.steps), args.copy_calib, json_out)
        return
    if args.verify_sweep:
        verify_sweep(ps, flush, max(1, args.steps), json_out)
        return

    only = None if args.only is None else set(args.only.split(","))
    want = lambda name: only is None or name in only
    recs = {}
    insts = {}

    for name in ("tiny", "grpo", "verify16k", "verify_fp8", "grpo_ragged"):
        if not want(name):
            continue
        log(f"generating {name}")
        inst = make_config(name)
        paged = name.startswith("verify")
        run = PagedRunner(ps, inst) if paged else FlatRunner(ps, inst)
        if not args.no_check:
            check_finite(run, name)
        steps = args.steps
        log(f"timing {name} ({steps} calls)")
        t = time_calls(run, flush, steps, args.warmup)
        if paged:
            recs[name] = paged_record(inst, t, run)
        elif name == "tiny":
            # fp32, 96 tokens: a single small launch, bound by latency; the
            # fraction is against the fp32 peak for completeness
            recs[name] = flat_record(inst, t, PEAK_F32_TFLOPS, bound="latency (fp32 peak)")
        else:
            recs[name] = flat_record(inst, t, PEAK_BF16_TFLOPS)
            recs[name]["grid_threads"] = run.grid_threads()
        if name == "grpo_ragged":
            recs[name]["total_tokens"] = inst.total_tokens
            insts[name] = inst
        del run

    if want("grpo_bwd"):
        log("timing the grpo backward")
        g_inst = make_config("grpo")
        gb = BwdRunner(ps, g_inst)
        if not args.no_check:
            check_finite(gb, "grpo_bwd")
        tb = time_calls(gb, flush, max(3, args.steps // 2), 2)
        b_flops = 2.5 * flat_useful_flops(g_inst)  # S, dP, dV, dK, dQ: 10 D flop per visible pair and head
        tf = b_flops / (tb["mean"] * 1e-3) / 1e12
        recs["grpo_bwd"] = {"useful_flop": b_flops, "useful_tflops": round(tf, 2), "bound": "mfma",
                            "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        recs["grpo_bwd"].update(time_record(tb))
        del gb

    if args.all and (want("grpo_chain") or want("grpo_chain_bwd")):
        # multi-level sharing at the GRPO shape: two shared 512-token
        # continuations of the prompt, each continued by three rollouts
        c_inst = make_flat(2048, [512] * 8, 32, 8, 128, dtype=BF16, seed=77, name="grpo_chain")
        parents = [-1, -1, 0, 0, 0, 1, 1, 1]
        cf = flat_tree_useful_flops(c_inst, parents)
        if want("grpo_chain"):
            log("timing grpo_chain")
            cr = FlatRunner(ps, c_inst, seg_parent=parents)
            if not args.no_check:
                check_finite(cr, "grpo_chain")
            tc = time_calls(cr, flush, args.steps, args.warmup)
            recs["grpo_chain"] = {"useful_tflops": round(cf / (tc["mean"] * 1e-3) / 1e12, 2),
                                  "frac": round(cf / (tc["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "parents": parents}
            recs["grpo_chain"].update(time_record(tc))
            del cr
        if want("grpo_chain_bwd"):
            # and its backward
            log("timing grpo_chain_bwd")
            cb = BwdRunner(ps, c_inst, seg_parent=parents)
            if not args.no_check:
                check_finite(cb, "grpo_chain_bwd")
            tcb = time_calls(cb, flush, max(3, args.steps // 2), 2)
            cbf = 2.5 * cf
            recs["grpo_chain_bwd"] = {"useful_tflops": round(cbf / (tcb["mean"] * 1e-3) / 1e12, 2),
                                      "frac": round(cbf / (tcb["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                      "parents": parents}
            recs["grpo_chain_bwd"].update(time_record(tcb))
            del cb
    if args.all and want("mla_dsa"):
        # sparse shared-latent MLA (DSA prefill): 16384 tokens, 64 heads,
        # top-2048 lists over the prompt's own 512-wide latent rows
        log("timing mla_dsa")
        mr = MlaRunner(ps, make_config("mla_dsa"))
        if not args.no_check:
            check_finite(mr, "mla_dsa")
        tm = time_calls(mr, flush, max(5, args.steps // 3), 2)
        mf, mb = mr.useful_flops(), mr.gathered_bytes()
        recs["mla_dsa"] = {"useful_tflops": round(mf / (tm["mean"] * 1e-3) / 1e12, 2),
                           "frac": round(mf / (tm["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "gathered_gbs": round(mb / (tm["mean"] * 1e-3) / 1e9, 1)}
        recs["mla_dsa"].update(time_record(tm, "ms"))
        del mr
    if args.all and want("mla_dense"):
        # the dense causal form: a 4096-token prefill over its own latent
        # rows, 64 heads
        log("timing mla_dense")
        from psattn_inputs import make_mla
        md = MlaRunner(ps, make_mla(4096, 64, 512, 1, seed=11, num_kv=4096, name="mla_dense"), dense=True)
        if not args.no_check:
            check_finite(md, "mla_dense")
        tmd = time_calls(md, flush, max(5, args.steps // 3), 2)
        mdf = md.useful_flops()
        recs["mla_dense"] = {"useful_tflops": round(mdf / (tmd["mean"] * 1e-3) / 1e12, 2),
                             "frac": round(mdf / (tmd["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        recs["mla_dense"].update(time_record(tmd, "ms"))
        del md

    copy_calib = copy_calibration() if args.copy_calib else None

    if only is not None or HEADLINE not in recs:
        out = {"workloads": recs}
        if copy_calib:
            out["copy_calib_bytes"] = copy_calib
        print(json.dumps(out), file=json_out, flush=True)
        return

    h = recs[HEADLINE]
    h_inst = insts[HEADLINE]
    ms = h["mean_us"] / 1e3
    traffic = traffic_from_profile("flat2_kernel<128, false>", h["grid_threads"])
    out = {
        "metric": METRIC,
        "value": h["useful_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"grpo_ragged: P=8192 shared prompt + 16 rollouts of U{{256..1024}} tokens "
                               f"(seed 5, T={h_inst.total_tokens}), Hq=64, Hkv=8, D=128, bf16 N(0,1) with 1% of "
                               f"key rows x8, flat packed with seg_offsets",
                   "global_batch": 16, "seq_len": int(h_inst.total_tokens), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": h["useful_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": h["frac"], "traffic": traffic,
                     "kernel": "flat2_kernel<128, false> (bf16), one launch per call",
                     "per_launch_useful_flop": h["useful_flop"]},
        "verify_us_at_16k": recs.get("verify16k", {}).get("mean_us"),
        "workloads": recs,
    }
    if copy_calib:
        out["copy_calib_bytes"] = copy_calib
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu baseline)")
        out["cpu_baseline"] = cpu_baseline(h_inst, args.cpu_rows)
    print(json.dumps(out), file=json_out, flush=True)


if __name__ == "__main__":
    main()
