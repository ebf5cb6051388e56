"""Benchmark of prefix-shared attention forward on one MI355X.

Headline workload (the step timed K times): the GRPO flat-packed forward,
P=2048 shared prompt + 8 rollouts x 512 tokens, Hq=32, Hkv=8, D=128, bf16 --
planner, prefix pass, own-rollout diagonal and epilogue in one launch.
``value`` is useful TFLOP/s: 4*D*Hq per visible (query row, key) pair,
masked pairs and softmax excluded.

In the same run the verify path (paged split-KV pass + log-sum-exp combine)
is timed on 8 requests x 16384 prefix tokens, Lx=4, Hq=32, Hkv=8, D=128,
bf16 ("verify us @16k", with its HBM GB/s against the algorithmic bytes that
count every prefix K/V byte once), and, with --all, the fp8 verify and the
large ragged GRPO workloads.

Every timed call is preceded (outside the timed events) by a 1 GiB read
(a reduction over a scratch buffer) that evicts L2 and the 256 MiB MALL, so
every K/V byte is read from HBM.  A read is used rather than a write so that
no dirty lines are left to be written back while the timed kernel runs.
Before timing, each workload's first call is checked for finite outputs.
Parity with the float64 oracle at these same shapes and launch configurations
is the GPU test suite's job (the full-size sampled tests); the oracle runs
here only as the host baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "useful TFLOP/s + HBM GB/s (% roofline) of prefix-shared attn fwd; verify µs @16k"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 1 << 30


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ work counts
def flat_visible_pairs(inst) -> int:
    p = inst.prefix_len
    s = inst.seg_lens.astype(np.int64)
    return int(p * (p + 1) // 2 + np.sum(s * p + s * (s + 1) // 2))


def flat_useful_flops(inst) -> float:
    return 4.0 * inst.d * inst.hq * flat_visible_pairs(inst)


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

    def check(self):
        import torch

        self()
        torch.cuda.synchronize()
        ok = bool(torch.isfinite(self.o).all().item() and torch.isfinite(self.lse).all().item())
        log(f"{self.inst.name}: outputs finite: {ok}")
        if not ok:
            raise RuntimeError(f"{self.inst.name}: non-finite output")


class MlaRunner:
    """The sparse shared-latent MLA forward at one instance."""

    def __init__(self, ps, inst):
        import torch

        self.ps, self.inst = ps, inst
        self.q = torch.from_numpy(inst.q.view(np.int16)).view(torch.bfloat16).cuda()
        self.ckv = torch.from_numpy(inst.ckv.view(np.int16)).view(torch.bfloat16).cuda()
        self.idx = torch.from_numpy(inst.indices).cuda()
        self.sink = None if inst.sink is None else torch.from_numpy(inst.sink.astype(np.float32)).cuda()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
        self.n_keys = int(((inst.indices >= 0) & (inst.indices < inst.ckv.shape[0])).sum())

    def __call__(self):
        self.ps.fwd_mla(self.q, self.ckv, self.idx, sm_scale=self.inst.sm_scale, sink=self.sink, out=self.o,
                        lse=self.lse)

    def useful_flops(self) -> float:
        # 4 * D per (token, head, listed key): the score and value products
        return 4.0 * self.inst.dim * self.inst.num_heads * self.n_keys

    def gathered_bytes(self) -> float:
        # every listed latent row once per token (2 * D bytes), plus Q and O
        return float(self.n_keys * 2 * self.inst.dim + 2 * self.q.numel() * 2)

    def check(self):
        import torch

        self()
        torch.cuda.synchronize()
        ok = bool(torch.isfinite(self.o).all().item() and torch.isfinite(self.lse).all().item())
        log(f"{self.inst.name}: outputs finite: {ok}")
        if not ok:
            raise RuntimeError(f"{self.inst.name}: non-finite output")


class BwdRunner:
    """The flat backward at one instance: forward outputs computed once, then
    each call runs psattn_bwd (row terms, dQ, dK/dV, conversion)."""

    def __init__(self, ps, inst):
        import torch
        from gpu_util import to_dev
        from psattn_inputs import f32_to_bf16_bits

        self.ps, self.inst = ps, inst
        self.q = to_dev(inst.q, inst.dtype)
        self.k = to_dev(inst.k, inst.dtype)
        self.v = to_dev(inst.v, inst.dtype)
        self.seg = torch.from_numpy(inst.seg_offsets).cuda()
        self.o, self.lse = ps.fwd_flat(self.q, self.k, self.v, inst.prefix_len, self.seg, inst.max_seg_len,
                                       sm_scale=inst.sm_scale)
        rng = np.random.default_rng(inst.seed + 1000)
        self.do = to_dev(f32_to_bf16_bits(rng.standard_normal(inst.q.shape).astype(np.float32)), inst.dtype)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        desc = ps.flat_desc(inst.total_tokens, inst.prefix_len, inst.num_segments, self.seg.data_ptr(),
                            inst.max_seg_len)
        nb = ps.psattn_bwd_workspace_size(desc, inst.hq, inst.hkv, inst.d, inst.dtype)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def __call__(self):
        i = self.inst
        self.ps.bwd_flat(self.q, self.k, self.v, self.o, self.lse, self.do, i.prefix_len, self.seg, i.max_seg_len,
                         sm_scale=i.sm_scale, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)

    def finite(self) -> bool:
        import torch

        return all(bool(torch.isfinite(t.float()).all().item()) for t in (self.dq, self.dk, self.dv))


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
        desc = ps.paged_desc(inst.batch, inst.draft_len, 16, inst.num_pages, self.plens.data_ptr(),
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

    def check(self):
        import torch

        self()
        torch.cuda.synchronize()
        ok = bool(torch.isfinite(self.o).all().item() and torch.isfinite(self.lse).all().item())
        log(f"{self.inst.name}: outputs finite: {ok}")
        if not ok:
            raise RuntimeError(f"{self.inst.name}: non-finite output")


def evict(flush):
    """Read 1 GiB so that L2 and the MALL hold none of the workload's bytes."""
    return flush.sum()


def time_calls(fn, flush, steps: int, warmup: int):
    """Mean, min and p50 of per-call event times (ms), each call preceded by a
    cache-evicting read outside the events."""
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
    return dict(mean=float(ms.mean()), min=float(ms.min()), p50=float(np.median(ms)), wall_s=wall)


def cpu_baseline(inst, flops_fn):
    """The float64 oracle on the host cores, on the whole GRPO workload."""
    from oracle.attention import attn_flat

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    attn_flat(inst.q, inst.k, inst.v, inst.prefix_len, inst.seg_offsets, inst.sm_scale, dtype=inst.dtype)
    dt = time.perf_counter() - t0
    return {"value": flops_fn(inst) / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"whole {inst.name} workload ({inst.total_tokens} rows x {inst.hq} heads), "
                      f"float64 build_kv expansion, {dt:.2f} s"}


# the sources the headline kernel (flat2_kernel) is compiled from
HEADLINE_SOURCES = ("device_common.h", "launch.h", "plan.h", "psattn_flat.hip")


def kernel_source_digest() -> str:
    """sha256 over the headline kernel's source files (sorted by name):
    profiler counters are only reused while this digest is unchanged."""
    import hashlib

    csrc = os.path.join(ROOT, "prefix_shared_block_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(HEADLINE_SOURCES):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
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


def prefix_sweep(ps, flush, calls: int, copy_calib: bool, json_out=None):
    """The GRPO shape with N = 1, 2, 4, 8, 16 rollouts of 512 tokens (P = 2048,
    Hq = 32, Hkv = 8, D = 128, bf16): a few evicted calls each, for a counter
    run that checks that the prefix K/V is read about once per call whatever
    N is.  Prints one JSON line with, per N, the launch grid (to match the
    counter rows) and the algorithmic bytes split into Q, prefix K/V and
    rollout K/V."""
    import torch
    from psattn_inputs import BF16, make_flat

    rows = []
    for n in (1, 2, 4, 8, 16):
        inst = make_flat(2048, [512] * n, 32, 8, 128, dtype=BF16, seed=200 + n, name=f"grpo_n{n}")
        run = FlatRunner(ps, inst)
        t = time_calls(run, flush, calls, 1)
        tok, p = inst.total_tokens, inst.prefix_len
        rows.append({"n": n, "grid_threads": run.grid_threads(), "calls": calls + 1, "us": round(t["mean"] * 1e3, 2),
                     "q_bytes": tok * 32 * 128 * 2, "o_bytes": tok * 32 * 128 * 2,
                     "prefix_kv_bytes": 2 * p * 8 * 128 * 2, "rollout_kv_bytes": 2 * (tok - p) * 8 * 128 * 2})
        del run, inst
    out = {"prefix_sweep": rows}
    if copy_calib:
        n = (256 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calib_bytes"] = {"read": n * 4, "write": n * 4}
    print(json.dumps(out), file=json_out or sys.stdout, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--all", action="store_true", help="also time the fp8 verify and ragged GRPO workloads")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) to scale profiler byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--prefix-sweep", action="store_true",
                    help="instead of the benchmark: GRPO with 1..16 rollouts, for the prefix-K/V-read-once counter check")
    args = ap.parse_args()
    # the one JSON line is the only thing on stdout; progress and parity
    # reports go to stderr
    json_out = sys.stdout
    sys.stdout = sys.stderr
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
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

    log("generating grpo workload")
    g_inst = make_config("grpo")
    grpo = FlatRunner(ps, g_inst)
    if not args.no_check:
        grpo.check()
    log("timing grpo")
    tg = time_calls(grpo, flush, args.steps, args.warmup)
    g_flops = flat_useful_flops(g_inst)
    g_tflops = g_flops / (tg["mean"] * 1e-3) / 1e12
    g_tflops_best = g_flops / (tg["min"] * 1e-3) / 1e12
    traffic = traffic_from_profile("flat2_kernel<128, false>", grpo.grid_threads())
    out = {
        "metric": METRIC,
        "value": round(g_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tg["mean"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "grpo: P=2048 + 8 rollouts x 512, Hq=32, Hkv=8, D=128, bf16 N(0,1), flat packed",
                   "global_batch": 8, "seq_len": 2048 + 512, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(g_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(g_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "flat2_kernel<128, false> (bf16)",
                     "per_launch_useful_flop": g_flops, "best_call_tflops": round(g_tflops_best, 2)},
        "grpo_hbm_gbs": round(flat_alg_bytes(g_inst) / (tg["mean"] * 1e-3) / 1e9, 1),
    }
    del grpo

    log("timing the grpo backward")
    gb = BwdRunner(ps, g_inst)
    tb = time_calls(gb, flush, max(3, args.steps // 3), 2)
    assert gb.finite(), "non-finite gradients"
    b_flops = 2.5 * g_flops  # S, dP, dV, dK and dQ products: 10 D flop per visible pair and query head
    out["grpo_bwd"] = {"us": round(tb["mean"] * 1e3, 1), "us_min": round(tb["min"] * 1e3, 1),
                       "useful_tflops": round(b_flops / (tb["mean"] * 1e-3) / 1e12, 2),
                       "frac_mfma": round(b_flops / (tb["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "per_call_useful_flop": b_flops}
    del gb

    log("generating verify16k workload")
    v_inst = make_config("verify16k")
    ver = PagedRunner(ps, v_inst)
    if not args.no_check:
        ver.check()
    log("timing verify16k")
    tv = time_calls(ver, flush, args.steps, args.warmup)
    vb = paged_alg_bytes(v_inst)
    v_gbs = vb / (tv["mean"] * 1e-3) / 1e9
    out["verify16k"] = {"us": round(tv["mean"] * 1e3, 2), "us_min": round(tv["min"] * 1e3, 2),
                        "hbm_gbs": round(v_gbs, 1), "frac_hbm": round(v_gbs / PEAK_HBM_GBS, 4),
                        "alg_bytes": vb, "useful_tflops": round(paged_useful_flops(v_inst) / (tv["mean"] * 1e-3) / 1e12, 2),
                        "n_splits": ver.info.n_splits, "split_len": ver.info.split_len}
    del ver

    if args.all:
        log("generating verify_fp8 workload")
        f_inst = make_config("verify_fp8")
        fr = PagedRunner(ps, f_inst)
        if not args.no_check:
            fr.check()
        tf = time_calls(fr, flush, args.steps, args.warmup)
        fb = paged_alg_bytes(f_inst)
        out["verify_fp8"] = {"us": round(tf["mean"] * 1e3, 2), "hbm_gbs": round(fb / (tf["mean"] * 1e-3) / 1e9, 1),
                             "frac_hbm": round(fb / (tf["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "n_splits": fr.info.n_splits}
        del fr
        log("generating grpo_ragged workload")
        r_inst = make_config("grpo_ragged")
        rr = FlatRunner(ps, r_inst)
        if not args.no_check:
            rr.check()
        tr = time_calls(rr, flush, max(5, args.steps // 3), 2)
        rf = flat_useful_flops(r_inst)
        out["grpo_ragged"] = {"ms": round(tr["mean"], 4), "useful_tflops": round(rf / (tr["mean"] * 1e-3) / 1e12, 2),
                              "frac_mfma": round(rf / (tr["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del rr
        # multi-level sharing at the GRPO shape: two shared 512-token
        # continuations of the prompt, each continued by three rollouts
        log("generating grpo_chain workload")
        c_inst = make_flat(2048, [512] * 8, 32, 8, 128, dtype=BF16, seed=77, name="grpo_chain")
        parents = [-1, -1, 0, 0, 0, 1, 1, 1]
        cr = FlatRunner(ps, c_inst, seg_parent=parents)
        if not args.no_check:
            cr.check()
        tc = time_calls(cr, flush, args.steps, args.warmup)
        cf = flat_tree_useful_flops(c_inst, parents)
        out["grpo_chain"] = {"us": round(tc["mean"] * 1e3, 2),
                             "useful_tflops": round(cf / (tc["mean"] * 1e-3) / 1e12, 2),
                             "frac_mfma": round(cf / (tc["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "parents": parents}
        del cr

    if args.all:
        # sparse shared-latent MLA (DSA prefill): 16384 tokens, 64 heads,
        # top-2048 lists over the prompt's own 512-wide latent rows
        log("generating mla_dsa workload")
        m_inst = make_config("mla_dsa")
        mr = MlaRunner(ps, m_inst)
        if not args.no_check:
            mr.check()
        tm = time_calls(mr, flush, max(5, args.steps // 3), 2)
        mf = mr.useful_flops()
        mb = mr.gathered_bytes()
        out["mla_dsa"] = {"ms": round(tm["mean"], 4), "useful_tflops": round(mf / (tm["mean"] * 1e-3) / 1e12, 2),
                          "frac_mfma": round(mf / (tm["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "gathered_gbs": round(mb / (tm["mean"] * 1e-3) / 1e9, 1)}
        del mr

    if args.copy_calib:
        n = (256 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calib_bytes"] = {"read": n * 4, "write": n * 4}
        del src, dst

    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu baseline)")
        out["cpu_baseline"] = cpu_baseline(g_inst, flat_useful_flops)
    print(json.dumps(out), file=json_out, flush=True)


if __name__ == "__main__":
    main()
