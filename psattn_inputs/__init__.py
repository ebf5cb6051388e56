"""Seeded synthetic inputs for prefix-shared attention.

This module only draws random numbers and stores them in the byte formats the
library consumes (fp32, bf16, OCP fp8 e4m3fn). It holds none of the attention
arithmetic: the float64 reference under ``oracle/`` and the HIP library both
read the exact same bytes produced here.

Workloads (shapes taken from the two workloads the source pages describe:
GRPO rollouts that share one prompt, packed flat as ``[P | S1 | ... | SN]``,
and EAGLE top-k=1 target-verify over a paged KV cache):

* ``tiny``      P=64, N=2 x S=16, Hq=Hkv=2, D=64, fp32.
* ``grpo``      P=2048, N=8 x S=512, Hq=32, Hkv=8, D=128, bf16.
* ``verify16k`` B=8 requests x 16384 prefix tokens in 16-token pages drawn
  from a shuffled 16384-page pool, 4 draft tokens, Hq=32, Hkv=8, D=128, bf16.
* ``verify_fp8`` B=4 x 32768 prefix tokens, 8 draft tokens, Hq=16, Hkv=2,
  D=256, K/V stored as fp8 e4m3fn with per-tensor scales in [0.5, 2].
* ``grpo_ragged`` P=8192, N=16 suffixes with lengths uniform in [256, 1024],
  Hq=64, Hkv=8, D=128, bf16, 1% of key rows scaled by 8 (outlier logits).
* ``mla_dsa``   sparse shared-latent MLA prefill: 16384 prompt tokens, 64
  heads reading one 512-wide latent row per cached token, top-2048 index
  lists (``make_mla``), bf16.

Draw order inside one instance (fixed, so a seed names the bytes):
segment lengths -> Q -> K -> V -> outlier rows -> page permutation ->
draft K -> draft V -> scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

PAGE_SIZE = 16

# storage codes shared with the C ABI's dtype enum
F32, BF16, FP8 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3"}

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def f32_to_fp8_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> OCP fp8 e4m3fn bit patterns (uint8).

    Uses PyTorch's CPU cast to ``torch.float8_e4m3fn`` (a library routine).
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _encode(x: np.ndarray, dt: int) -> np.ndarray:
    if dt == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dt == BF16:
        return f32_to_bf16_bits(x)
    if dt == FP8:
        return f32_to_fp8_bits(x)
    raise ValueError(dt)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


@dataclasses.dataclass
class FlatInstance:
    """Flat-packed ``[P | S1 | ... | SN]`` instance (GRPO layout).

    q: [T, Hq, D], k/v: [T, Hkv, D] in storage form (float32 array for f32,
    uint16 bf16 bit patterns for bf16).  ``seg_offsets`` has N+1 entries,
    ``seg_offsets[0] == prefix_len`` and ``seg_offsets[N] == T``.
    """

    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    prefix_len: int
    seg_offsets: np.ndarray  # int32 [N+1]
    hq: int
    hkv: int
    d: int
    dtype: int
    sm_scale: float
    seed: int

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_segments(self) -> int:
        return int(self.seg_offsets.shape[0] - 1)

    @property
    def seg_lens(self) -> np.ndarray:
        return np.diff(self.seg_offsets.astype(np.int64))

    @property
    def max_seg_len(self) -> int:
        s = self.seg_lens
        return int(s.max()) if s.size else 0


@dataclasses.dataclass
class PagedInstance:
    """Paged verify instance (speculative-decoding target-verify layout).

    q: [B*Lx, Hq, D] bf16 bits.  k_pool/v_pool: [num_pages, 16, Hkv, D] in kv
    storage form.  Request b owns pages ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]``
    in order; prefix token t sits in slot ``t % 16`` of the ``t // 16``-th of
    them.  k_ext/v_ext: [B*Lx, Hkv, D] draft K/V in kv storage form.  Stored
    K/V values are multiplied by k_scale / v_scale.
    """

    name: str
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    kv_indptr: np.ndarray   # int32 [B+1]
    kv_indices: np.ndarray  # int32 [kv_indptr[B]]
    prefix_lens: np.ndarray  # int32 [B]
    k_ext: np.ndarray
    v_ext: np.ndarray
    draft_len: int
    hq: int
    hkv: int
    d: int
    q_dtype: int
    kv_dtype: int
    k_scale: float
    v_scale: float
    sm_scale: float
    seed: int
    page_size: int = PAGE_SIZE
    # ragged draft lengths: request b's draft rows are qo_indptr[b] .. qo_indptr[b+1]
    # (draft_len is then their upper bound); None: b * draft_len .. (b + 1) * draft_len
    qo_indptr: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max()) if self.prefix_lens.size else 0


def make_flat(prefix_len: int, seg_lens: Sequence[int], hq: int, hkv: int, d: int,
              dtype: int = BF16, seed: int = 0, outlier_frac: float = 0.0,
              outlier_scale: float = 8.0, sm_scale: Optional[float] = None,
              name: str = "flat") -> FlatInstance:
    rng = _rng(seed)
    seg_lens = [int(s) for s in seg_lens]
    offs = np.zeros(len(seg_lens) + 1, dtype=np.int64)
    offs[0] = prefix_len
    offs[1:] = prefix_len + np.cumsum(np.asarray(seg_lens, dtype=np.int64))
    t = int(offs[-1])
    q = _normal(rng, (t, hq, d))
    k = _normal(rng, (t, hkv, d))
    v = _normal(rng, (t, hkv, d))
    if outlier_frac > 0 and t > 0:
        n_out = int(round(outlier_frac * t))
        rows = rng.choice(t, size=n_out, replace=False)
        k[rows] *= np.float32(outlier_scale)
    return FlatInstance(
        name=name, q=_encode(q, dtype), k=_encode(k, dtype), v=_encode(v, dtype),
        prefix_len=int(prefix_len), seg_offsets=offs.astype(np.int32), hq=hq, hkv=hkv, d=d,
        dtype=dtype, sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)),
        seed=seed)


def make_flat_random_lens(prefix_len: int, n_seg: int, lo: int, hi: int, hq: int, hkv: int,
                          d: int, dtype: int = BF16, seed: int = 0, **kw) -> FlatInstance:
    """Segment lengths drawn uniformly in [lo, hi] first, from the same stream."""
    rng = _rng(seed)
    lens = rng.integers(lo, hi + 1, size=n_seg)
    # continue with a derived seed so the lengths are the first draw of `seed`
    inst = make_flat(prefix_len, lens.tolist(), hq, hkv, d, dtype=dtype,
                     seed=seed * 1000003 + 17, **kw)
    inst.seed = seed
    return inst


def make_paged(prefix_lens: Sequence[int], draft_len: int, hq: int, hkv: int, d: int,
               kv_dtype: int = BF16, seed: int = 0, num_pages: Optional[int] = None,
               scales: bool = False, poison_unused: bool = True,
               sm_scale: Optional[float] = None, name: str = "paged",
               draft_lens: Optional[Sequence[int]] = None, page_size: int = PAGE_SIZE) -> PagedInstance:
    """draft_lens: per-request draft lengths (ragged); draft_len is then taken
    as their maximum and the draft rows are packed back to back.  page_size:
    token slots per page (16 for the named workloads; with 16 the draws are
    the same as before the argument existed)."""
    rng = _rng(seed)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    b = int(prefix_lens.shape[0])
    qo = None
    n_rows = b * draft_len
    if draft_lens is not None:
        dl = np.asarray(draft_lens, dtype=np.int64)
        qo = np.zeros(b + 1, dtype=np.int64)
        qo[1:] = np.cumsum(dl)
        n_rows = int(qo[-1])
        draft_len = int(dl.max()) if dl.size else 0
    if page_size < 1:
        raise ValueError("page_size must be >= 1")
    n_b = (prefix_lens + page_size - 1) // page_size
    used = int(n_b.sum())
    if num_pages is None:
        num_pages = max(used, 1)
    if num_pages < used:
        raise ValueError("pool too small")
    q = _normal(rng, (n_rows, hq, d))
    # prefix K/V drawn per used page (unused pages are poisoned), then placed
    kp = _normal(rng, (used, page_size, hkv, d))
    vp = _normal(rng, (used, page_size, hkv, d))
    perm = rng.permutation(num_pages).astype(np.int64)
    kx = _normal(rng, (n_rows, hkv, d))
    vx = _normal(rng, (n_rows, hkv, d))
    if scales:
        k_scale = float(rng.uniform(0.5, 2.0))
        v_scale = float(rng.uniform(0.5, 2.0))
    else:
        k_scale = v_scale = 1.0
    indptr = np.zeros(b + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(n_b)
    indices = perm[:used]
    sdt = np.float32 if kv_dtype == F32 else (np.uint16 if kv_dtype == BF16 else np.uint8)
    nan = {F32: np.float32(np.nan), BF16: BF16_NAN, FP8: FP8_NAN}[kv_dtype]
    shape = (num_pages, page_size, hkv, d)
    if poison_unused:
        k_pool = np.full(shape, nan, dtype=sdt)
        v_pool = np.full(shape, nan, dtype=sdt)
    else:
        k_pool = np.zeros(shape, dtype=sdt)
        v_pool = np.zeros(shape, dtype=sdt)
    k_pool[indices] = _encode(kp, kv_dtype)
    v_pool[indices] = _encode(vp, kv_dtype)
    if poison_unused:
        # slots past the end of a request's last, partial page are never read
        for bi in range(b):
            tail = int(prefix_lens[bi] % page_size)
            if tail and n_b[bi] > 0:
                last = indices[indptr[bi + 1] - 1]
                k_pool[last, tail:] = nan
                v_pool[last, tail:] = nan
    q_dtype = F32 if kv_dtype == F32 else BF16
    return PagedInstance(
        name=name, q=_encode(q, q_dtype), k_pool=k_pool, v_pool=v_pool,
        kv_indptr=indptr.astype(np.int32), kv_indices=indices.astype(np.int32),
        prefix_lens=prefix_lens.astype(np.int32), k_ext=_encode(kx, kv_dtype),
        v_ext=_encode(vx, kv_dtype), draft_len=int(draft_len), hq=hq, hkv=hkv, d=d,
        q_dtype=q_dtype, kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
        sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(d)), seed=seed,
        page_size=int(page_size), qo_indptr=None if qo is None else qo.astype(np.int32))


# ---------------------------------------------------------------------------
# spike inputs: every query non-negative and a few key rows set to +16 in
# every element, so that a query's score for a spike key exceeds its other
# scores by far more than 128 ln 2 (a softmax that lost track of its row
# maximum overflows on these).  Bit-level edits only.
# ---------------------------------------------------------------------------
def _abs_bits(x: np.ndarray, dt: int) -> np.ndarray:
    if dt == F32:
        return np.abs(x)
    if dt == BF16:
        return x & np.uint16(0x7FFF)
    raise ValueError(dt)


def make_flat_spikes(prefix_len: int, seg_lens: Sequence[int], hq: int, hkv: int, d: int,
                     spikes: Sequence[int], dtype: int = BF16, seed: int = 0,
                     name: str = "flat_spikes") -> FlatInstance:
    inst = make_flat(prefix_len, seg_lens, hq, hkv, d, dtype=dtype, seed=seed, name=name)
    inst.q = _abs_bits(inst.q, dtype)
    for t in spikes:
        inst.k[t] = _encode(np.full((hkv, d), 16.0, np.float32), dtype)
    return inst


def make_paged_spikes(prefix_lens: Sequence[int], draft_len: int, hq: int, hkv: int, d: int,
                      spikes: Sequence[int], kv_dtype: int = BF16, seed: int = 0,
                      num_pages: Optional[int] = None, name: str = "paged_spikes",
                      page_size: int = PAGE_SIZE) -> PagedInstance:
    """Spikes at the given prefix positions of every request that has them."""
    inst = make_paged(prefix_lens, draft_len, hq, hkv, d, kv_dtype=kv_dtype, seed=seed,
                      num_pages=num_pages, scales=(kv_dtype == FP8), name=name, page_size=page_size)
    inst.q = _abs_bits(inst.q, inst.q_dtype)
    row = _encode(np.full((hkv, d), 16.0, np.float32), kv_dtype)
    for b, pl in enumerate(inst.prefix_lens):
        for t in spikes:
            if t < pl:
                page = inst.kv_indices[inst.kv_indptr[b] + t // inst.page_size]
                inst.k_pool[page, t % inst.page_size] = row
    return inst


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------
CONFIG_NAMES = ["tiny", "grpo", "verify16k", "verify_fp8", "grpo_ragged"]


def make_tree_mask(batch: int, draft_len: int, seed: int, chain: bool = False) -> np.ndarray:
    """Seeded draft trees as a [batch, draft_len, draft_len] uint8 visibility
    mask: token t has a parent drawn uniformly from the earlier tokens (or none,
    hanging off the prefix), and sees its ancestors and itself.  chain=True
    gives the causal chain (the lower triangle)."""
    rng = _rng(seed)
    m = np.zeros((batch, draft_len, draft_len), dtype=np.uint8)
    for b in range(batch):
        parent = [-1] + [int(rng.integers(-1, t)) if not chain else t - 1 for t in range(1, draft_len)]
        for t in range(draft_len):
            j = t
            while j >= 0:
                m[b, t, j] = 1
                j = parent[j]
    return m


@dataclasses.dataclass
class MlaInstance:
    """Sparse shared-latent MLA instance (DSA prefill layout).

    q: [T, H, D] bf16 bits; ckv: [S, D] bf16 bits, one latent row per cached
    token (key and value alike); indices: int32 [T, topk], -1 = padding;
    sink: optional float32 [H] per-head logits."""

    name: str
    q: np.ndarray
    ckv: np.ndarray
    indices: np.ndarray
    sink: Optional[np.ndarray]
    sm_scale: float
    seed: int

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])


def make_mla_indices(num_tokens: int, topk: int, seed: int, num_kv: Optional[int] = None,
                     scatter_pad: bool = False) -> np.ndarray:
    """Seeded top-k index lists of a causal prefill: token t names
    min(t + 1, topk) distinct cached positions drawn uniformly from [0, t]
    (every position when there are at most topk of them), in random order,
    then -1 padding (scattered through the row with scatter_pad).  With
    num_kv the positions are drawn from [0, num_kv) instead of [0, t]."""
    rng = _rng(seed)
    out = np.full((num_tokens, topk), -1, dtype=np.int32)
    for t in range(num_tokens):
        pool = (t + 1) if num_kv is None else num_kv
        n = min(pool, topk)
        if n == 0:
            continue
        pick = rng.permutation(pool)[:n] if pool <= 4 * topk else _distinct(rng, pool, n)
        out[t, :n] = pick
        if scatter_pad:
            out[t] = out[t, rng.permutation(topk)]
    return out


def _distinct(rng: np.random.Generator, pool: int, n: int) -> np.ndarray:
    # n distinct integers of [0, pool), uniformly, in random order (draws with
    # rejection of repeats; pool > 4 n, so a few rounds suffice)
    got = np.unique(rng.integers(0, pool, size=n + n // 4 + 8))
    while got.size < n:
        got = np.union1d(got, rng.integers(0, pool, size=n))
    got = rng.permutation(got)[:n]
    return got


def make_mla(num_tokens: int, num_heads: int, dim: int, topk: int, seed: int = 0, sink: bool = False,
             num_kv: Optional[int] = None, scatter_pad: bool = False, sm_scale: Optional[float] = None,
             name: str = "mla") -> MlaInstance:
    """Draw order: indices, Q, latent cache, sink.  The cache holds the
    prompt's own latent rows (S = num_tokens) unless num_kv is given."""
    s_n = num_tokens if num_kv is None else num_kv
    idx = make_mla_indices(num_tokens, topk, seed, num_kv=num_kv, scatter_pad=scatter_pad)
    rng = _rng(seed * 7919 + 1)
    q = _normal(rng, (num_tokens, num_heads, dim))
    c = _normal(rng, (s_n, dim))
    sk = _normal(rng, (num_heads,)) if sink else None
    return MlaInstance(name=name, q=f32_to_bf16_bits(q), ckv=f32_to_bf16_bits(c), indices=idx, sink=sk,
                       sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dim)), seed=seed)


def make_seg_parents(n_seg: int, seed: int, root_frac: float = 0.3) -> np.ndarray:
    """Seeded multi-level sharing structure: segment i continues the prefix
    (-1) with probability root_frac (always for i = 0), else an earlier
    segment drawn uniformly.  int32 [N]."""
    rng = _rng(seed)
    par = np.full(n_seg, -1, dtype=np.int32)
    for i in range(1, n_seg):
        if rng.random() >= root_frac:
            par[i] = int(rng.integers(0, i))
    return par


def make_config(name: str, seed: Optional[int] = None):
    if name == "tiny":
        return make_flat(64, [16, 16], 2, 2, 64, dtype=F32, seed=1 if seed is None else seed,
                         sm_scale=1.0 / 8.0, name=name)
    if name == "grpo":
        return make_flat(2048, [512] * 8, 32, 8, 128, dtype=BF16,
                         seed=2 if seed is None else seed, name=name)
    if name == "verify16k":
        return make_paged([16384] * 8, 4, 32, 8, 128, kv_dtype=BF16,
                          seed=3 if seed is None else seed, num_pages=16384, name=name)
    if name == "verify_fp8":
        return make_paged([32768] * 4, 8, 16, 2, 256, kv_dtype=FP8,
                          seed=4 if seed is None else seed, num_pages=16384, scales=True,
                          name=name)
    if name == "mla_dsa":
        return make_mla(16384, 64, 512, 2048, seed=6 if seed is None else seed, name=name)
    if name == "grpo_ragged":
        inst = make_flat_random_lens(8192, 16, 256, 1024, 64, 8, 128, dtype=BF16,
                                     seed=5 if seed is None else seed, outlier_frac=0.01)
        inst.name = name
        return inst
    raise KeyError(name)


def is_paged(inst) -> bool:
    return isinstance(inst, PagedInstance)
