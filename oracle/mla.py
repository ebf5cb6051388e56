"""Sparse shared-latent MLA forward, float64 (oracle, test-only).

Page: the vLLM issue "[Perf] SM8x sparse-MLA prefill fallback re-reads the
shared MLA latent once per head", sections 适用环境 (environment) and 原因分析
(root-cause analysis).  The workload is DSA / sparse-MLA prefill: each query
token attends to the index_topk (2048) cached tokens its indexer selected; the
64 query heads of a token all read the same latent rows (kv_lora_rank = 512,
qk_rope_head_dim = 0, the NoPE layout); the cache is bf16.

Definition followed here (readings where the page is silent):

1. one latent row c[s] (D values) per cached token is both the key and the
   value of every head (absorbed MLA with no rope part);
2. token t attends to the rows its index list names, once per list entry;
   entries outside [0, S) (the -1 padding) are skipped;
3. z_j = sm_scale * <q[t, h], c[s_j]>; an optional per-head sink logit
   sigma_h joins the softmax normaliser and carries no value;
4. o[t, h] = sum_j e^{z_j} c[s_j] / (sum_j e^{z_j} + e^{sigma_h}),
   lse[t, h] = ln(sum_j e^{z_j} + e^{sigma_h});
5. with no listed key and no sink, o = 0 and lse = -inf.

No blocking, fusion or reordering: one token at a time, a gather and two
matrix products.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .decode import decode


def mla_sparse(q, ckv, indices, sm_scale: float, sink=None, dtype: Optional[int] = 1,
               tokens: Optional[Sequence[int]] = None):
    """q: [T, H, D], ckv: [S, D] in storage form ``dtype`` (0 fp32, 1 bf16
    bits) or float64 when dtype is None; indices: int [T, K]; sink: optional
    [H] natural-log logits.  tokens: optional subset of query tokens.
    Returns o [n, H, D] and lse [n, H] in float64."""
    def dec(x):
        return np.asarray(x, dtype=np.float64) if dtype is None else decode(x, dtype)

    idx = np.asarray(indices, dtype=np.int64)
    t_n, hq, d = q.shape
    s_n = ckv.shape[0]
    sel_t = np.arange(t_n) if tokens is None else np.asarray(tokens, dtype=np.int64)
    c = dec(ckv)
    sk = None if sink is None else np.asarray(sink, dtype=np.float64)
    o = np.zeros((sel_t.size, hq, d), dtype=np.float64)
    lse = np.full((sel_t.size, hq), -np.inf, dtype=np.float64)
    for n, t in enumerate(sel_t):
        row = idx[t]
        keys = row[(row >= 0) & (row < s_n)]
        if keys.size == 0 and sk is None:
            continue
        qt = dec(q[t])                                   # [H, D]
        cs = c[keys]                                     # [n, D]
        z = (qt @ cs.T) * sm_scale                       # [H, n]
        if sk is not None:
            z = np.concatenate([z, sk[:, None]], axis=1)  # the sink column
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        den = e.sum(axis=1)
        o[n] = (e[:, :keys.size] @ cs) / den[:, None]
        lse[n] = m + np.log(den)
    return o, lse


def mla_dense(q, ckv, sm_scale: float, sink=None, dtype: Optional[int] = 1,
              tokens: Optional[Sequence[int]] = None):
    """Dense causal shared-latent MLA prefill (the same head-stacked latent
    attention with every earlier cached row listed): the T query tokens are
    the last T positions of the S-row cache, so token t sits at row
    S - T + t and attends to rows 0 .. S - T + t (ordinary causal attention
    with one latent row as key and value for every head).  Steps 3-5 as in
    ``mla_sparse``.  q: [T, H, D], ckv: [S, D] (S >= T); returns o [n, H, D]
    and lse [n, H] in float64."""
    def dec(x):
        return np.asarray(x, dtype=np.float64) if dtype is None else decode(x, dtype)

    t_n, hq, d = q.shape
    s_n = ckv.shape[0]
    if s_n < t_n:
        raise ValueError("the cache must hold the query tokens (S >= T)")
    sel_t = np.arange(t_n) if tokens is None else np.asarray(tokens, dtype=np.int64)
    c = dec(ckv)
    sk = None if sink is None else np.asarray(sink, dtype=np.float64)
    o = np.zeros((sel_t.size, hq, d), dtype=np.float64)
    lse = np.full((sel_t.size, hq), -np.inf, dtype=np.float64)
    for n, t in enumerate(sel_t):
        cs = c[: s_n - t_n + int(t) + 1]                 # rows 0 .. S - T + t
        z = (dec(q[t]) @ cs.T) * sm_scale                # [H, rows]
        if sk is not None:
            z = np.concatenate([z, sk[:, None]], axis=1)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        den = e.sum(axis=1)
        o[n] = (e[:, : cs.shape[0]] @ cs) / den[:, None]
        lse[n] = m + np.log(den)
    return o, lse
