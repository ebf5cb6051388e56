"""Gradients of the flat prefix-shared forward, float64 (oracle, test-only).

PrefixSharing PR #50 ("关键变更" / key changes) builds each rollout's KV with
``build_kv``, which copies the provider prefix into the rollout with
``.copy_()`` so that gradients flow back through the copy; its test plan asks
for gradients equal to the expanded route's.  The stored prefix rows therefore
receive the sum of the gradients of all their copies.

Definition followed here, step by step:

1. expand every rollout i to the ordinary sequence [P | S_i] (``build_kv``);
2. run textbook causal attention on it: z = sm_scale * Q K^T for key j <= row
   r, P = softmax over the visible keys of each row, O = P V;
3. give it the upstream gradient dO of its rows.  The flat output takes its
   prefix rows from expansion 0 (every expansion computes the same prefix
   rows), so the prefix rows' dO enters expansion 0 and the prefix rows of the
   other expansions get zero;
4. the textbook backward of step 2:
       dV = P^T dO,   dP = dO V^T,   delta_r = sum_j P_rj dP_rj,
       dS = P * (dP - delta),   dQ = sm_scale dS K,   dK = sm_scale dS^T Q,
   where query head h reads kv head floor(h / G), so a kv head's dK and dV sum
   over its G query heads;
5. the copies' gradients flow back to the stored rows: a stored row's gradient
   is the sum over every expansion that holds a copy of it.

With N = 0 the buffer is the prefix alone (one expansion with an empty suffix),
as in the forward oracle.  Nothing here is blocked, fused or reordered beyond
row-chunking the matrix products to bound memory.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import build_kv, chain_of
from .decode import decode

_ROW_CHUNK = 512


def causal_attention_bwd(qx: np.ndarray, kx: np.ndarray, vx: np.ndarray, dox: np.ndarray,
                         sm_scale: float, q_rows=None, k_rows=None):
    """Backward of causal softmax attention over one whole sequence.

    qx, dox: [L, Hq, D] float64 queries and upstream output gradient;
    kx, vx:  [L, Hkv, D] float64 keys and values.  Row r sees keys j <= r.
    q_rows / k_rows: optional index arrays restricting which dQ rows and which
    dK / dV rows are returned (every row's softmax terms are still formed).
    Returns dQ [L or |q_rows|, Hq, D], dK and dV [L or |k_rows|, Hkv, D].
    """
    l_n, hq, d = qx.shape
    hkv = kx.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    qsel = np.arange(l_n) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    ksel = np.arange(l_n) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    qpos = np.full(l_n, -1, dtype=np.int64)
    qpos[qsel] = np.arange(qsel.size)
    dq = np.zeros((qsel.size, hq, d), dtype=np.float64)
    dk = np.zeros((ksel.size, hkv, d), dtype=np.float64)
    dv = np.zeros((ksel.size, hkv, d), dtype=np.float64)
    cols = np.arange(l_n)
    for c0 in range(0, l_n, _ROW_CHUNK):
        c1 = min(l_n, c0 + _ROW_CHUNK)
        masked = cols[None, :] > np.arange(c0, c1)[:, None]
        want = qpos[c0:c1] >= 0
        for h in range(hq):
            kvh = h // g
            z = (qx[c0:c1, h, :] @ kx[:, kvh, :].T) * sm_scale
            z[masked] = -np.inf
            m = z.max(axis=1)
            p = np.exp(z - m[:, None])
            p /= p.sum(axis=1)[:, None]
            do_r = dox[c0:c1, h, :]
            dp = do_r @ vx[:, kvh, :].T
            delta = (p * dp).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dv[:, kvh, :] += p[:, ksel].T @ do_r
            dk[:, kvh, :] += (ds[:, ksel].T @ qx[c0:c1, h, :]) * sm_scale
            if want.any():
                dq[qpos[c0:c1][want], h, :] = (ds[want] @ kx[:, kvh, :]) * sm_scale
    return dq, dk, dv


def attn_flat_bwd(q, k, v, do, prefix_len: int, seg_offsets: Sequence[int], sm_scale: float,
                  dtype: int = 0, rows=None, keys=None):
    """Gradients of the flat-packed forward [P | S1 | ... | SN].

    q, do: [T, Hq, D]; k, v: [T, Hkv, D], in storage form ``dtype`` (0 fp32,
    1 bf16 bits) or already float64 when dtype is None.  seg_offsets: N+1
    offsets, seg_offsets[0] = P, seg_offsets[N] = T.  rows / keys: optional
    flat indices restricting which dQ rows and which dK / dV rows are formed.
    Returns dQ [T or |rows|, Hq, D], dK and dV [T or |keys|, Hkv, D] in float64.
    """
    def dec(x):
        return x if dtype is None else decode(x, dtype)

    offs = [int(x) for x in seg_offsets]
    t_n, hq, d = q.shape
    hkv = k.shape[1]
    p = int(prefix_len)
    n = len(offs) - 1
    if offs[0] != p or offs[-1] != t_n or any(b < a for a, b in zip(offs, offs[1:])):
        raise ValueError("bad seg_offsets")
    want_r = np.arange(t_n) if rows is None else np.asarray(rows, dtype=np.int64)
    want_k = np.arange(t_n) if keys is None else np.asarray(keys, dtype=np.int64)
    slot_r = np.full(t_n, -1, dtype=np.int64)
    slot_r[want_r] = np.arange(want_r.size)
    slot_k = np.full(t_n, -1, dtype=np.int64)
    slot_k[want_k] = np.arange(want_k.size)
    dq = np.zeros((want_r.size, hq, d), dtype=np.float64)
    dk = np.zeros((want_k.size, hkv, d), dtype=np.float64)
    dv = np.zeros((want_k.size, hkv, d), dtype=np.float64)
    segs = [(offs[i], offs[i + 1]) for i in range(n)] if n > 0 else [(p, p)]
    for si, (a, b) in enumerate(segs):
        idx = np.concatenate([np.arange(p), np.arange(a, b)]).astype(np.int64)
        if idx.size == 0:
            continue
        qx = dec(build_kv(q, p, a, b))
        kx = dec(build_kv(k, p, a, b))
        vx = dec(build_kv(v, p, a, b))
        dox = np.array(dec(build_kv(do, p, a, b)), dtype=np.float64)
        if si > 0:
            dox[:p] = 0.0  # the flat prefix rows are expansion 0's
        lr = np.nonzero(slot_r[idx] >= 0)[0]  # local rows / keys of this expansion that are wanted
        lk = np.nonzero(slot_k[idx] >= 0)[0]
        gq, gk, gv = causal_attention_bwd(qx, kx, vx, dox, sm_scale, q_rows=lr, k_rows=lk)
        # each stored row appears once per expansion, so each copy adds once
        dq[slot_r[idx[lr]]] += gq
        dk[slot_k[idx[lk]]] += gk
        dv[slot_k[idx[lk]]] += gv
    return dq, dk, dv


def attn_flat_tree_bwd(q, k, v, do, prefix_len: int, seg_offsets: Sequence[int], seg_parent: Sequence[int],
                       sm_scale: float, dtype: int = 0, rows=None, keys=None):
    """Gradients of the multi-level flat forward (``attn_flat_tree``).

    The forward takes the prefix rows from the prefix alone and the own rows of
    segment i from its expansion [P | ancestors, root-most first | own] (the
    build_kv copy extended down the chain, PrefixSharing PR #50, mask
    construction and the planned multi-level tree support).  The copies keep
    the gradient flowing back to the stored rows (the page's key changes,
    ``.copy_()``), so, step by step:

    1. the prefix expansion [P] with the prefix rows' dO;
    2. for each segment i, its expansion with dO on its own rows only (the
       other rows of the expansion are copies whose outputs come from their
       own expansions, so they receive no upstream gradient there);
    3. the textbook causal attention backward of each expansion
       (``causal_attention_bwd``);
    4. every stored row collects the gradients of all its copies.

    q, do: [T, Hq, D]; k, v: [T, Hkv, D], storage form ``dtype`` or float64
    when dtype is None.  seg_parent[i] in [-1, i).  rows / keys restrict the
    dQ rows and dK / dV rows formed.  Returns dQ, dK, dV in float64.
    """
    def dec(x):
        return x if dtype is None else decode(x, dtype)

    offs = [int(x) for x in seg_offsets]
    t_n, hq, d = q.shape
    hkv = k.shape[1]
    p = int(prefix_len)
    n = len(offs) - 1
    if offs[0] != p or offs[-1] != t_n or any(b < a for a, b in zip(offs, offs[1:])):
        raise ValueError("bad seg_offsets")
    if any(not (-1 <= int(seg_parent[i]) < i) for i in range(n)):
        raise ValueError("seg_parent[i] must lie in [-1, i)")
    want_r = np.arange(t_n) if rows is None else np.asarray(rows, dtype=np.int64)
    want_k = np.arange(t_n) if keys is None else np.asarray(keys, dtype=np.int64)
    slot_r = np.full(t_n, -1, dtype=np.int64)
    slot_r[want_r] = np.arange(want_r.size)
    slot_k = np.full(t_n, -1, dtype=np.int64)
    slot_k[want_k] = np.arange(want_k.size)
    dq = np.zeros((want_r.size, hq, d), dtype=np.float64)
    dk = np.zeros((want_k.size, hkv, d), dtype=np.float64)
    dv = np.zeros((want_k.size, hkv, d), dtype=np.float64)
    expansions = []
    if p > 0:
        expansions.append((np.arange(p), np.arange(p)))  # (stored rows, rows that take dO)
    for i in range(n):
        a, b = offs[i], offs[i + 1]
        if b == a:
            continue
        idx = np.concatenate([np.arange(p)] + [np.arange(offs[j], offs[j + 1]) for j in chain_of(i, seg_parent)])
        expansions.append((idx, np.arange(a, b)))
    for idx, own in expansions:
        idx = idx.astype(np.int64)
        dox = np.zeros((idx.size, hq, d), dtype=np.float64)
        m = idx.size
        dox[m - own.size:] = np.asarray(dec(do[own]), dtype=np.float64)  # own rows close the expansion
        lr = np.nonzero(slot_r[idx] >= 0)[0]
        lk = np.nonzero(slot_k[idx] >= 0)[0]
        gq, gk, gv = causal_attention_bwd(dec(q[idx]), dec(k[idx]), dec(v[idx]), dox, sm_scale, q_rows=lr,
                                          k_rows=lk)
        dq[slot_r[idx[lr]]] += gq
        dk[slot_k[idx[lk]]] += gk
        dv[slot_k[idx[lk]]] += gv
    return dq, dk, dv
