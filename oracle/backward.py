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

from .attention import build_kv
from .decode import decode

_ROW_CHUNK = 512


def causal_attention_bwd(qx: np.ndarray, kx: np.ndarray, vx: np.ndarray, dox: np.ndarray,
                         sm_scale: float):
    """Backward of causal softmax attention over one whole sequence.

    qx, dox: [L, Hq, D] float64 queries and upstream output gradient;
    kx, vx:  [L, Hkv, D] float64 keys and values.  Row r sees keys j <= r.
    Returns dQ [L, Hq, D], dK [L, Hkv, D], dV [L, Hkv, D] (float64).
    """
    l_n, hq, d = qx.shape
    hkv = kx.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    dq = np.zeros((l_n, hq, d), dtype=np.float64)
    dk = np.zeros((l_n, hkv, d), dtype=np.float64)
    dv = np.zeros((l_n, hkv, d), dtype=np.float64)
    cols = np.arange(l_n)
    for c0 in range(0, l_n, _ROW_CHUNK):
        c1 = min(l_n, c0 + _ROW_CHUNK)
        masked = cols[None, :] > np.arange(c0, c1)[:, None]
        for h in range(hq):
            kvh = h // g
            z = (qx[c0:c1, h, :] @ kx[:, kvh, :].T) * sm_scale
            z[masked] = -np.inf
            m = z.max(axis=1)
            p = np.exp(z - m[:, None])
            p /= p.sum(axis=1)[:, None]
            do_r = dox[c0:c1, h, :]
            dv[:, kvh, :] += p.T @ do_r
            dp = do_r @ vx[:, kvh, :].T
            delta = (p * dp).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[c0:c1, h, :] = (ds @ kx[:, kvh, :]) * sm_scale
            dk[:, kvh, :] += (ds.T @ qx[c0:c1, h, :]) * sm_scale
    return dq, dk, dv


def attn_flat_bwd(q, k, v, do, prefix_len: int, seg_offsets: Sequence[int], sm_scale: float,
                  dtype: int = 0):
    """Gradients of the flat-packed forward [P | S1 | ... | SN].

    q, do: [T, Hq, D]; k, v: [T, Hkv, D], in storage form ``dtype`` (0 fp32,
    1 bf16 bits) or already float64 when dtype is None.  seg_offsets: N+1
    offsets, seg_offsets[0] = P, seg_offsets[N] = T.
    Returns dQ [T, Hq, D], dK [T, Hkv, D], dV [T, Hkv, D] in float64.
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
    dq = np.zeros((t_n, hq, d), dtype=np.float64)
    dk = np.zeros((t_n, hkv, d), dtype=np.float64)
    dv = np.zeros((t_n, hkv, d), dtype=np.float64)
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
        gq, gk, gv = causal_attention_bwd(qx, kx, vx, dox, sm_scale)
        # idx holds distinct stored rows, so each copy adds once
        dq[idx] += gq
        dk[idx] += gk
        dv[idx] += gv
    return dq, dk, dv
