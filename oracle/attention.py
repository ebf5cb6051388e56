"""build_kv expansion + ordinary causal attention, float64 (oracle, test-only).

Flat mode follows PrefixSharing PR #50 ("设计简介" / design summary and
"关键变更" / key changes): the current route physically copies the provider
prefix into every rollout's KV (``build_kv``, done with ``.copy_()``), so each
rollout i is the ordinary sequence ``[P | Si]`` of length P + S_i; the
flat-packed, mask-controlled route is stated to give exactly the same result.
The oracle performs that copy explicitly and then runs textbook causal
attention on each expanded sequence:

    z_j   = sm_scale * <q_r, k_j>            for j <= r (inclusive causal)
    LSE_r = log(sum_j exp(z_j))              (natural log)
    O_r   = sum_j exp(z_j - LSE_r) * v_j

with query head h reading kv head floor(h / G), G = Hq / Hkv.

Paged (verify) mode follows sglang PR #27382 ("实现拆解"): each request's
prefix K/V is gathered page by page from the pool, the request's own draft
K/V block is appended, stored K/V values are multiplied by the per-tensor
k_scale / v_scale, and draft row t (position prefix_b + t) attends causally
over that concatenation.

Where the pages are silent this oracle reads them as follows: prefix rows
are queries too (they see the prefix causally); causality includes the
diagonal; GQA maps consecutive query heads to one kv head; LSE is a natural
log.  O and LSE are returned in float64.

No blocking, fusion or reordering beyond row-chunking of the matmuls (to
bound memory) is done here.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .decode import decode

_ROW_CHUNK = 512


def causal_attention(qr: np.ndarray, qpos: np.ndarray, kx: np.ndarray, vx: np.ndarray,
                     sm_scale: float):
    """Causal softmax attention of selected query rows over one sequence.

    qr:   [R, Hq, D] float64 query rows
    qpos: [R] int   position of each query row in the sequence
    kx,vx:[L, Hkv, D] float64 keys / values of the whole sequence
    Row r sees keys j with j <= qpos[r].
    Returns O [R, Hq, D] and LSE [R, Hq] (float64).
    """
    r_n, hq, d = qr.shape
    l_n, hkv, _ = kx.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    o = np.empty((r_n, hq, d), dtype=np.float64)
    lse = np.empty((r_n, hq), dtype=np.float64)
    cols = np.arange(l_n)
    for c0 in range(0, r_n, _ROW_CHUNK):
        c1 = min(r_n, c0 + _ROW_CHUNK)
        pos = np.asarray(qpos[c0:c1])
        if pos.size and (pos.max() >= l_n or pos.min() < 0):
            raise ValueError("query position outside the sequence")
        masked = cols[None, :] > pos[:, None]
        for h in range(hq):
            kvh = h // g
            z = (qr[c0:c1, h, :] @ kx[:, kvh, :].T) * sm_scale
            z[masked] = -np.inf
            m = z.max(axis=1)
            p = np.exp(z - m[:, None])
            s = p.sum(axis=1)
            o[c0:c1, h, :] = (p @ vx[:, kvh, :]) / s[:, None]
            lse[c0:c1, h] = m + np.log(s)
    return o, lse


def masked_attention(qr: np.ndarray, vis: np.ndarray, kx: np.ndarray, vx: np.ndarray, sm_scale: float):
    """Softmax attention of query rows over the keys each of them sees.

    qr:   [R, Hq, D] float64 query rows
    vis:  [R, L] bool, row r sees key j iff vis[r, j]
    kx,vx:[L, Hkv, D] float64 keys / values
    Returns O [R, Hq, D] and LSE [R, Hq] (float64).
    """
    r_n, hq, d = qr.shape
    hkv = kx.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    o = np.empty((r_n, hq, d), dtype=np.float64)
    lse = np.empty((r_n, hq), dtype=np.float64)
    hidden = ~np.asarray(vis, dtype=bool)
    for h in range(hq):
        kvh = h // g
        z = (qr[:, h, :] @ kx[:, kvh, :].T) * sm_scale
        z[hidden] = -np.inf
        m = z.max(axis=1)
        p = np.exp(z - m[:, None])
        s = p.sum(axis=1)
        o[:, h, :] = (p @ vx[:, kvh, :]) / s[:, None]
        lse[:, h] = m + np.log(s)
    return o, lse


def build_kv(x: np.ndarray, prefix_len: int, seg_begin: int, seg_end: int) -> np.ndarray:
    """Physical expansion of one rollout: a copy of [prefix | own segment]."""
    idx = np.concatenate([np.arange(prefix_len), np.arange(seg_begin, seg_end)])
    return x[idx].copy()


def chain_of(i: int, seg_parent) -> list:
    """Segments from the root-most ancestor down to segment i (parents precede
    their children; -1 is the shared prefix)."""
    out = []
    j = int(i)
    while j >= 0:
        out.append(j)
        j = int(seg_parent[j])
    return out[::-1]


def attn_flat_tree(q, k, v, prefix_len: int, seg_offsets: Sequence[int], seg_parent: Sequence[int],
                   sm_scale: float, dtype: int = 0):
    """Multi-level prefix sharing on the flat buffer [P | S1 | ... | SN].

    seg_parent[i] is the segment whose tokens segment i continues (-1: the
    shared prefix itself), with seg_parent[i] < i.  Each segment is expanded
    the build_kv way to [P | its ancestors' tokens, root-most first | its own
    tokens] and run through ordinary causal attention; its own rows land at
    their flat positions, and the prefix rows come from the prefix alone.
    """
    def dec(x):
        return x if dtype is None else decode(x, dtype)

    offs = [int(x) for x in seg_offsets]
    t_n, hq, d = q.shape
    p = int(prefix_len)
    n = len(offs) - 1
    if offs[0] != p or offs[-1] != t_n or any(b < a for a, b in zip(offs, offs[1:])):
        raise ValueError("bad seg_offsets")
    if any(not (-1 <= int(seg_parent[i]) < i) for i in range(n)):
        raise ValueError("seg_parent[i] must lie in [-1, i)")
    o = np.full((t_n, hq, d), np.nan)
    lse = np.full((t_n, hq), np.nan)
    if p > 0:
        idx = np.arange(p)
        oo, ll = causal_attention(dec(q[idx]), idx, dec(k[idx]), dec(v[idx]), sm_scale)
        o[:p], lse[:p] = oo, ll
    for i in range(n):
        a, b = offs[i], offs[i + 1]
        if b == a:
            continue
        idx = np.concatenate([np.arange(p)] + [np.arange(offs[j], offs[j + 1]) for j in chain_of(i, seg_parent)])
        m = idx.size
        own = np.arange(m - (b - a), m)  # positions of the segment's own tokens in its expansion
        oo, ll = causal_attention(dec(q[idx[own]]), own, dec(k[idx]), dec(v[idx]), sm_scale)
        o[a:b], lse[a:b] = oo, ll
    return o, lse


def attn_flat(q, k, v, prefix_len: int, seg_offsets: Sequence[int], sm_scale: float,
              dtype: int = 0, rows: Optional[Sequence[int]] = None, check_prefix: bool = False):
    """Reference for the flat-packed layout [P | S1 | ... | SN].

    q: [T, Hq, D], k/v: [T, Hkv, D] in storage form ``dtype`` (0 fp32, 1 bf16
    bits, 2 fp8 bits) or already float64 when dtype is None.
    seg_offsets: N+1 offsets, seg_offsets[0] = P, seg_offsets[N] = T.
    rows: optional flat row indices to compute (default: all T rows).

    Each rollout i is expanded to [P | S_i] (build_kv) and run through ordinary
    causal attention; its suffix rows land at their flat positions.  Prefix rows
    are read from rollout 0's expansion (every expansion holds the same prefix
    rows; ``check_prefix`` recomputes them from every rollout and asserts
    agreement).  With N = 0 the buffer is the prefix alone, an expansion with
    an empty suffix.
    """
    def dec(x):
        # decoding is elementwise and exact, so gathering first is the same
        return x if dtype is None else decode(x, dtype)

    offs = [int(x) for x in seg_offsets]
    t_n = q.shape[0]
    p = int(prefix_len)
    n = len(offs) - 1
    if offs[0] != p or offs[-1] != t_n or any(b < a for a, b in zip(offs, offs[1:])):
        raise ValueError("bad seg_offsets")
    hq, d = q.shape[1], q.shape[2]
    want = np.arange(t_n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.full((want.size, hq, d), np.nan)
    lse = np.full((want.size, hq), np.nan)
    where = {int(r): i for i, r in enumerate(want)}

    segs = [(offs[i], offs[i + 1]) for i in range(n)] if n > 0 else [(p, p)]
    pre_rows = [int(r) for r in want if r < p]
    for si, (a, b) in enumerate(segs):
        sel = [int(r) for r in want if a <= r < b]
        sel_pre = pre_rows if (si == 0 or check_prefix) else []
        flat_rows = list(sel_pre) + list(sel)
        if not flat_rows:
            continue
        kx = dec(build_kv(k, p, a, b))
        vx = dec(build_kv(v, p, a, b))
        # query rows of the expanded sequence [P | S_i]: prefix row r stays at
        # r, suffix row r moves to P + (r - o_i)
        local = np.array(list(sel_pre) + [p + (r - a) for r in sel], dtype=np.int64)
        qr = dec(q[np.asarray(flat_rows, dtype=np.int64)])
        oo, ll = causal_attention(qr, local, kx, vx, sm_scale)
        for j, r in enumerate(flat_rows):
            slot = where[r]
            if r < p and si > 0:
                if not (np.allclose(o[slot], oo[j], rtol=0, atol=1e-12)
                        and np.allclose(lse[slot], ll[j], rtol=0, atol=1e-12)):
                    raise AssertionError("prefix rows differ between expansions")
                continue
            o[slot] = oo[j]
            lse[slot] = ll[j]
    return o, lse


def gather_prefix(pool: np.ndarray, kv_indptr, kv_indices, prefix_len: int, b: int,
                  page_size: int) -> np.ndarray:
    """Prefix tokens of request b in order: token t is slot t % page_size of
    the (t // page_size)-th page listed for b."""
    t = np.arange(prefix_len)
    pages = np.asarray(kv_indices)[int(kv_indptr[b]) + t // page_size]
    return pool[pages, t % page_size]


def attn_paged(q, k_pool, v_pool, kv_indptr, kv_indices, prefix_lens, k_ext, v_ext,
               draft_len: int, sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
               q_dtype: int = 1, kv_dtype: int = 1, page_size: int = 16,
               requests: Optional[Sequence[int]] = None, draft_mask: Optional[np.ndarray] = None,
               qo_indptr: Optional[Sequence[int]] = None):
    """Reference for speculative verify over a paged prefix.

    q: [B*Lx, Hq, D]; k_pool/v_pool: [num_pages, page_size, Hkv, D];
    k_ext/v_ext: [B*Lx, Hkv, D] draft K/V.  Returns O [B*Lx, Hq, D], LSE [B*Lx, Hq]
    (rows of requests not listed in ``requests`` are NaN).

    draft_mask: optional [B, Lx, Lx]; draft row t of request b sees draft key j
    iff draft_mask[b, t, j] is nonzero (a draft tree: a token sees its
    ancestors and itself), and every prefix key as before.  The sglang page's
    verify takes such a custom mask over the draft part only (its prefix part is
    skipped); without it, row t sees draft keys 0..t.

    qo_indptr: optional [B+1] ragged draft lengths: request b's draft rows (of
    q, k_ext, v_ext and the outputs) are qo_indptr[b] .. qo_indptr[b+1], and
    draft_mask (if any) is read in its top-left [n_b, n_b] corner.
    """
    qf = decode(q, q_dtype)
    lx = int(draft_len)
    bn = len(prefix_lens)
    hq, d = qf.shape[1], qf.shape[2]
    o = np.full((qf.shape[0], hq, d), np.nan)
    lse = np.full((qf.shape[0], hq), np.nan)
    reqs = range(bn) if requests is None else requests
    for b in reqs:
        pl = int(prefix_lens[b])
        r0 = int(qo_indptr[b]) if qo_indptr is not None else b * lx
        n = int(qo_indptr[b + 1]) - r0 if qo_indptr is not None else lx
        if n == 0:
            continue
        kp = decode(gather_prefix(k_pool, kv_indptr, kv_indices, pl, b, page_size), kv_dtype)
        vp = decode(gather_prefix(v_pool, kv_indptr, kv_indices, pl, b, page_size), kv_dtype)
        kd = decode(k_ext[r0:r0 + n], kv_dtype)
        vd = decode(v_ext[r0:r0 + n], kv_dtype)
        kx = np.concatenate([kp, kd], axis=0) * k_scale
        vx = np.concatenate([vp, vd], axis=0) * v_scale
        if draft_mask is None:
            pos = pl + np.arange(n)
            oo, ll = causal_attention(qf[r0:r0 + n], pos, kx, vx, sm_scale)
        else:
            vis = np.concatenate([np.ones((n, pl), dtype=bool), np.asarray(draft_mask[b])[:n, :n] != 0], axis=1)
            oo, ll = masked_attention(qf[r0:r0 + n], vis, kx, vx, sm_scale)
        o[r0:r0 + n] = oo
        lse[r0:r0 + n] = ll
    return o, lse
