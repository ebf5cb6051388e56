"""Pins for the float64 backward oracle (CPU only).

``oracle.backward`` is the expansion route (build_kv copies, textbook causal
attention backward per expansion, copy gradients summed).  It is tied to:

* central finite differences of the forward oracle's loss <dO, O>;
* PyTorch autograd through dense attention over the flat buffer with the
  block-causal visibility written as a mask (a different route: no expansion,
  no hand-written backward);
* exact invariants: sum_c dV[c] = sum of dO over the kv head's query heads,
  sum_c dK[c] = 0 (a common shift of all keys leaves every row's softmax
  unchanged);
* a closed form: with all value rows equal, O does not depend on Q or K, so
  dQ = dK = 0.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attn_flat
from oracle.backward import attn_flat_bwd
from psattn_inputs import BF16, make_flat

SHAPES = [
    # P, rollout lengths, Hq, Hkv, D
    (3, [2, 0, 3], 4, 2, 3),
    (0, [4, 2], 2, 1, 4),
    (5, [], 2, 2, 2),
    (4, [1], 3, 1, 2),
    (2, [3, 3, 1], 4, 4, 3),
]


def _rand(seed, p, lens, hq, hkv, d):
    rng = np.random.default_rng(seed)
    t = p + sum(lens)
    offs = [p] + list(p + np.cumsum(lens)) if lens else [p]
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    do = rng.standard_normal((t, hq, d))
    return q, k, v, do, [int(x) for x in offs]


def _visible(t, p, offs):
    seg = np.full(t, -1)
    for i in range(len(offs) - 1):
        seg[offs[i]:offs[i + 1]] = i
    r = np.arange(t)[:, None]
    c = np.arange(t)[None, :]
    return (c <= r) & ((c < p) | (seg[None, :] == seg[:, None]))


def _torch_grads(q, k, v, do, p, offs, scale):
    """Autograd through dense masked attention over the flat buffer."""
    t, hq, _ = q.shape
    g = hq // k.shape[1]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    vis = torch.from_numpy(_visible(t, p, offs))
    kr = kt.repeat_interleave(g, dim=1)
    vr = vt.repeat_interleave(g, dim=1)
    z = torch.einsum("rhd,chd->hrc", qt, kr) * scale
    z = z.masked_fill(~vis[None], float("-inf"))
    o = torch.einsum("hrc,chd->rhd", torch.softmax(z, dim=-1), vr)
    o.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_matches_autograd_on_the_mask_route(shape):
    p, lens, hq, hkv, d = shape
    q, k, v, do, offs = _rand(11 + len(lens), p, lens, hq, hkv, d)
    scale = 0.7
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, scale, dtype=None)
    tq, tk, tv = _torch_grads(q, k, v, do, p, offs, scale)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("shape", SHAPES[:3])
def test_backward_matches_finite_differences(shape):
    p, lens, hq, hkv, d = shape
    q, k, v, do, offs = _rand(3 + p, p, lens, hq, hkv, d)
    scale = 0.9
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, scale, dtype=None)

    def loss(qq, kk, vv):
        o, _ = attn_flat(qq, kk, vv, p, offs, scale, dtype=None)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[i] += eps
            xm[i] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name] = xp
            args_m[name] = xm
            fd[i] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        assert np.max(np.abs(fd - grad)) < 1e-7, name


def test_backward_invariants():
    p, lens, hq, hkv, d = 6, [5, 2, 7], 8, 2, 4
    q, k, v, do, offs = _rand(5, p, lens, hq, hkv, d)
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, 0.5, dtype=None)
    g = hq // hkv
    for kvh in range(hkv):
        want = do[:, kvh * g:(kvh + 1) * g, :].sum(axis=(0, 1))
        assert np.allclose(dv[:, kvh, :].sum(axis=0), want, rtol=0, atol=1e-12)
        assert np.allclose(dk[:, kvh, :].sum(axis=0), 0.0, rtol=0, atol=1e-12)


def test_backward_constant_values_closed_form():
    p, lens, hq, hkv, d = 4, [3, 5], 4, 2, 3
    q, k, v, do, offs = _rand(9, p, lens, hq, hkv, d)
    v[:] = np.array([0.3, -1.2, 2.0])
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, 1.1, dtype=None)
    assert np.max(np.abs(dq)) < 1e-13
    assert np.max(np.abs(dk)) < 1e-13


def test_backward_prefix_gradient_sums_over_rollouts():
    # a prefix key's dK/dV is the sum of what each expansion alone gives it
    p, lens, hq, hkv, d = 5, [4, 3, 6], 4, 2, 3
    q, k, v, do, offs = _rand(21, p, lens, hq, hkv, d)
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, 0.8, dtype=None)
    acc_k = np.zeros_like(dk[:p])
    acc_v = np.zeros_like(dv[:p])
    for i in range(len(lens)):
        a, b = offs[i], offs[i + 1]
        keep = np.zeros(q.shape[0], dtype=bool)
        keep[a:b] = True
        if i == 0:
            keep[:p] = True
        # the flat loss restricted to the rows expansion i supplies
        gq, gk, gv = attn_flat_bwd(q, k, v, do * keep[:, None, None], p, offs, 0.8, dtype=None)
        acc_k += gk[:p]
        acc_v += gv[:p]
    assert np.allclose(acc_k, dk[:p], rtol=0, atol=1e-12)
    assert np.allclose(acc_v, dv[:p], rtol=0, atol=1e-12)


def test_backward_reads_bf16_storage():
    # storage-form inputs (bf16 bits, dO included) decode exactly to the values
    # that the float64 route receives directly
    from oracle.decode import decode
    from psattn_inputs import f32_to_bf16_bits

    inst = make_flat(6, [3, 4], 4, 2, 8, dtype=BF16, seed=31)
    rng = np.random.default_rng(2)
    do_bits = f32_to_bf16_bits(rng.standard_normal(inst.q.shape).astype(np.float32))
    want = attn_flat_bwd(decode(inst.q, BF16), decode(inst.k, BF16), decode(inst.v, BF16), decode(do_bits, BF16),
                         inst.prefix_len, inst.seg_offsets, inst.sm_scale, dtype=None)
    got = attn_flat_bwd(inst.q, inst.k, inst.v, do_bits, inst.prefix_len, inst.seg_offsets, inst.sm_scale,
                        dtype=BF16)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_backward_restricted_rows_and_keys_match_the_full_result():
    p, lens, hq, hkv, d = 7, [6, 3, 9], 8, 2, 4
    q, k, v, do, offs = _rand(17, p, lens, hq, hkv, d)
    full = attn_flat_bwd(q, k, v, do, p, offs, 0.6, dtype=None)
    rows = np.array([0, 3, 6, 7, 12, 20, 24])
    keys = np.array([1, 5, 6, 8, 14, 15, 24])
    dq, dk, dv = attn_flat_bwd(q, k, v, do, p, offs, 0.6, dtype=None, rows=rows, keys=keys)
    assert np.allclose(dq, full[0][rows], rtol=0, atol=1e-13)
    assert np.allclose(dk, full[1][keys], rtol=0, atol=1e-13)
    assert np.allclose(dv, full[2][keys], rtol=0, atol=1e-13)
