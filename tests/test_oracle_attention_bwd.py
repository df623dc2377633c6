"""Pins of the attention backward oracle (oracle/attention.py,
draft_attention_backward_f64) to things other than itself: central finite differences of
the forward oracle, torch autograd through a masked attention written out here
independently (mask from the predicate pair by pair, RoPE as explicit rotations),
closed-form sums, and the rows that see a single key."""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import cod as ocod
from oracle import rope as orope


def _layout(n, K, cu, seed=3):
    sel = ocod.cod_select(n, K, 0.7, 0.2, seed, np.asarray(cu))
    return sel["idx"], sel["depth_off"]


def _inputs(rng, T, Hq, Hkv, D):
    return (rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)),
            rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hq, D)))


def test_rotate_transpose_is_the_adjoint_and_inverse():
    rng = np.random.default_rng(0)
    x, y = rng.standard_normal((7, 3, 16)), rng.standard_normal((7, 3, 16))
    pos = rng.integers(0, 5000, 7)
    lhs = np.sum(orope.rotate(x, pos, 1e4) * y)
    rhs = np.sum(x * orope.rotate_transpose(y, pos, 1e4))
    assert abs(lhs - rhs) < 1e-12 * np.abs(x).sum()
    np.testing.assert_allclose(orope.rotate_transpose(orope.rotate(x, pos, 5e5), pos, 5e5), x,
                               atol=1e-12)


def test_backward_matches_finite_differences():
    """L = sum(out * dout); every input element perturbed by +-1e-6 (two packed sequences,
    K = 3, G = 2)."""
    rng = np.random.default_rng(1)
    cu = np.array([0, 4, 9])
    idx, depth_off = _layout(9, 3, cu)
    T, Hq, Hkv, D, theta = len(idx), 2, 1, 8, 1e4
    q, k, v, dout = _inputs(rng, T, Hq, Hkv, D)
    got = oattn.draft_attention_backward_f64(q, k, v, idx, depth_off, cu, theta, dout)

    def loss(q_, k_, v_):
        return float(np.sum(oattn.draft_attention_f64(q_, k_, v_, idx, depth_off, cu,
                                                      theta)["out"] * dout))
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for i in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(got[name], num, rtol=0, atol=1e-7, err_msg=name)


def _torch_reference(q, k, v, dout, idx, depth_off, cu, theta):
    """Masked attention in torch float64, the mask written from the predicate pair by pair
    and RoPE as rotate-half with angles pos * theta^(-2j/D); gradients by autograd."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    cu = np.asarray(cu)
    depth = np.zeros(T, dtype=int)
    for d in range(len(depth_off) - 1):
        depth[depth_off[d]:depth_off[d + 1]] = d
    start = np.array([cu[np.searchsorted(cu, p, side="right") - 1] for p in idx])
    pos = idx - start + depth
    allowed = np.zeros((T, T), dtype=bool)
    for r in range(T):
        for c in range(T):
            allowed[r, c] = (depth[c] == 0 and start[c] == start[r] and idx[c] <= idx[r]) or \
                (idx[c] == idx[r] and 1 <= depth[c] <= depth[r])
    j = torch.arange(D // 2, dtype=torch.float64)
    ang = torch.from_numpy(pos.astype(np.float64))[:, None] * theta ** (-2.0 * j / D)
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rope(x):
        x1, x2 = x[..., :D // 2], x[..., D // 2:]
        return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (q, k, v))
    qr, kr = rope(tq), rope(tk)
    G = Hq // Hkv
    kr_h = kr.repeat_interleave(G, dim=1)        # [T, Hq, D]
    v_h = tv.repeat_interleave(G, dim=1)
    sc = torch.einsum("ihd,jhd->hij", qr, kr_h) / np.sqrt(D)
    sc = sc.masked_fill(~torch.from_numpy(allowed)[None], float("-inf"))
    out = torch.einsum("hij,jhd->ihd", torch.softmax(sc, dim=-1), v_h)
    (out * torch.from_numpy(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("n,K,cu,Hq,Hkv,D", [(40, 4, [0, 40], 4, 2, 16),
                                            (50, 3, [0, 17, 30, 50], 2, 2, 8),
                                            (30, 1, [0, 30], 4, 1, 16)])
def test_backward_matches_torch_autograd(n, K, cu, Hq, Hkv, D):
    rng = np.random.default_rng(n)
    cu = np.asarray(cu)
    idx, depth_off = _layout(n, K, cu)
    q, k, v, dout = _inputs(rng, len(idx), Hq, Hkv, D)
    got = oattn.draft_attention_backward_f64(q, k, v, idx, depth_off, cu, 1e4, dout, block=16)
    want = _torch_reference(q, k, v, dout, idx, depth_off, cu, 1e4)
    for name, w in zip(("dq", "dk", "dv"), want):
        np.testing.assert_allclose(got[name], w, rtol=0, atol=1e-10, err_msg=name)


def test_backward_closed_forms():
    """Softmax rows sum to 1, so the dv of a kv head sums (over keys) to the sum of dout
    over its q heads and rows; rows of dS sum to 0, so dk' sums to 0 over keys; a depth-0
    row at a sequence start sees only itself, so its dq is 0."""
    rng = np.random.default_rng(5)
    cu = np.array([0, 30, 64])
    idx, depth_off = _layout(64, 4, cu)
    T, Hq, Hkv, D = len(idx), 4, 2, 16
    q, k, v, dout = _inputs(rng, T, Hq, Hkv, D)
    got = oattn.draft_attention_backward_f64(q, k, v, idx, depth_off, cu, 1e4, dout)
    G = Hq // Hkv
    for g in range(Hkv):
        np.testing.assert_allclose(got["dv"][:, g, :].sum(axis=0),
                                   dout[:, g * G:(g + 1) * G, :].sum(axis=(0, 1)), atol=1e-10)
        np.testing.assert_allclose(got["dk_rot"][:, g, :].sum(axis=0), 0.0, atol=1e-10)
    for a in cu[:-1]:
        assert np.all(got["dq"][a] == 0.0)  # row a of depth 0 is anchor a


def test_row_restricted_backward_equals_full():
    """The subset form (for full-size workloads) reproduces the full oracle's dq rows and
    dk, dv key rows: the last depth-0 keys of each sequence, depth >= 1 rows, and spread
    query rows."""
    rng = np.random.default_rng(11)
    cu = np.array([0, 70, 150])
    idx, depth_off = _layout(150, 4, cu)
    T, Hq, Hkv, D = len(idx), 4, 2, 16
    q, k, v, dout = _inputs(rng, T, Hq, Hkv, D)
    full = oattn.draft_attention_backward_f64(q, k, v, idx, depth_off, cu, 1e4, dout)
    q_rows = np.array([0, 5, 69, 70, 149, 150, T - 1])
    k_rows = np.array([66, 69, 146, 149, 150, 200, T - 1])
    sub = oattn.draft_attention_backward_rows_f64(q, k, v, idx, depth_off, cu, 1e4, dout,
                                                  q_rows, k_rows)
    np.testing.assert_allclose(sub["dq"], full["dq"][q_rows], atol=1e-12)
    np.testing.assert_allclose(sub["dk"], full["dk"][k_rows], atol=1e-12)
    np.testing.assert_allclose(sub["dv"], full["dv"][k_rows], atol=1e-12)
