"""Pins for the draft-attention oracle.

- K = 1 is ordinary causal varlen attention (torch's scaled_dot_product_attention
  per packed sequence), the "K=1 == EAGLE-3 step 0" invariant of the NeMo PR.
- The flat expanded layout [context, mask_1..mask_D] under plain causal attention
  reproduces every depth of an anchor (the NeMo PR's parity section).
- Brute-force per-query loops on tiny inputs.
- With q = 0 and one-hot v the output spells out the exact key set.
- Invariants: depth-0 rows ignore K, packed equals standalone, |o| <= max |v|.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, cod, rope
from oracle.bf16 import to_f64
from token_drafting_amd import synth


def _case(n, K, r, r_min, cu, Hq, Hkv, D, seed=5, theta=1.0e4):
    sel = cod.cod_select(n, K, r, r_min, seed, cu)
    T = int(sel["depth_off"][-1])
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    return sel, qkv, theta


def _run(sel, qkv, cu, theta, rows=None):
    return attention.draft_attention(qkv["q"], qkv["k"], qkv["v"], sel["idx"], sel["depth_off"],
                                     cu, theta, rows=rows)


def _sdpa_causal(qr, kr, v):
    """qr [L,Hq,D], kr/v [L,Hkv,D] float64 -> causal attention [L,Hq,D] via torch."""
    G = qr.shape[1] // kr.shape[1]
    q = torch.from_numpy(qr).permute(1, 0, 2)
    k = torch.from_numpy(kr).permute(1, 0, 2).repeat_interleave(G, dim=0)
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, is_causal=True)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("cu,Hq,Hkv,D", [([0, 40], 4, 1, 16), ([0, 13, 30, 48], 8, 2, 32)])
def test_k1_is_causal_varlen_attention(cu, Hq, Hkv, D):
    n = cu[-1]
    sel, qkv, theta = _case(n, 1, 0.7, 0.2, cu, Hq, Hkv, D)
    got = _run(sel, qkv, cu, theta)["out"]
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        pos = np.arange(b - a)
        qr = rope.rotate(to_f64(qkv["q"][a:b]), pos, theta)
        kr = rope.rotate(to_f64(qkv["k"][a:b]), pos, theta)
        want = _sdpa_causal(qr, kr, to_f64(qkv["v"][a:b]))
        assert np.abs(got[a:b] - want).max() < 1e-12


@pytest.mark.parametrize("cu,K,Hq,Hkv", [([0, 36], 4, 4, 1), ([0, 11, 29, 40], 6, 4, 2)])
def test_flat_expanded_layout_matches(cu, K, Hq, Hkv):
    n, D = cu[-1], 16
    sel, qkv, theta = _case(n, K, 0.7, 0.2, cu, Hq, Hkv, D, seed=8)
    got = _run(sel, qkv, cu, theta)["out"]
    row_of = sel["row_of"]
    q, k, v = to_f64(qkv["q"]), to_f64(qkv["k"]), to_f64(qkv["v"])
    checked = 0
    for s in range(len(cu) - 1):
        a = cu[s]
        for p in range(a, cu[s + 1]):
            depths = [e for e in range(K) if row_of[e, p] >= 0]
            top = max(depths)
            assert depths == list(range(top + 1))            # nested sets
            flat = [row_of[0, pp] for pp in range(a, p + 1)] + [row_of[e, p] for e in range(1, top + 1)]
            pos = np.arange(len(flat))                         # 0..p-a, then p-a+1..p-a+top
            o = _sdpa_causal(rope.rotate(q[flat], pos, theta), rope.rotate(k[flat], pos, theta), v[flat])
            for e in range(top + 1):
                r = row_of[e, p]
                assert np.abs(got[r] - o[p - a + e]).max() < 1e-12
                checked += 1
    assert checked == len(sel["idx"])


def _key_rows(sel, cu, r):
    """Constructive key list of draft row r: context rows a_s..p, then (1,p)..(d,p)."""
    idx, off, row_of = sel["idx"], sel["depth_off"], sel["row_of"]
    d = int(np.searchsorted(off, r, side="right") - 1)
    p = int(idx[r])
    a = max(c for c in cu if c <= p)
    return [int(row_of[0, pp]) for pp in range(a, p + 1)] + [int(row_of[e, p]) for e in range(1, d + 1)]


def test_brute_force_tiny():
    cu = [0, 9, 20]
    n, K, Hq, Hkv, D = 20, 4, 2, 1, 8
    sel, qkv, theta = _case(n, K, 0.7, 0.2, cu, Hq, Hkv, D, seed=21)
    res = _run(sel, qkv, cu, theta)
    pos = rope.row_positions(sel["idx"], sel["depth_off"], cu)
    qr = rope.rotate(to_f64(qkv["q"]), pos, theta)
    kr = rope.rotate(to_f64(qkv["k"]), pos, theta)
    v = to_f64(qkv["v"])
    for r in range(len(sel["idx"])):
        keys = _key_rows(sel, cu, r)
        for h in range(Hq):
            sc = [sum(qr[r, h, t] * kr[c, 0, t] for t in range(D)) / math.sqrt(D) for c in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            den = sum(w)
            for t in range(D):
                o = sum(wi * v[c, 0, t] for wi, c in zip(w, keys)) / den
                assert abs(res["out"][r, h, t] - o) < 1e-12
            assert abs(res["lse"][h, r] - (mx + math.log(den))) < 1e-12


def test_one_hot_values_spell_the_key_set():
    cu = [0, 5, 12]
    n, K = 12, 3
    sel = cod.cod_select(n, K, 0.7, 0.2, 4, cu)
    T = int(sel["depth_off"][-1])
    D = 32
    assert T <= D
    q = np.zeros((T, 2, D), dtype=np.uint16)                 # +0.0: uniform softmax
    k = synth.normal_bf16(1, 1, (T, 1, D))
    v = np.zeros((T, 1, D), dtype=np.uint16)
    v[np.arange(T), 0, np.arange(T)] = 0x3F80                # one-hot rows (1.0)
    out = attention.draft_attention(q, k, v, sel["idx"], sel["depth_off"], cu, 1.0e4)["out"]
    for r in range(T):
        keys = _key_rows(sel, cu, r)
        want = np.zeros(D)
        want[keys] = 1.0 / len(keys)
        assert np.abs(out[r, 0] - want).max() < 1e-15 and np.abs(out[r, 1] - want).max() < 1e-15


def test_invariants():
    cu = [0, 14, 33]
    n, Hq, Hkv, D = 33, 4, 2, 16
    sel4, qkv4, theta = _case(n, 4, 0.7, 0.2, cu, Hq, Hkv, D, seed=2)
    res4 = _run(sel4, qkv4, cu, theta)
    # |o| <= max |v| (convex combination)
    assert np.abs(res4["out"]).max() <= np.abs(to_f64(qkv4["v"])).max() + 1e-12
    # depth-0 rows do not depend on K (same depth-0 q/k/v)
    sel1 = cod.cod_select(n, 1, 0.7, 0.2, 2, cu)
    qkv1 = {t: qkv4[t][:n] for t in ("q", "k", "v")}
    res1 = _run(sel1, qkv1, cu, theta)
    assert np.abs(res1["out"] - res4["out"][:n]).max() < 1e-13
    # packed sequence 1 equals a standalone run of it with the same kept anchors
    a, b = cu[1], cu[2]
    rows = [r for r in range(len(sel4["idx"])) if a <= sel4["idx"][r] < b]
    depth = cod.row_depths(sel4["depth_off"])
    idx_s = sel4["idx"][rows] - a
    off_s = np.searchsorted(depth[rows], np.arange(5), side="left").astype(np.int32)
    sub = attention.draft_attention(qkv4["q"][rows], qkv4["k"][rows], qkv4["v"][rows], idx_s, off_s,
                                    [0, b - a], theta)
    assert np.abs(sub["out"] - res4["out"][rows]).max() < 1e-13
    # useful pairs = allowed entries of the dense mask = sum of key-list lengths
    meta = attention.row_meta(sel4["idx"], sel4["depth_off"], cu)
    m = attention.allowed_mask(meta, np.arange(len(sel4["idx"])))
    assert attention.useful_pairs(sel4["idx"], sel4["depth_off"], cu) == int(m.sum())
    assert int(m.sum()) == sum(len(_key_rows(sel4, cu, r)) for r in range(len(sel4["idx"])))


def test_row_subset_equals_full():
    cu = [0, 50]
    sel, qkv, theta = _case(50, 4, 0.7, 0.2, cu, 4, 1, 16, seed=6)
    full = _run(sel, qkv, cu, theta)
    rows = np.array([0, 7, 49, 50, len(sel["idx"]) - 1])
    sub = _run(sel, qkv, cu, theta, rows=rows)
    assert np.array_equal(sub["out"], full["out"][rows])
    assert np.array_equal(sub["lse"], full["lse"][:, rows])
