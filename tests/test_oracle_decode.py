"""Pins for the decode-shape oracle (one base position per request over a KV cache).

- The last K rows of plain causal attention (torch's scaled_dot_product_attention)
  over the flat sequence [context, anchor, mask_1 .. mask_{K-1}], the layout the NeMo
  PR's parity section says vLLM runs at inference.
- The forward oracle with r = 1 (every position kept at every depth): its rows of the
  last anchor are the decode rows of a context of n - 1 tokens.
- Closed form: an empty cache and K = 1 leaves the anchor alone.
- Requests of a batch are independent of one another.
"""
import numpy as np
import pytest
import torch

from oracle import attention, cod, decode, rope
from oracle.bf16 import to_f64
from token_drafting_amd import synth


def _inputs(seed, lens, K, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    L = int(sum(lens))
    kc = rng.standard_normal((L, Hkv, D))
    vc = rng.standard_normal((L, Hkv, D))
    B = len(lens)
    q = rng.standard_normal((B, K, Hq, D))
    k = rng.standard_normal((B, K, Hkv, D))
    v = rng.standard_normal((B, K, Hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return kc, vc, cu, q, k, v


@pytest.mark.parametrize("lens,K,Hq,Hkv,D", [([37], 4, 4, 1, 64), ([5, 70, 1], 8, 8, 2, 32),
                                             ([0, 12], 3, 2, 2, 16)])
def test_last_rows_of_flat_causal_attention(lens, K, Hq, Hkv, D):
    theta = 1.0e4
    kc_raw, vc, cu, q, k, v = _inputs(3, lens, K, Hq, Hkv, D)
    # cache keys rotated at their positions inside each request
    kc = np.concatenate([rope.rotate(kc_raw[cu[b]:cu[b + 1]], np.arange(lens[b]), theta)
                         for b in range(len(lens))], axis=0) if sum(lens) else kc_raw
    got = decode.decode_attention_f64(kc, vc, cu, q, k, v, theta)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        # flat sequence of L + K tokens: context keys rotated at 0..L-1, new rows at L..L+K-1
        pos = np.arange(L + K)
        k_flat = rope.rotate(np.concatenate([kc_raw[cu[b]:cu[b + 1]], k[b]], axis=0), pos, theta)
        v_flat = np.concatenate([vc[cu[b]:cu[b + 1]], v[b]], axis=0)
        q_flat = np.zeros((L + K, Hq, D))
        q_flat[L:] = rope.rotate(q[b], pos[L:], theta)
        qt = torch.from_numpy(q_flat).permute(1, 0, 2)
        kt = torch.from_numpy(k_flat).permute(1, 0, 2).repeat_interleave(G, dim=0)
        vt = torch.from_numpy(v_flat).permute(1, 0, 2).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        want = o.permute(1, 0, 2).numpy()[L:]
        np.testing.assert_allclose(got["out"][b], want, rtol=0, atol=1e-12)
        # lse: log-sum-exp over the causal prefix of each flat row
        s = torch.einsum("hqd,hkd->hqk", qt, kt) / np.sqrt(D)
        s = s.masked_fill(torch.triu(torch.ones(L + K, L + K, dtype=torch.bool), 1), float("-inf"))
        lse = torch.logsumexp(s, dim=-1).permute(1, 0).numpy()[L:]
        np.testing.assert_allclose(got["lse"][b], lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,K,Hq,Hkv,D", [(40, 4, 4, 1, 64), (9, 6, 4, 2, 32)])
def test_forward_oracle_rows_of_the_last_anchor(n, K, Hq, Hkv, D):
    theta, seed = 1.0e4, 11
    cu = np.array([0, n])
    sel = cod.cod_select(n, K, 1.0, 0.0, seed, cu)          # r = 1: every position, every depth
    T = int(sel["depth_off"][-1])
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    fwd = attention.draft_attention(qkv["q"], qkv["k"], qkv["v"], sel["idx"], sel["depth_off"], cu,
                                    theta)
    rows = sel["row_of"][:, n - 1]                           # rows (d, n - 1), d = 0..K-1
    assert (rows >= 0).all()
    q, k, v = to_f64(qkv["q"]), to_f64(qkv["k"]), to_f64(qkv["v"])
    ctx = sel["row_of"][0, : n - 1]                          # depth-0 rows of positions 0..n-2
    kc = rope.rotate(k[ctx], np.arange(n - 1), theta)
    got = decode.decode_attention_f64(kc, v[ctx], np.array([0, n - 1]), q[rows][None], k[rows][None],
                                      v[rows][None], theta)
    np.testing.assert_allclose(got["out"][0], fwd["out"][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"][0], fwd["lse"][:, rows].T, rtol=0, atol=1e-12)


def test_empty_cache_single_row_is_the_anchor_alone():
    _, _, _, q, k, v = _inputs(5, [0], 1, 4, 2, 16)
    theta = 1.0e4
    got = decode.decode_attention_f64(np.zeros((0, 2, 16)), np.zeros((0, 2, 16)), np.array([0, 0]),
                                      q, k, v, theta)
    # one key: out = its value; lse = its scaled score (position 0: no rotation)
    for h in range(4):
        np.testing.assert_allclose(got["out"][0, 0, h], v[0, 0, h // 2], rtol=0, atol=1e-14)
        np.testing.assert_allclose(got["lse"][0, 0, h], q[0, 0, h] @ k[0, 0, h // 2] / 4.0,
                                   rtol=0, atol=1e-12)


def test_requests_are_independent():
    lens = [17, 3, 40]
    kc, vc, cu, q, k, v = _inputs(7, lens, 5, 4, 1, 32)
    theta = 5.0e5
    batch = decode.decode_attention_f64(kc, vc, cu, q, k, v, theta)
    for b in range(len(lens)):
        one = decode.decode_attention_f64(kc[cu[b]:cu[b + 1]], vc[cu[b]:cu[b + 1]],
                                          np.array([0, lens[b]]), q[b:b + 1], k[b:b + 1],
                                          v[b:b + 1], theta)
        np.testing.assert_allclose(batch["out"][b], one["out"][0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(batch["lse"][b], one["lse"][0], rtol=0, atol=1e-13)
