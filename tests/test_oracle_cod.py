"""Pins for the COD oracle: published SplitMix64 outputs, hand-computed counts,
brute-force selection by counting, and the structural invariants of the layout."""
import json
import os

import numpy as np
import pytest

from oracle import cod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M64 = (1 << 64) - 1


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    state = g["seed"]
    for want in g["outputs_hex"]:
        # the generator hands out mix(state + gamma) and then advances state by gamma;
        # cod.splitmix64(x) is defined as the first output from state x.
        assert cod.splitmix64(state) == int(want, 16)
        state = (state + cod.GOLDEN_GAMMA) & M64


def _unmix_xorshift(z, s):
    # inverse of z ^ (z >> s) on 64-bit words
    x = z
    for _ in range(64 // s + 1):
        x = z ^ (x >> s)
    return x


def test_splitmix64_is_a_bijection():
    # Invert the hash step by step; a bijection on 64-bit words means COD hashes never tie.
    rng = np.random.default_rng(0)
    for x in rng.integers(0, 2**63, size=200, dtype=np.uint64).tolist() + [0, M64, 1 << 63]:
        z = cod.splitmix64(x)
        z = _unmix_xorshift(z, 31)
        z = (z * pow(0x94D049BB133111EB, -1, 1 << 64)) & M64
        z = _unmix_xorshift(z, 27)
        z = (z * pow(0xBF58476D1CE4E5B9, -1, 1 << 64)) & M64
        z = _unmix_xorshift(z, 30)
        assert (z - cod.GOLDEN_GAMMA) & M64 == x


def test_retained_counts_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "cod_counts.json")))
    for c in g["cases"]:
        assert cod.retained_counts(c["n"], c["K"], c["r"], c["r_min"]) == c["m"], c


@pytest.mark.parametrize("n,K,r", [(1, 4, 1.0), (37, 5, 1.0), (300, 3, 1.0)])
def test_ratio_one_keeps_everything(n, K, r):
    out = cod.cod_select(n, K, r, 0.2, seed=11, cu_seqlens=[0, n])
    assert out["m"] == [n] * K
    for d in range(K):
        assert out["idx"][out["depth_off"][d]:out["depth_off"][d + 1]].tolist() == list(range(n))


def _brute_kept(n, m_d, seed):
    """p is kept iff fewer than m_d positions have a strictly smaller (unsigned) hash."""
    h = [cod.splitmix64((seed & M64) ^ p) for p in range(n)]
    return [p for p in range(n) if sum(1 for q in range(n) if h[q] < h[p]) < m_d]


@pytest.mark.parametrize("n,K,r,r_min,seed", [(40, 4, 0.7, 0.2, 1), (33, 6, 0.6, 0.0, 2**63 + 5),
                                             (17, 3, 0.5, 0.3, 12345), (5, 8, 0.7, 0.2, 7)])
def test_selection_matches_brute_force_counting(n, K, r, r_min, seed):
    out = cod.cod_select(n, K, r, r_min, seed, [0, n])
    for d in range(K):
        got = out["idx"][out["depth_off"][d]:out["depth_off"][d + 1]].tolist()
        assert got == _brute_kept(n, out["m"][d], seed)


@pytest.mark.parametrize("cu", [[0, 64], [0, 10, 25, 64], [0, 1, 2, 63, 64]])
def test_layout_invariants(cu):
    n, K = cu[-1], 5
    out = cod.cod_select(n, K, 0.7, 0.2, seed=3, cu_seqlens=cu)
    m, idx, off, cu_d, row_of = out["m"], out["idx"], out["depth_off"], out["cu_seqlens_d"], out["row_of"]
    assert len(m) == K and m[0] == n
    assert off.tolist() == [sum(m[:d]) for d in range(K + 1)]
    prev = set(range(n))
    for d in range(K):
        kept = idx[off[d]:off[d + 1]].tolist()
        assert len(kept) == m[d]
        assert kept == sorted(set(kept))                 # ascending, no duplicates
        assert set(kept) <= prev                         # nested
        prev = set(kept)
        for j, p in enumerate(kept):
            assert row_of[d, p] == off[d] + j
        assert int((row_of[d] >= 0).sum()) == m[d]
        for s, start in enumerate(cu):
            assert cu_d[d, s] == len([p for p in kept if p < start])
        assert cu_d[d, -1] == m[d]


def test_hash_is_over_global_index_in_packed_buffer():
    # one ranking over the whole buffer: packing does not change which indices are kept
    a = cod.cod_select(64, 4, 0.7, 0.2, seed=9, cu_seqlens=[0, 64])
    b = cod.cod_select(64, 4, 0.7, 0.2, seed=9, cu_seqlens=[0, 20, 41, 64])
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["row_of"], b["row_of"])


def test_empty_depths():
    out = cod.cod_select(4, 3, 0.1, 0.0, seed=1, cu_seqlens=[0, 4])
    assert out["m"] == [4, 0, 0]
    assert out["depth_off"].tolist() == [0, 4, 4, 4]
    assert (out["row_of"][1:] == -1).all()
