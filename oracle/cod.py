"""Conditional Drop-token (COD) sampling and the draft row layout (oracle).

Source: speculators P-EAGLE guide, section "COD Sampling": depth 0 keeps all n
positions; depth d keeps about n * r^d positions (r = down-sample-ratio) with a
floor set by down-sample-ratio-min; deeper depths train on fewer positions.
Defaults 0.7 and 0.2 come from that guide's "Key Parameters" table.

Readings taken where the page is not exact:

- count: m_d = max(round(n * r^d), round(n * r_min)), rounding half up in float64
  (floor(x + 1/2)), capped at n; so m_0 = n.
- which positions: the m_d positions whose hash SplitMix64(seed XOR p) is
  smallest, compared as unsigned 64-bit integers, with p the index in the whole
  packed buffer. Taking the m_d smallest of one ranking makes the sets nested,
  R_d within R_{d-1}, which the diagonal-extension attention needs (every depth
  e <= d of an anchor kept at depth d exists).
- SplitMix64(x) is the first output of the SplitMix64 generator whose state is
  x: add the golden gamma 0x9E3779B97F4A7C15, then the variant-13 mixer
  (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014). It is a bijection on 64-bit words, so hashes never tie.
- row layout: rows are depth-major; within a depth they are ascending by anchor.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(x: int) -> int:
    """First SplitMix64 output from state x (Python integers, mod 2^64)."""
    z = (x + GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def position_hashes(n: int, seed: int) -> list:
    """h[p] = SplitMix64(seed XOR p) for every buffer index p in [0, n)."""
    seed &= MASK64
    return [splitmix64(seed ^ p) for p in range(n)]


def retained_counts(n: int, K: int, r: float, r_min: float) -> list:
    """m_d for d in [0, K): max(round(n r^d), round(n r_min)), capped at n."""
    floor_count = math.floor(n * r_min + 0.5)
    m = []
    for d in range(K):
        geometric = math.floor(n * (r ** d) + 0.5)
        m.append(min(n, max(geometric, floor_count)))
    return m


def cod_select(n: int, K: int, r: float, r_min: float, seed: int, cu_seqlens) -> dict:
    """Retained sets and the draft row layout.

    Returns:
      m            list of K counts
      idx          int32 [T]: anchors, depth-major, ascending within a depth
      depth_off    int32 [K+1]: first row of each depth (prefix sum of m)
      cu_seqlens_d int32 [K, S+1]: kept anchors of depth d before each sequence start
      row_of       int32 [K, n]: draft row of (d, p), or -1 if p is not kept at d
    """
    cu = [int(c) for c in cu_seqlens]
    m = retained_counts(n, K, r, r_min)
    h = position_hashes(n, seed)
    order = sorted(range(n), key=lambda p: h[p])   # Python ints: unsigned order
    rank = [0] * n
    for i, p in enumerate(order):
        rank[p] = i
    idx, depth_off = [], [0]
    row_of = np.full((K, n), -1, dtype=np.int32)
    cu_d = np.zeros((K, len(cu)), dtype=np.int32)
    for d in range(K):
        kept = [p for p in range(n) if rank[p] < m[d]]   # ascending by p
        for j, p in enumerate(kept):
            row_of[d, p] = depth_off[d] + j
        for s, start in enumerate(cu):
            cu_d[d, s] = sum(1 for p in kept if p < start)
        idx.extend(kept)
        depth_off.append(depth_off[d] + len(kept))
    return dict(m=m, idx=np.array(idx, dtype=np.int32),
                depth_off=np.array(depth_off, dtype=np.int32),
                cu_seqlens_d=cu_d, row_of=row_of)


def row_depths(depth_off) -> np.ndarray:
    """Depth of every draft row."""
    K = len(depth_off) - 1
    out = np.empty(int(depth_off[-1]), dtype=np.int64)
    for d in range(K):
        out[depth_off[d]:depth_off[d + 1]] = d
    return out
