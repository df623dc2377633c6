"""Shared test plumbing: device transfer, tolerance checks, workload cases."""
from __future__ import annotations

import numpy as np

# Floating-point parity bar for projection and attention outputs.
MAX_ABS = 1e-2
MAX_REL_L2 = 5e-3


def to_dev(a: np.ndarray):
    """numpy -> CUDA tensor; bf16 bit patterns (uint16) travel as int16."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    a = t.detach().cpu().numpy()
    if t.dtype == torch.int16:
        a = a.view(np.uint16)
    return a


def assert_close(got, want, what: str, max_abs=MAX_ABS, max_rel_l2=MAX_REL_L2):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = got - want
    mabs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    assert mabs <= max_abs, f"{what}: max|diff| {mabs:.3e} > {max_abs}"
    assert rel <= max_rel_l2, f"{what}: rel-L2 {rel:.3e} > {max_rel_l2}"
    return mabs, rel


def sample_rows(depth_off, cu_seqlens, idx, count=96, seed=0) -> np.ndarray:
    """Rows the oracle recomputes at full size: both ends of every depth, the rows of
    each sequence's first and last anchor, and a seeded random spread."""
    rng = np.random.default_rng(seed)
    depth_off = np.asarray(depth_off)
    T = int(depth_off[-1])
    rows = set()
    for d in range(len(depth_off) - 1):
        a, b = int(depth_off[d]), int(depth_off[d + 1])
        rows.update(range(a, min(a + 4, b)))
        rows.update(range(max(a, b - 4), b))
    idx = np.asarray(idx)
    for c in np.asarray(cu_seqlens)[:-1]:
        hit = np.nonzero(idx == c)[0]
        rows.update(hit.tolist())
        hit = np.nonzero(idx == c - 1)[0]
        rows.update(hit.tolist())
    rows.update(rng.integers(0, T, size=count).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T), dtype=np.int64)
