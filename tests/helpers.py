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


# Bar for projections whose operands and outputs are bf16 (the first layer's q, k, v),
# derived from the arithmetic. bf16 keeps 8 significant bits, so rounding the GEMM's
# input row x moves each term by up to 2^-8 of itself (RMS about 2^-8 / sqrt(3) over a
# binade), and an output by a sum of 2H such terms: standard deviation about
# 2^-8 / sqrt(3) * ||x * W_row||, i.e. 0.0023 for unit-RMS x and W ~ N(0, 1/(2H)) (outputs
# of unit variance, the synthetic recipe), ~0.013 at the extremes of 10^6 outputs;
# storing the output as bf16 adds up to 2^-8 |q|. Hence 2e-2, absolute below magnitude 1
# and relative above it; relative L2 keeps 5e-3 (the model gives ~2.5e-3).
BF16_PROJ_MAX = 2e-2


def assert_close_bf16_out(got, want, what: str, max_abs=BF16_PROJ_MAX, max_rel_l2=MAX_REL_L2):
    """max |got - want| / max(1, |want|) <= max_abs and relative L2 <= max_rel_l2."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = got - want
    scaled = float((np.abs(diff) / np.maximum(1.0, np.abs(want))).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    assert scaled <= max_abs, f"{what}: max|diff|/max(1,|want|) {scaled:.3e} > {max_abs}"
    assert rel <= max_rel_l2, f"{what}: rel-L2 {rel:.3e} > {max_rel_l2}"
    return scaled, rel


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


def chunk_rows(depth_off, cu_seqlens, idx, group: int, seed=0, inside=1) -> np.ndarray:
    """Rows that touch every workgroup of the attention forward. The kernel visits draft
    rows in anchor-major order (all depths of an anchor, anchors ascending) and gives each
    workgroup QR = 256 / group consecutive entries of one sequence's part of that list.
    Returned: the first and last entry of every such chunk, ``inside`` seeded random
    entries of each, and every entry of the first and last chunk of the buffer."""
    rng = np.random.default_rng(seed)
    depth_off = np.asarray(depth_off, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    T = int(depth_off[-1])
    depth = np.repeat(np.arange(len(depth_off) - 1), np.diff(depth_off))
    order = np.lexsort((depth, idx))          # anchor-major: by anchor, then by depth
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    starts = np.searchsorted(idx[order], cu, side="left")   # list entry of each sequence start
    QR = 256 // group
    rows = []
    chunks = []
    for s in range(len(cu) - 1):
        a, b = int(starts[s]), int(starts[s + 1])
        for c0 in range(a, b, QR):
            chunks.append((c0, min(c0 + QR, b)))
    for c0, c1 in chunks:
        rows += [c0, c1 - 1]
        rows += rng.integers(c0, c1, size=inside).tolist()
    if chunks:
        for c0, c1 in (chunks[0], chunks[-1]):
            rows += list(range(c0, c1))
    ent = np.unique(np.asarray(rows, dtype=np.int64))
    return np.unique(order[ent[(ent >= 0) & (ent < T)]])


# Sampling verification decides integers from fp32 arithmetic. A depth's decision is
# compared with float64 unless u lies within SPEC_RATIO_TOL (relative) of p / q, and the
# resampled token unless w * Z lies within SPEC_CDF_TOL (absolute, probability units) of a
# boundary of the residual's running sum; inside those windows either side is valid.
SPEC_RATIO_TOL = 1e-4
SPEC_CDF_TOL = 1e-5


def check_sampled(inp: dict, tau: float, got_len, got_next, ratio_tol=SPEC_RATIO_TOL,
                  cdf_tol=SPEC_CDF_TOL, drafts=None) -> dict:
    """Check accept_len / next_tok of sampling verification against the float64 oracle on
    the drafts listed (all by default); target logits with K + 1 rows check the bonus draw. Exact wherever the oracle's decisions are clear of
    the windows above; elsewhere the kernel's decisions must lie inside them. Returns
    counts and the largest miss of each kind (0 for a decision the oracle shares)."""
    from oracle import verify as over
    dl, tl, tok = inp["draft_logits"], inp["target_logits"], inp["draft_tok"]
    u = np.asarray(inp["u"], dtype=np.float64)
    w = np.asarray(inp["w"], dtype=np.float64)
    N, K, V = dl.shape
    drafts = range(N) if drafts is None else drafts
    sub = [int(i) for i in drafts]
    bonus = tl.shape[1] == K + 1
    want = (over.speculative_accept_bonus if bonus else over.speculative_accept)(
        dl[sub], tl[sub], tok[sub], u[sub], w[sub], tau)
    stats = dict(drafts=len(sub), exact=0, ratio_miss=0.0, cdf_miss=0.0, rejected=0)
    for j, i in enumerate(sub):
        L, t = int(got_len[i]), int(got_next[i])
        assert 0 <= L <= K, f"draft {i}: accept_len {L} outside [0, {K}]"
        ratio = want["ratio"][j]
        for d in range(L):  # accepted: u < ratio, up to the window
            miss = max(0.0, u[i, d] - ratio[d]) / max(ratio[d], 1e-300)
            stats["ratio_miss"] = max(stats["ratio_miss"], miss)
            assert miss <= ratio_tol, f"draft {i} depth {d}: accepted with u {u[i, d]} >= ratio {ratio[d]}"
        if L == K and tl.shape[1] == K:
            assert t == -1, f"draft {i}: all {K} accepted but next_tok {t}"
        elif L == K:   # bonus draw from p_K, the target's K+1-th row
            assert 0 <= t < V, f"draft {i}: bonus token {t} outside [0, {V})"
            c = np.cumsum(over.softmax_f64(tl[i, K], tau))
            theta = w[i] * c[-1]
            lo = c[t - 1] if t > 0 else 0.0
            miss = max(0.0, lo - theta, theta - c[t] if c[t] <= theta else 0.0)
            stats["cdf_miss"] = max(stats["cdf_miss"], miss)
            assert miss <= cdf_tol, (f"draft {i}: bonus token {t} spans "
                                     f"[{lo:.9g}, {c[t]:.9g}) but w*Z = {theta:.9g}")
        else:
            stats["rejected"] += 1
            miss = max(0.0, ratio[L] - u[i, L]) / max(ratio[L], 1e-300)
            stats["ratio_miss"] = max(stats["ratio_miss"], miss)
            assert miss <= ratio_tol, f"draft {i} depth {L}: rejected with u {u[i, L]} < ratio {ratio[L]}"
            assert 0 <= t < V, f"draft {i}: next_tok {t} outside [0, {V})"
            c = np.cumsum(over.residual_f64(dl[i, L], tl[i, L], tau))
            theta = w[i] * c[-1]
            lo = c[t - 1] if t > 0 else 0.0
            # token t owns the running sums in [lo, c[t]); theta must fall inside
            miss = max(0.0, lo - theta, theta - c[t] if c[t] <= theta else 0.0)
            stats["cdf_miss"] = max(stats["cdf_miss"], miss)
            assert miss <= cdf_tol, (f"draft {i} depth {L}: token {t} spans "
                                     f"[{lo:.9g}, {c[t]:.9g}) but w*Z = {theta:.9g}")
        if L == int(want["accept_len"][j]) and t == int(want["next_tok"][j]):
            stats["exact"] += 1
    return stats
