"""Multi-depth draft attention with the diagonal extension (oracle).

Sources:

- NeMo Automodel PR 2376, description: P-EAGLE reuses the EAGLE-3
  ``cache_hidden`` diagonal-extension attention, which matches vLLM's
  single-base-position decode; its parity section states that the K-step
  ``cache_hidden`` forward equals a flat parallel forward over
  [context, mask_1, ..., mask_{K-1}].
- snxtyle/P_Eagle README: packed conversations are isolated by ``cu_seqlens``
  (no attention across conversations).
- speculators P-EAGLE guide, "Architecture": all depths in one pass, depth d at
  position anchor + d.

Predicate (reading of the pages): the query of draft row (d, p, head h) may see
key row (e, p') iff

    (e == 0 and p' is in the same packed sequence as p and p' <= p)     causal context
 or (e >= 1 and p' == p and e <= d)                                     own anchor's depths 1..d

so row (d, p) sees (p - a_s + 1) + d keys. Scores are <q', k'> / sqrt(D) on the
RoPE-rotated q', k' (positions p - a_s + d, module ``rope``); q head h reads kv
head floor(h / G), G = Hq / Hkv. Softmax over the allowed keys; out = P v; lse is
the natural log of the softmax denominator of the scaled scores.

The oracle builds the explicit dense boolean mask over all T key rows for each
block of query rows and computes the softmax in float64. It never derives the
mask from a tiling.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64
from .cod import row_depths
from .rope import rotate, row_positions


def row_meta(idx, depth_off, cu_seqlens) -> dict:
    """depth, anchor, sequence id and position value of every draft row."""
    idx = np.asarray(idx, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return dict(depth=row_depths(depth_off), anchor=idx,
                seq=np.searchsorted(cu, idx, side="right") - 1,
                pos=row_positions(idx, depth_off, cu_seqlens))


def allowed_mask(meta: dict, qrows) -> np.ndarray:
    """Dense boolean mask [len(qrows), T]: may query row i see key row c."""
    qd = meta["depth"][qrows][:, None]
    qa = meta["anchor"][qrows][:, None]
    qs = meta["seq"][qrows][:, None]
    kd = meta["depth"][None, :]
    ka = meta["anchor"][None, :]
    ks = meta["seq"][None, :]
    context = (kd == 0) & (ks == qs) & (ka <= qa)
    diagonal = (kd >= 1) & (ka == qa) & (kd <= qd)
    return context | diagonal


def draft_attention(q, k, v, idx, depth_off, cu_seqlens, theta: float,
                    scale: float | None = None, rows=None, block: int = 256) -> dict:
    """out [R, Hq, D] and lse [Hq, R] (float64) for the draft rows ``rows``.

    q: bf16 bits [T, Hq, D]; k, v: bf16 bits [T, Hkv, D], all pre-RoPE.
    """
    return draft_attention_f64(to_f64(q), to_f64(k), to_f64(v), idx, depth_off, cu_seqlens,
                               theta, scale, rows, block)


def draft_attention_f64(q, k, v, idx, depth_off, cu_seqlens, theta: float,
                        scale: float | None = None, rows=None, block: int = 256) -> dict:
    """The same on float64 arrays q [T, Hq, D], k and v [T, Hkv, D] (pre-RoPE)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    meta = row_meta(idx, depth_off, cu_seqlens)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    kr = rotate(np.asarray(k, np.float64), meta["pos"], theta)   # [T, Hkv, D]
    vf = np.asarray(v, np.float64)
    out = np.empty((len(rows), Hq, D), dtype=np.float64)
    lse = np.empty((Hq, len(rows)), dtype=np.float64)
    for b0 in range(0, len(rows), block):
        br = rows[b0:b0 + block]
        mask = allowed_mask(meta, br)                      # [B, T]
        qr = rotate(np.asarray(q[br], np.float64), meta["pos"][br], theta)  # [B, Hq, D]
        for h in range(Hq):
            g = h // G
            s = (qr[:, h, :] @ kr[:, g, :].T) * scale       # [B, T]
            s = np.where(mask, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            out[b0:b0 + len(br), h, :] = (p @ vf[:, g, :]) / den
            lse[h, b0:b0 + len(br)] = mx[:, 0] + np.log(den[:, 0])
    return dict(out=out, lse=lse)


def draft_attention_backward_f64(q, k, v, idx, depth_off, cu_seqlens, theta: float, dout,
                                 scale: float | None = None, block: int = 256) -> dict:
    """Gradients of the draft attention (float64): given dout = dL/d out [T, Hq, D], returns
    dq [T, Hq, D], dk and dv [T, Hkv, D] with respect to the pre-RoPE inputs, plus dq_rot
    and dk_rot with respect to the rotated q', k'.

    With P the masked softmax of S = q' k'^T * scale (per row and head):
      dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
      dq' = dS k' * scale,  dk' = dS^T q' * scale,
    summed over the q heads sharing a kv head; dq and dk are dq', dk' rotated back (the
    transpose of the RoPE rotation at each row's position)."""
    from .rope import rotate_transpose

    q = np.asarray(q, np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    meta = row_meta(idx, depth_off, cu_seqlens)
    qr = rotate(q, meta["pos"], theta)
    kr = rotate(np.asarray(k, np.float64), meta["pos"], theta)
    vf = np.asarray(v, np.float64)
    do = np.asarray(dout, np.float64)
    dq_rot = np.zeros_like(qr)
    dk_rot = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    for b0 in range(0, T, block):
        br = np.arange(b0, min(T, b0 + block))
        mask = allowed_mask(meta, br)
        for h in range(Hq):
            g = h // G
            s = np.where(mask, (qr[br, h, :] @ kr[:, g, :].T) * scale, -np.inf)
            P = np.exp(s - s.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = do[br, h, :] @ vf[:, g, :].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq_rot[br, h, :] = (dS @ kr[:, g, :]) * scale
            dk_rot[:, g, :] += (dS.T @ qr[br, h, :]) * scale
            dv[:, g, :] += P.T @ do[br, h, :]
    return dict(dq=rotate_transpose(dq_rot, meta["pos"], theta),
                dk=rotate_transpose(dk_rot, meta["pos"], theta), dv=dv, dq_rot=dq_rot,
                dk_rot=dk_rot)


def draft_attention_backward_rows_f64(q, k, v, idx, depth_off, cu_seqlens, theta: float, dout,
                                      q_rows, k_rows, scale: float | None = None) -> dict:
    """The same gradients restricted to a subset, for workloads too large for the full
    oracle: dq of the query rows q_rows, and dk, dv of the key rows k_rows. The softmax of
    every query row involved (q_rows, and every row that sees one of k_rows) is still taken
    over all of its keys; only the outputs are restricted."""
    from .rope import rotate_transpose

    q = np.asarray(q, np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    meta = row_meta(idx, depth_off, cu_seqlens)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    kr = rotate(np.asarray(k, np.float64), meta["pos"], theta)
    vf = np.asarray(v, np.float64)
    do = np.asarray(dout, np.float64)
    # query rows that see any of k_rows
    seers = np.zeros(T, dtype=bool)
    for b0 in range(0, T, 4096):
        br = np.arange(b0, min(T, b0 + 4096))
        seers[br] = allowed_mask(meta, br)[:, k_rows].any(axis=1)
    rows = np.union1d(q_rows, np.nonzero(seers)[0])
    qr = rotate(q[rows], meta["pos"][rows], theta)
    mask = allowed_mask(meta, rows)
    pos_in = {int(r): i for i, r in enumerate(rows)}
    dq_rot = np.zeros((len(q_rows), Hq, D))
    dk_rot = np.zeros((len(k_rows), Hkv, D))
    dv = np.zeros((len(k_rows), Hkv, D))
    qi = np.array([pos_in[int(r)] for r in q_rows], dtype=np.int64)
    for h in range(Hq):
        g = h // G
        s = np.where(mask, (qr[:, h, :] @ kr[:, g, :].T) * scale, -np.inf)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = do[rows, h, :] @ vf[:, g, :].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq_rot[:, h, :] = (dS[qi] @ kr[:, g, :]) * scale
        dk_rot[:, g, :] += (dS[:, k_rows].T @ qr[:, h, :]) * scale
        dv[:, g, :] += P[:, k_rows].T @ do[rows, h, :]
    return dict(dq=rotate_transpose(dq_rot, meta["pos"][q_rows], theta),
                dk=rotate_transpose(dk_rot, meta["pos"][k_rows], theta), dv=dv)


def draft_attention_backward(q, k, v, idx, depth_off, cu_seqlens, theta: float, dout,
                             scale: float | None = None) -> dict:
    """Same on the library's input formats: q, k, v bf16 bits, dout float32."""
    return draft_attention_backward_f64(to_f64(q), to_f64(k), to_f64(v), idx, depth_off,
                                        cu_seqlens, theta, dout, scale)


def useful_pairs(idx, depth_off, cu_seqlens) -> int:
    """Number of allowed (query row, key row) pairs per head: sum of (p - a_s + 1) + d."""
    meta = row_meta(idx, depth_off, cu_seqlens)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return int(np.sum(meta["anchor"] - cu[meta["seq"]] + 1 + meta["depth"]))
