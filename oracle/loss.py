"""Depth-weighted cross-entropy of the draft rows (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

Sources:

- NeMo Automodel PR 2376, description: the P-EAGLE trainer runs the parallel masked-depth
  loss with EAGLE-3's draft-vocab projection and its 0.8**d weighted-mean schedule; the
  validation section gives a starting loss of about ln(draft vocab) = ln 8192 ~ 9.0, and
  the pre-checks list out-of-draft-vocab masking.

Readings (the pages name the schedule, not the formula):

- Each draft row (d, p) has a label: the draft-vocabulary id of the token it should
  predict, or -1 when that token is outside the draft vocabulary (masked rows add nothing).
- The loss of depth d is the mean, over its unmasked rows, of the cross-entropy
  lse(logits) - logits[label] (natural log).
- The total is the weighted mean over the depths that have at least one unmasked row:
  sum_d w_d L_d / sum_d w_d with w_d = decay**d, decay = 0.8. A depth with no unmasked row
  has no loss and no weight.
- Its gradient with respect to a row's logits is w_d / (W n_d) * (softmax(logits) -
  onehot(label)) for an unmasked row of depth d (n_d its unmasked rows, W the weight sum),
  zero for a masked row.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64


def depth_weighted_ce_f64(logits, labels, depth_off, decay: float = 0.8, want_grad=True,
                          block: int = 2048, grad_rows=None) -> dict:
    """logits [T, V] (float64 or bf16 bits), labels int [T] (-1: masked), depth_off [K+1].
    Returns loss, depth_loss [K] (nan where a depth has no unmasked row), row_loss [T]
    (0 for masked rows), count [K] and, with want_grad, grad [T, V] (or, with grad_rows,
    the gradient of those rows only, for workloads too large for the whole tensor)."""
    logits = to_f64(logits) if np.asarray(logits).dtype == np.uint16 else np.asarray(logits, np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    depth_off = np.asarray(depth_off, dtype=np.int64)
    T, V = logits.shape
    K = len(depth_off) - 1
    row_loss = np.zeros(T)
    lse = np.zeros(T)
    for b0 in range(0, T, block):
        x = logits[b0:b0 + block]
        m = x.max(axis=1)
        lse[b0:b0 + block] = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    valid = (labels >= 0) & (labels < V)
    rows = np.nonzero(valid)[0]
    row_loss[rows] = lse[rows] - logits[rows, labels[rows]]
    count = np.array([int(valid[depth_off[d]:depth_off[d + 1]].sum()) for d in range(K)])
    depth_loss = np.full(K, np.nan)
    W = 0.0
    total = 0.0
    for d in range(K):
        if count[d] > 0:
            depth_loss[d] = row_loss[depth_off[d]:depth_off[d + 1]].sum() / count[d]
            W += decay ** d
            total += decay ** d * depth_loss[d]
    out = dict(loss=total / W if W > 0 else 0.0, depth_loss=depth_loss, row_loss=row_loss,
               count=count)
    if want_grad and grad_rows is not None:
        gr = np.asarray(grad_rows, dtype=np.int64)
        dep = np.searchsorted(depth_off, gr, side="right") - 1
        g = np.exp(logits[gr] - lse[gr, None])
        for i, (r, d) in enumerate(zip(gr, dep)):
            if not valid[r] or count[d] == 0:
                g[i] = 0.0
                continue
            g[i, labels[r]] -= 1.0
            g[i] *= decay ** d / (W * count[d])
        out["grad"] = g
    elif want_grad:
        grad = np.zeros((T, V))
        for d in range(K):
            if count[d] == 0:
                continue
            c = decay ** d / (W * count[d])
            for b0 in range(int(depth_off[d]), int(depth_off[d + 1]), block):
                b1 = min(int(depth_off[d + 1]), b0 + block)
                g = np.exp(logits[b0:b1] - lse[b0:b1, None])
                r = np.arange(b0, b1)
                ok = valid[r]
                g[np.nonzero(ok)[0], labels[r[ok]]] -= 1.0
                g[~ok] = 0.0
                grad[b0:b1] = c * g
        out["grad"] = grad
    return out
