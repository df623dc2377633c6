"""Fused input stage of the draft forward (oracle).

Source: NeMo Automodel PR 2376, description. The draft registers a learnable
``mask_hidden`` of shape [1, num_aux_hidden_states * target_hidden_size] and
projects it through the draft's fc layer; depth 0 consumes the real token and the
projected target aux hidden states, depths >= 1 consume the reserved
``ptd_token_id`` token and the projected ``mask_hidden`` with no recurrence.
The speculators P-EAGLE guide ("Architecture") states that the target hidden
states from the selected layers are concatenated and projected.

Readings: fc has no bias; the weight is stored [H, aux_dim] (output-major, as a
linear layer's weight). fc_norm (the PR projects mask_hidden "through fc/fc_norm", after
EAGLE-3.1's toggle) is off by default; when a weight is given it is an RMSNorm of the fc
output (Llama form, eps 1e-6), applied to the real and the mask projections alike. Output
``hidden`` is float64 here; the embedding rows are copies of bf16 table rows, returned as
the same bit patterns.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64
from .cod import row_depths


def fuse_inputs(aux, fc_weight, mask_hidden, tokens, embed, ptd_token_id,
                idx, depth_off, rows=None, fc_norm_weight=None, eps: float = 1e-6) -> dict:
    """hidden [R, H] float64 and embed_rows [R, H] bf16 bits for draft rows.

    rows: optional subset of draft rows (default: all T rows, in order).
    fc_norm_weight: optional bf16 bits [H] of the RMSNorm after fc.
    """
    idx = np.asarray(idx)
    T = len(idx)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    depth = row_depths(depth_off)[rows]
    anchor = idx[rows]
    W = to_f64(fc_weight)                                  # [H, A]
    y_mask = to_f64(mask_hidden) @ W.T                     # projected mask_hidden, [H]
    H = W.shape[0]
    hidden = np.empty((len(rows), H), dtype=np.float64)
    embed_rows = np.empty((len(rows), H), dtype=np.uint16)
    real = depth == 0
    if real.any():
        hidden[real] = to_f64(aux[anchor[real]]) @ W.T     # fc(aux) of the anchor
        embed_rows[real] = embed[tokens[anchor[real]]]
    if (~real).any():
        hidden[~real] = y_mask
        embed_rows[~real] = embed[ptd_token_id]
    if fc_norm_weight is not None:
        from .layer import rms_norm
        hidden = rms_norm(hidden, to_f64(fc_norm_weight), eps)
        y_mask = rms_norm(y_mask, to_f64(fc_norm_weight), eps)
    return dict(hidden=hidden, embed_rows=embed_rows, y_mask=y_mask)
