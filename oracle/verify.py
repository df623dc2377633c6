"""Greedy verification and the longest accepted prefix (oracle).

Source: speculators P-EAGLE guide, "Inference Process": the drafter proposes all
depths in one pass, the target verifies all draft tokens in one forward pass, and
the longest correct prefix is accepted.

Readings: greedy decoding, so a draft token is correct iff it equals the target's
argmax at the same depth; draft and target share one vocabulary (identity map);
argmax takes the lowest index among equal maxima. Logits are bf16; the decision
is taken on their exact values (float32 upcast is exact).
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f32


def argmax_rows(logits_bits: np.ndarray, chunk: int = 64) -> np.ndarray:
    """int32 [N, K]: first index of the maximum of every [.., .., V] row."""
    N, K, V = logits_bits.shape
    out = np.empty((N, K), dtype=np.int32)
    for lo in range(0, N, chunk):
        x = to_f32(logits_bits[lo:lo + chunk])
        out[lo:lo + chunk] = np.argmax(x, axis=-1)   # numpy returns the first maximum
    return out


def accept_lengths(draft_tok: np.ndarray, target_tok: np.ndarray) -> np.ndarray:
    """Number of leading depths whose draft token equals the target token."""
    N, K = draft_tok.shape
    L = np.empty(N, dtype=np.int32)
    for i in range(N):
        length = 0
        while length < K and draft_tok[i, length] == target_tok[i, length]:
            length += 1
        L[i] = length
    return L


def verify(draft_logits, target_logits) -> dict:
    a = argmax_rows(draft_logits)
    b = argmax_rows(target_logits)
    return dict(draft_tok=a, target_tok=b, accept_len=accept_lengths(a, b))
