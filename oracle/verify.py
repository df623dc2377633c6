"""Greedy verification and the longest accepted prefix (oracle).

Source: speculators P-EAGLE guide, "Inference Process": the drafter proposes all
depths in one pass, the target verifies all draft tokens in one forward pass, and
the longest correct prefix is accepted.

Readings: greedy decoding, so a draft token is correct iff it equals the target's
argmax at the same depth; draft and target share one vocabulary (identity map);
argmax takes the lowest index among equal maxima. Logits are bf16; the decision
is taken on their exact values (float32 upcast is exact).

Draft vocabulary smaller than the target's (NeMo Automodel PR 2376: a draft vocabulary
of 8192 in its validation run, and out-of-draft-vocab masking among its checks): the
draft head scores Vd draft ids; a table d2t gives the target id of each draft id; a
draft token is correct iff its target id equals the target's argmax over the Vt target
ids. A target argmax outside the table's image can never be matched. (The pages name
the map, not its encoding; a plain table of target ids is taken here.)

Sampling acceptance (snxtyle/P_Eagle README, "How Speculative Decoding Works", step 6:
accepted tokens are used, rejected tokens resampled), read as speculative sampling:
p = softmax(target logits / tau) and q = softmax(draft logits / tau) at each depth; the
drafter's token x_d (sampled from q, an input here) is accepted while u_d < p(x_d) / q(x_d)
for the given uniforms u_d; at the first rejected depth j the next token is drawn from
the residual max(0, p_j - q_j) (normalised) by inverse CDF: the smallest t whose
cumulative residual exceeds w * Z, Z the residual's total, w a given uniform. When all K
depths are accepted the next token is -1 in ``speculative_accept``. With a K+1-th target
row (the target's distribution after the last drafted token, which the target's one
verification pass also yields), ``speculative_accept_bonus`` draws that extra token from
p_K = softmax(target row K / tau) by the same inverse CDF with w, so every draft then
emits accept_len + 1 tokens.
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


def verify_d2t(draft_logits, target_logits, d2t) -> dict:
    """draft_logits [N, K, Vd], target_logits [N, K, Vt] (bf16 bits), d2t int [Vd].
    draft_tok holds draft ids; the comparison uses d2t[draft_tok]."""
    a = argmax_rows(draft_logits)
    b = argmax_rows(target_logits)
    mapped = np.asarray(d2t, dtype=np.int64)[a]
    return dict(draft_tok=a, target_tok=b, accept_len=accept_lengths(mapped, b))


def softmax_f64(logits_bits, tau: float) -> np.ndarray:
    x = to_f32(logits_bits).astype(np.float64) / float(tau)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def residual_f64(draft_row_bits, target_row_bits, tau: float) -> np.ndarray:
    """max(0, p - q) of one depth (unnormalised)."""
    return np.maximum(0.0, softmax_f64(target_row_bits, tau) - softmax_f64(draft_row_bits, tau))


def speculative_accept(draft_logits, target_logits, draft_tok, u, w, tau: float = 1.0) -> dict:
    """draft_logits, target_logits [N, K, V] bf16 bits; draft_tok int [N, K]; u [N, K] and
    w [N] uniforms in [0, 1). Returns accept_len [N], next_tok [N] and the ratios
    p(x_d) / q(x_d) [N, K]."""
    N, K, V = draft_logits.shape
    ratio = np.empty((N, K), dtype=np.float64)
    accept = np.empty(N, dtype=np.int32)
    nxt = np.full(N, -1, dtype=np.int32)
    for i in range(N):
        for d in range(K):
            x = int(draft_tok[i, d])
            p = softmax_f64(target_logits[i, d], tau)[x]
            q = softmax_f64(draft_logits[i, d], tau)[x]
            ratio[i, d] = p / q
        L = 0
        while L < K and u[i, L] < ratio[i, L]:
            L += 1
        accept[i] = L
        if L < K:
            r = residual_f64(draft_logits[i, L], target_logits[i, L], tau)
            c = np.cumsum(r)
            nxt[i] = int(np.searchsorted(c, w[i] * c[-1], side="right"))
    return dict(accept_len=accept, next_tok=nxt, ratio=ratio)


def speculative_accept_bonus(draft_logits, target_logits, draft_tok, u, w, tau: float = 1.0) -> dict:
    """As ``speculative_accept`` with target_logits [N, K + 1, V]: rows 0..K-1 verify the K
    depths; when all K are accepted, next_tok is drawn from p_K = softmax(target row K / tau)
    by inverse CDF: the smallest t with p_0 + .. + p_t > w * (p_0 + .. + p_{V-1})."""
    N, K, V = draft_logits.shape
    assert target_logits.shape == (N, K + 1, V), target_logits.shape
    out = speculative_accept(draft_logits, target_logits[:, :K], draft_tok, u, w, tau)
    for i in np.nonzero(out["accept_len"] == K)[0]:
        c = np.cumsum(softmax_f64(target_logits[i, K], tau))
        out["next_tok"][i] = int(np.searchsorted(c, w[i] * c[-1], side="right"))
    return out
