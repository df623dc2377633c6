"""Attention inputs of the first draft decoder layer (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

Sources:

- snxtyle/P_Eagle README, "How Speculative Decoding Works", step 3 (EAGLE-3 injection):
  the drafter's input is the concatenation [embeddings ⊕ hidden].
- speculators P-EAGLE guide, "Architecture": the projected target hidden states pass
  through Llama-style decoder layers.
- NeMo Automodel PR 2376, changelog: depths >= 1 consume the ptd token and the projected
  mask_hidden placeholder, with no recurrence.

Readings (the pages name the pieces, not their formulas):

- RMSNorm as in Llama: y = x / sqrt(mean(x^2) + eps) * w, eps = 1e-6; the embedding half
  and the hidden half each have their own weight vector.
- The layer's attention input is x = [rms(emb; w_emb) ⊕ rms(hidden; w_hidden)], width 2H,
  the embedding half first (the order the README gives).
- q, k and v are one bias-free projection of x by the stacked weight
  W_qkv = [W_q; W_k; W_v] of shape ((Hq + 2 Hkv) D, 2H), output-major (linear layout);
  q is split into Hq heads of D, k and v into Hkv heads. RoPE comes after (module rope).
- Every depth >= 1 row has the same x (the projected mask_hidden and the ptd embedding),
  so its q, k and v before RoPE are the same in every such row. The oracle does not use
  that: it projects every row.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64

EPS = 1e-6


def rms_norm(x, w, eps: float = EPS):
    """Llama RMSNorm over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def layer1_qkv_f64(hidden, embed, w_emb, w_hidden, w_qkv, Hq: int, Hkv: int, D: int,
                   eps: float = EPS) -> dict:
    """hidden, embed [T, H]; w_emb, w_hidden [H]; w_qkv [(Hq + 2 Hkv) D, 2H].
    Returns q [T, Hq, D], k and v [T, Hkv, D] (before RoPE) and x [T, 2H]."""
    x = np.concatenate([rms_norm(embed, w_emb, eps), rms_norm(hidden, w_hidden, eps)], axis=-1)
    y = x @ np.asarray(w_qkv, np.float64).T
    T = y.shape[0]
    q = y[:, :Hq * D].reshape(T, Hq, D)
    k = y[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = y[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    return dict(q=q, k=k, v=v, x=x)


def layer1_qkv(hidden_f32, embed_bf16, w_emb_bf16, w_hidden_bf16, w_qkv_bf16, Hq: int, Hkv: int,
               D: int, eps: float = EPS) -> dict:
    """Same, on the library's input formats: hidden float32 (the fused stage's output),
    embeddings and weights as bf16 bit patterns."""
    return layer1_qkv_f64(np.asarray(hidden_f32, np.float64), to_f64(embed_bf16),
                          to_f64(w_emb_bf16), to_f64(w_hidden_bf16), to_f64(w_qkv_bf16), Hq, Hkv,
                          D, eps)
