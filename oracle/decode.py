"""Draft attention at inference: one base position per request over a KV cache (oracle).

TEST INFRASTRUCTURE ONLY (see the package header).

Sources:

- NeMo Automodel PR 2376, parity section: at inference vLLM runs one flat parallel
  forward over [context, mask_1, ..., mask_{K-1}], and the K-step ``cache_hidden``
  training forward equals it.
- speculators P-EAGLE guide, "Inference Process": all depths are drafted in one
  pass, the target verifies them, the longest correct prefix is accepted, and
  drafting repeats from the last accepted token.

Readings:

- Request b has a context of L_b tokens whose keys and values are already in the
  KV cache, the keys rotated at their positions 0 .. L_b - 1. Its anchor (the last
  accepted token) is the first of K new rows: new row d sits at position L_b + d
  (the anchor at L_b, mask row d at L_b + d), the base position of the flat layout.
- New row d attends to every cache key of its request and to new rows 0 .. d:
  causal attention over the flat sequence [context, anchor, mask_1 .. mask_{K-1}].
  This is the forward's predicate with a single anchor (module ``attention``).
- q and k of the new rows are pre-RoPE and rotated here (rotate-half, position
  value, module ``rope``); cache keys are taken as given. v is never rotated.
  Scale 1/sqrt(D); q head h reads kv head floor(h / G).
- Outputs: out [B, K, Hq, D] and lse [B, K, Hq] (natural log of the softmax
  denominator of the scaled scores), float64.
"""
from __future__ import annotations

import numpy as np

from .bf16 import to_f64
from .rope import rotate


def decode_attention_f64(k_cache, v_cache, cu_ctx, q_new, k_new, v_new, theta: float,
                         scale: float | None = None) -> dict:
    """The computation on float64 arrays: k_cache, v_cache [Ltot, Hkv, D] (keys already
    rotated), q_new [B, K, Hq, D], k_new, v_new [B, K, Hkv, D] (pre-RoPE)."""
    cu = np.asarray(cu_ctx, dtype=np.int64)
    B, K, Hq, D = q_new.shape
    Hkv = k_new.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((B, K, Hq, D), dtype=np.float64)
    lse = np.empty((B, K, Hq), dtype=np.float64)
    for b in range(B):
        L = int(cu[b + 1] - cu[b])
        pos = L + np.arange(K)
        qr = rotate(q_new[b], pos, theta)                      # [K, Hq, D]
        kr = rotate(k_new[b], pos, theta)                      # [K, Hkv, D]
        keys = np.concatenate([k_cache[cu[b]:cu[b + 1]], kr], axis=0)        # [L + K, Hkv, D]
        vals = np.concatenate([v_cache[cu[b]:cu[b + 1]], v_new[b]], axis=0)
        # row d: all L cache keys, new keys e <= d
        e = np.arange(K)
        allowed = np.concatenate([np.ones((K, L), dtype=bool), e[None, :] <= e[:, None]], axis=1)
        for h in range(Hq):
            g = h // G
            s = (qr[:, h, :] @ keys[:, g, :].T) * scale        # [K, L + K]
            s = np.where(allowed, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (p @ vals[:, g, :]) / den
            lse[b, :, h] = mx[:, 0] + np.log(den[:, 0])
    return dict(out=out, lse=lse)


def decode_attention(k_cache, v_cache, cu_ctx, q_new, k_new, v_new, theta: float,
                     scale: float | None = None) -> dict:
    """Same, on bf16 bit patterns (uint16): the library's input format."""
    return decode_attention_f64(to_f64(k_cache), to_f64(v_cache), cu_ctx, to_f64(q_new),
                                to_f64(k_new), to_f64(v_new), theta, scale)
