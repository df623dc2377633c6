"""The draft decoder layers (oracle): the first layer's attention inputs, attention, output
projection and MLP, the layers stacked after it, and the draft-vocab head.

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
- After the attention (module ``attention``), the layer is a Llama decoder layer's second
  half: h1 = r + o W_o^T with o the attention output flattened over heads; h2 = h1 +
  W_down (silu(W_gate m) * (W_up m)) with m = rms(h1; w_post) (SwiGLU MLP, bias-free).
- The residual r: the speculators guide ("Key Parameters") lists a flag that disables
  normalization before the residual connection, so by default the residual stream starts
  from the normalised hidden state, r = rms(hidden; w_hidden); with the flag off it is the
  raw hidden state.
- Layers stacked after the first (speculators guide, "Key Parameters": the number of
  decoder layers is a parameter) are plain Llama decoder layers on the draft rows: the
  residual stream h is the previous layer's h2, x = rms(h; w_norm), q, k, v = x W_qkv^T
  (W_qkv of shape ((Hq + 2 Hkv) D, H)), the same RoPE, rows and attention predicate as the
  first layer, then h1 = h + o W_o^T and the same MLP. The head reads the last layer's h2.
- The draft-vocab head: logits = rms(h2; w_final) W_head^T (NeMo PR 2376: the P-EAGLE
  trainer shares EAGLE-3's draft-vocab projection); the draft token of a row is its
  argmax, lowest index on ties.
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


def silu(x):
    return x / (1.0 + np.exp(-x))


def post_attention_f64(attn_out, resid, w_o, w_post, w_gate, w_up, w_down,
                       eps: float = EPS) -> dict:
    """attn_out [T, Hq, D]; resid [T, H]; w_o [H, Hq D]; w_post [H]; w_gate, w_up [I, H];
    w_down [H, I]. Returns h1 (after the attention residual) and h2 (after the MLP's)."""
    a = np.asarray(attn_out, np.float64)
    h1 = np.asarray(resid, np.float64) + a.reshape(a.shape[0], -1) @ np.asarray(w_o, np.float64).T
    m = rms_norm(h1, w_post, eps)
    g = m @ np.asarray(w_gate, np.float64).T
    u = m @ np.asarray(w_up, np.float64).T
    h2 = h1 + (silu(g) * u) @ np.asarray(w_down, np.float64).T
    return dict(h1=h1, h2=h2)


def draft_head_f64(h2, w_final, w_head, eps: float = EPS) -> dict:
    """logits [T, V] = rms(h2; w_final) W_head^T and the argmax token of each row (lowest
    index on ties)."""
    logits = rms_norm(h2, w_final, eps) @ np.asarray(w_head, np.float64).T
    return dict(logits=logits, tokens=np.argmax(logits, axis=-1).astype(np.int32))


def layer1_forward_f64(hidden, embed, w: dict, idx, depth_off, cu_seqlens, theta: float,
                       Hq: int, Hkv: int, D: int, eps: float = EPS,
                       norm_before_residual: bool = True, rows=None) -> dict:
    """The whole first layer on float64 arrays: hidden, embed [T, H] of the draft rows;
    w holds w_norm_emb, w_norm_hidden, w_qkv, w_o, w_post, w_gate, w_up, w_down, w_final,
    w_head. rows: optional subset of draft rows whose outputs are wanted (the attention
    still sees every key row)."""
    from .attention import draft_attention_f64

    qkv = layer1_qkv_f64(hidden, embed, w["w_norm_emb"], w["w_norm_hidden"], w["w_qkv"], Hq, Hkv,
                         D, eps)
    att = draft_attention_f64(qkv["q"], qkv["k"], qkv["v"], idx, depth_off, cu_seqlens, theta,
                              rows=rows)
    sel = np.arange(len(hidden)) if rows is None else np.asarray(rows)
    resid = rms_norm(hidden[sel], w["w_norm_hidden"], eps) if norm_before_residual else \
        np.asarray(hidden, np.float64)[sel]
    post = post_attention_f64(att["out"], resid, w["w_o"], w["w_post"], w["w_gate"], w["w_up"],
                              w["w_down"], eps)
    head = draft_head_f64(post["h2"], w["w_final"], w["w_head"], eps)
    return dict(q=qkv["q"], k=qkv["k"], v=qkv["v"], attn=att["out"], h1=post["h1"],
                h2=post["h2"], logits=head["logits"], tokens=head["tokens"])


def layer_qkv_f64(h, w_norm, w_qkv, Hq: int, Hkv: int, D: int, eps: float = EPS) -> dict:
    """A stacked layer's attention inputs: h [T, H] (the residual stream); w_norm [H];
    w_qkv [(Hq + 2 Hkv) D, H]. Returns q [T, Hq, D], k and v [T, Hkv, D] before RoPE."""
    y = rms_norm(h, w_norm, eps) @ np.asarray(w_qkv, np.float64).T
    T = y.shape[0]
    return dict(q=y[:, :Hq * D].reshape(T, Hq, D),
                k=y[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D),
                v=y[:, (Hq + Hkv) * D:].reshape(T, Hkv, D))


def layer_forward_f64(h, w: dict, idx, depth_off, cu_seqlens, theta: float, Hq: int, Hkv: int,
                      D: int, eps: float = EPS, rows=None) -> dict:
    """One stacked layer on float64 arrays. w holds w_norm, w_qkv, w_o, w_post, w_gate,
    w_up, w_down. rows: optional subset of rows whose outputs are wanted."""
    from .attention import draft_attention_f64

    h = np.asarray(h, np.float64)
    qkv = layer_qkv_f64(h, w["w_norm"], w["w_qkv"], Hq, Hkv, D, eps)
    att = draft_attention_f64(qkv["q"], qkv["k"], qkv["v"], idx, depth_off, cu_seqlens, theta,
                              rows=rows)
    sel = np.arange(len(h)) if rows is None else np.asarray(rows)
    post = post_attention_f64(att["out"], h[sel], w["w_o"], w["w_post"], w["w_gate"], w["w_up"],
                              w["w_down"], eps)
    return dict(q=qkv["q"], k=qkv["k"], v=qkv["v"], attn=att["out"], h1=post["h1"],
                h2=post["h2"])


def stack_forward_f64(hidden, embed, w_first: dict, w_layers, idx, depth_off, cu_seqlens,
                      theta: float, Hq: int, Hkv: int, D: int, eps: float = EPS,
                      norm_before_residual: bool = True) -> dict:
    """The first layer, then each stacked layer of w_layers in order, then the head
    (w_final, w_head of w_first). Returns every layer's h2 and the head's logits and
    tokens."""
    first = layer1_forward_f64(hidden, embed, w_first, idx, depth_off, cu_seqlens, theta, Hq, Hkv,
                               D, eps, norm_before_residual)
    hs = [first["h2"]]
    for wl in w_layers:
        hs.append(layer_forward_f64(hs[-1], wl, idx, depth_off, cu_seqlens, theta, Hq, Hkv, D,
                                    eps)["h2"])
    head = draft_head_f64(hs[-1], w_first["w_final"], w_first["w_head"], eps)
    return dict(h=hs, logits=head["logits"], tokens=head["tokens"])
