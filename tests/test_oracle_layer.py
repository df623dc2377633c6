"""Pins for the first draft layer's attention inputs (oracle/layer.py).

- RMSNorm against transformers' Llama RMSNorm (an independent implementation), and its
  closed form: with unit weight and no epsilon every output row has mean square 1 and
  points along its input.
- The concatenation order and the q/k/v head split: with selection weights the projection
  must return the normalised embedding half, the normalised hidden half, or a chosen
  slice of them, in the right heads.
- Depth >= 1 rows: identical inputs give identical q, k, v (the shortcut the GPU path
  takes is a property of the definition, not of the oracle).
"""
import numpy as np
import pytest
import torch

from oracle import layer


def _llama_rms(x, w, eps):
    from transformers.models.llama.modeling_llama import LlamaRMSNorm
    m = LlamaRMSNorm(x.shape[-1], eps=eps).double()
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(np.asarray(w, np.float64)))
        return m(torch.from_numpy(x)).numpy()


@pytest.mark.parametrize("H,eps", [(8, 1e-6), (640, 1e-6), (96, 1e-2)])
def test_rms_norm_matches_llama_rmsnorm(H, eps):
    rng = np.random.default_rng(H)
    x = rng.standard_normal((5, H)) * rng.uniform(0.01, 10, size=(5, 1))
    w = 1.0 + 0.1 * rng.standard_normal(H)
    # the library module computes in float32 internally
    np.testing.assert_allclose(layer.rms_norm(x, w, eps), _llama_rms(x, w, eps), rtol=2e-6,
                               atol=1e-7)


def test_rms_norm_closed_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 33)) * 3.0
    y = layer.rms_norm(x, np.ones(33), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    cos = np.sum(x * y, axis=-1) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(y, axis=-1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)


def test_concat_order_and_head_split():
    """H = 8, Hq = 2, Hkv = 1, D = 8: q head 0 must be the normalised embedding, q head 1
    the normalised hidden state; k selects hidden dims 4..7 then embedding dims 0..3; v
    the embedding half reversed."""
    rng = np.random.default_rng(2)
    T, H, D = 6, 8, 8
    emb, hid = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    we, wh = 1.0 + 0.2 * rng.standard_normal(H), 1.0 + 0.2 * rng.standard_normal(H)
    sel_k = np.zeros((D, 2 * H))
    for i in range(4):
        sel_k[i, H + 4 + i] = 1.0          # hidden dims 4..7
        sel_k[4 + i, i] = 1.0              # embedding dims 0..3
    sel_v = np.zeros((D, 2 * H))
    for i in range(D):
        sel_v[i, H - 1 - i] = 1.0          # embedding half, reversed
    w_qkv = np.concatenate([np.eye(2 * H), sel_k, sel_v], axis=0)
    out = layer.layer1_qkv_f64(hid, emb, we, wh, w_qkv, Hq=2, Hkv=1, D=D, eps=1e-6)
    ne, nh = _llama_rms(emb, we, 1e-6), _llama_rms(hid, wh, 1e-6)
    np.testing.assert_allclose(out["q"][:, 0], ne, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(out["q"][:, 1], nh, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(out["k"][:, 0], np.concatenate([nh[:, 4:], ne[:, :4]], axis=1),
                               rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(out["v"][:, 0], ne[:, ::-1], rtol=2e-6, atol=1e-7)


def test_identical_inputs_give_identical_rows():
    rng = np.random.default_rng(3)
    T, n, H, Hq, Hkv, D = 10, 6, 16, 2, 1, 8
    emb, hid = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    emb[n:], hid[n:] = emb[n], hid[n]       # depth >= 1 rows share their inputs
    w_qkv = rng.standard_normal(((Hq + 2 * Hkv) * D, 2 * H))
    out = layer.layer1_qkv_f64(hid, emb, np.ones(H), np.ones(H), w_qkv, Hq, Hkv, D)
    for key in ("q", "k", "v"):
        assert np.array_equal(out[key][n:], np.broadcast_to(out[key][n], out[key][n:].shape))


def _llama_layer(H, I, Hq, Hkv, D, theta, eps, w):
    """transformers' Llama decoder layer (float64, eager attention) carrying the hidden
    half of the oracle's weights."""
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as m
    cfg = LlamaConfig(hidden_size=H, intermediate_size=I, num_attention_heads=Hq,
                      num_key_value_heads=Hkv, head_dim=D, rms_norm_eps=eps,
                      attention_bias=False, mlp_bias=False,
                      rope_parameters={"rope_type": "default", "rope_theta": theta})
    cfg._attn_implementation = "eager"
    lay = m.LlamaDecoderLayer(cfg, layer_idx=0).double()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    qd, kd = Hq * D, Hkv * D
    with torch.no_grad():
        lay.input_layernorm.weight.copy_(t(w["w_norm_hidden"]))
        lay.self_attn.q_proj.weight.copy_(t(w["w_qkv"][:qd, H:]))
        lay.self_attn.k_proj.weight.copy_(t(w["w_qkv"][qd:qd + kd, H:]))
        lay.self_attn.v_proj.weight.copy_(t(w["w_qkv"][qd + kd:, H:]))
        lay.self_attn.o_proj.weight.copy_(t(w["w_o"]))
        lay.post_attention_layernorm.weight.copy_(t(w["w_post"]))
        lay.mlp.gate_proj.weight.copy_(t(w["w_gate"]))
        lay.mlp.up_proj.weight.copy_(t(w["w_up"]))
        lay.mlp.down_proj.weight.copy_(t(w["w_down"]))
    return lay, m.LlamaRotaryEmbedding(cfg)


def _weights(rng, H, I, Hq, Hkv, D, V, zero_emb_half=False):
    w = dict(w_norm_emb=1 + 0.1 * rng.standard_normal(H), w_norm_hidden=1 + 0.1 * rng.standard_normal(H),
             w_qkv=rng.standard_normal(((Hq + 2 * Hkv) * D, 2 * H)) / np.sqrt(2 * H),
             w_o=rng.standard_normal((H, Hq * D)) / np.sqrt(Hq * D),
             w_post=1 + 0.1 * rng.standard_normal(H),
             w_gate=rng.standard_normal((I, H)) / np.sqrt(H), w_up=rng.standard_normal((I, H)) / np.sqrt(H),
             w_down=rng.standard_normal((H, I)) / np.sqrt(I),
             w_final=1 + 0.1 * rng.standard_normal(H), w_head=rng.standard_normal((V, H)) / np.sqrt(H))
    if zero_emb_half:
        w["w_qkv"][:, :H] = 0.0
    return w


@pytest.mark.parametrize("n,H,I,Hq,Hkv,D,theta", [(9, 32, 48, 4, 2, 8, 1e4), (40, 64, 96, 4, 1, 16, 5e5)])
def test_layer_matches_llama_decoder_layer(n, H, I, Hq, Hkv, D, theta):
    """K = 1 (plain causal attention over one sequence), the embedding half of W_qkv zero and
    the residual on the raw hidden state: the first draft layer is a Llama decoder layer
    applied to the hidden state."""
    rng = np.random.default_rng(n)
    w = _weights(rng, H, I, Hq, Hkv, D, V=11, zero_emb_half=True)
    hidden, embed = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    idx, depth_off, cu = np.arange(n), np.array([0, n]), np.array([0, n])
    got = layer.layer1_forward_f64(hidden, embed, w, idx, depth_off, cu, theta, Hq, Hkv, D,
                                   eps=1e-6, norm_before_residual=False)
    lay, rot = _llama_layer(H, I, Hq, Hkv, D, theta, 1e-6, w)
    x = torch.from_numpy(hidden)[None]
    pos = torch.arange(n)[None]
    mask = torch.triu(torch.full((n, n), float("-inf"), dtype=torch.float64), 1)[None, None]
    with torch.no_grad():
        want = lay(x, attention_mask=mask, position_ids=pos, position_embeddings=rot(x, pos))[0].numpy()
    np.testing.assert_allclose(got["h2"], want, rtol=0, atol=2e-6 * np.abs(want).max())


def test_mlp_matches_llama_mlp_and_residual_modes():
    from transformers import LlamaConfig
    from transformers.models.llama import modeling_llama as m
    rng = np.random.default_rng(4)
    T, H, I, Hq, D = 6, 16, 40, 2, 8
    w = _weights(rng, H, I, Hq, 1, D, V=5)
    attn = rng.standard_normal((T, Hq, D))
    hidden = rng.standard_normal((T, H))
    post = layer.post_attention_f64(attn, hidden, w["w_o"], w["w_post"], w["w_gate"], w["w_up"],
                                    w["w_down"])
    mlp = m.LlamaMLP(LlamaConfig(hidden_size=H, intermediate_size=I, mlp_bias=False,
                                 num_attention_heads=Hq, num_key_value_heads=1)).double()
    with torch.no_grad():
        mlp.gate_proj.weight.copy_(torch.from_numpy(w["w_gate"]))
        mlp.up_proj.weight.copy_(torch.from_numpy(w["w_up"]))
        mlp.down_proj.weight.copy_(torch.from_numpy(w["w_down"]))
        m_in = _llama_rms(post["h1"], w["w_post"], 1e-6)
        want = post["h1"] + mlp(torch.from_numpy(m_in)).numpy()
    np.testing.assert_allclose(post["h2"], want, rtol=1e-5, atol=1e-6)
    # the two residual readings differ by exactly rms(hidden) - hidden in h1
    idx, depth_off, cu = np.arange(T), np.array([0, T]), np.array([0, T])
    emb = rng.standard_normal((T, H))
    w2 = _weights(rng, H, I, Hq, 1, D, V=5)
    a = layer.layer1_forward_f64(hidden, emb, w2, idx, depth_off, cu, 1e4, Hq, 1, D,
                                 norm_before_residual=True)
    b = layer.layer1_forward_f64(hidden, emb, w2, idx, depth_off, cu, 1e4, Hq, 1, D,
                                 norm_before_residual=False)
    np.testing.assert_allclose(a["h1"] - b["h1"], _llama_rms(hidden, w2["w_norm_hidden"], 1e-6) - hidden,
                               rtol=1e-5, atol=1e-6)


def test_head_argmax_lowest_index_on_ties():
    rng = np.random.default_rng(6)
    T, H, V = 5, 8, 7
    h2 = rng.standard_normal((T, H))
    w_final = np.ones(H)
    w_head = np.zeros((V, H))
    # rows of W_head equal to a unit vector e_j give logits rms(h2)_j; tokens 2 and 5 tie
    w_head[2, 3] = w_head[5, 3] = 1.0
    w_head[4, 1] = 1.0
    out = layer.draft_head_f64(h2, w_final, w_head, eps=1e-6)
    nh = _llama_rms(h2, w_final, 1e-6)
    want = np.where(nh[:, 3] >= np.maximum(nh[:, 1], 0.0), 2, np.where(nh[:, 1] > 0.0, 4, 0))
    np.testing.assert_allclose(out["logits"][:, 2], nh[:, 3], rtol=2e-6)
    assert np.array_equal(out["tokens"], want)


def _stacked_weights(rng, H, I, Hq, Hkv, D):
    return dict(w_norm=1 + 0.1 * rng.standard_normal(H),
                w_qkv=rng.standard_normal(((Hq + 2 * Hkv) * D, H)) / np.sqrt(H),
                w_o=rng.standard_normal((H, Hq * D)) / np.sqrt(Hq * D),
                w_post=1 + 0.1 * rng.standard_normal(H),
                w_gate=rng.standard_normal((I, H)) / np.sqrt(H),
                w_up=rng.standard_normal((I, H)) / np.sqrt(H),
                w_down=rng.standard_normal((H, I)) / np.sqrt(I))


def _as_first_layer_weights(w, H):
    """The stacked layer's weights in the first layer's slots, the embedding half of
    W_qkv zero, so that (with the raw residual) the first layer computes the same layer."""
    w1 = dict(w)
    w1["w_norm_hidden"] = w["w_norm"]
    w1["w_norm_emb"] = np.ones(H)
    w1["w_qkv"] = np.concatenate([np.zeros_like(w["w_qkv"]), w["w_qkv"]], axis=1)
    return w1


def _multi_depth_layout(cu, R):
    """Draft rows of nested retained sets R[d] (R[0] = every position); returns idx,
    depth_off and, per row, its depth, anchor and position value p - a_s + d."""
    idx = np.concatenate([np.asarray(r, dtype=np.int64) for r in R])
    depth_off = np.concatenate([[0], np.cumsum([len(r) for r in R])])
    depth = np.concatenate([np.full(len(r), d) for d, r in enumerate(R)])
    start = np.asarray(cu)[np.searchsorted(cu, idx, side="right") - 1]
    return idx, depth_off, depth, idx - start + depth, start


@pytest.mark.parametrize("cu,R", [
    ([0, 12], [range(12), [1, 4, 5, 9, 11], [4, 9]]),
    ([0, 5, 12], [range(12), [0, 3, 4, 6, 10, 11], [3, 6, 11], [6]]),
])
def test_stacked_layer_matches_llama_decoder_layer_with_depth_mask(cu, R):
    """A stacked layer is a Llama decoder layer over the draft rows, with RoPE at the rows'
    position values and, as its attention mask, the multi-depth predicate written out
    here pair by pair: row (d, p) sees depth-0 rows of its own sequence at p' <= p and the
    rows (d', p) of its own anchor for 1 <= d' <= d."""
    H, I, Hq, Hkv, D, theta = 32, 48, 4, 2, 8, 1e4
    rng = np.random.default_rng(len(R))
    w = _stacked_weights(rng, H, I, Hq, Hkv, D)
    idx, depth_off, depth, pos, start = _multi_depth_layout(cu, R)
    T = len(idx)
    h = rng.standard_normal((T, H))
    got = layer.layer_forward_f64(h, w, idx, depth_off, np.asarray(cu), theta, Hq, Hkv, D)
    allowed = np.zeros((T, T), dtype=bool)
    for r in range(T):
        for c in range(T):
            same_seq = start[c] == start[r]
            allowed[r, c] = (depth[c] == 0 and same_seq and idx[c] <= idx[r]) or \
                (idx[c] == idx[r] and 1 <= depth[c] <= depth[r])
    w1 = _as_first_layer_weights(w, H)
    lay, rot = _llama_layer(H, I, Hq, Hkv, D, theta, 1e-6, w1)
    x = torch.from_numpy(h)[None]
    p = torch.from_numpy(pos)[None]
    mask = torch.from_numpy(np.where(allowed, 0.0, -np.inf))[None, None]
    with torch.no_grad():
        want = lay(x, attention_mask=mask, position_ids=p, position_embeddings=rot(x, p))[0].numpy()
    np.testing.assert_allclose(got["h2"], want, rtol=0, atol=2e-6 * np.abs(want).max())


def test_stack_matches_llama_layers_in_sequence():
    """K = 1 and the first layer reduced to a plain Llama layer (embedding half of W_qkv
    zero, raw residual): the draft stack is transformers' decoder layers applied in turn,
    then RMSNorm and the head's argmax."""
    n, H, I, Hq, Hkv, D, theta, V = 10, 32, 48, 4, 2, 8, 1e4, 13
    rng = np.random.default_rng(7)
    ws = [_stacked_weights(rng, H, I, Hq, Hkv, D) for _ in range(3)]
    w1 = _as_first_layer_weights(ws[0], H)
    w1["w_final"] = 1 + 0.1 * rng.standard_normal(H)
    w1["w_head"] = rng.standard_normal((V, H)) / np.sqrt(H)
    hidden, embed = rng.standard_normal((n, H)), rng.standard_normal((n, H))
    idx, depth_off, cu = np.arange(n), np.array([0, n]), np.array([0, n])
    got = layer.stack_forward_f64(hidden, embed, w1, ws[1:], idx, depth_off, cu, theta, Hq, Hkv,
                                  D, norm_before_residual=False)
    x = torch.from_numpy(hidden)[None]
    pos = torch.arange(n)[None]
    mask = torch.triu(torch.full((n, n), float("-inf"), dtype=torch.float64), 1)[None, None]
    with torch.no_grad():
        for wl in ws:
            lay, rot = _llama_layer(H, I, Hq, Hkv, D, theta, 1e-6, _as_first_layer_weights(wl, H))
            y = lay(x, attention_mask=mask, position_ids=pos, position_embeddings=rot(x, pos))
            x = y[0] if isinstance(y, tuple) else y     # [1, n, H] either way
    want_h = x[0].numpy()
    assert len(got["h"]) == 3
    np.testing.assert_allclose(got["h"][-1], want_h, rtol=0, atol=2e-6 * np.abs(want_h).max())
    norm = want_h / np.sqrt(np.mean(want_h ** 2, axis=-1, keepdims=True) + 1e-6) * w1["w_final"]
    np.testing.assert_array_equal(got["tokens"], np.argmax(norm @ w1["w_head"].T, axis=-1))
