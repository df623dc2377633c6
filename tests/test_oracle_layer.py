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
