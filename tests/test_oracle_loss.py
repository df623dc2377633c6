"""Pins of the depth-weighted cross-entropy oracle (oracle/loss.py): the starting loss the
pages report for uniform predictions (ln of the draft vocabulary), torch's cross_entropy
per depth (mean over rows, ignored label -1), finite differences of the gradient, masked
rows and empty depths, and the K = 1 reduction to a plain mean."""
import numpy as np
import pytest
import torch

from oracle import loss as oloss


def _layout(counts):
    return np.concatenate([[0], np.cumsum(counts)])


def test_uniform_logits_give_ln_vocab():
    """NeMo PR 2376, validation: starting loss ~ ln(draft vocab = 8192) ~ 9.0."""
    off = _layout([50, 35, 25, 17])
    T, V = int(off[-1]), 8192
    labels = np.random.default_rng(0).integers(0, V, T)
    got = oloss.depth_weighted_ce_f64(np.zeros((T, V)), labels, off, want_grad=False)
    assert abs(got["loss"] - np.log(8192)) < 1e-12
    assert abs(np.log(8192) - 9.0) < 0.02


@pytest.mark.parametrize("decay", [0.8, 0.5])
def test_matches_torch_cross_entropy_per_depth(decay):
    rng = np.random.default_rng(1)
    off = _layout([40, 28, 0, 12])                       # depth 2 empty
    T, V = int(off[-1]), 37
    x = 3.0 * rng.standard_normal((T, V))
    labels = rng.integers(0, V, T)
    labels[rng.random(T) < 0.2] = -1                     # out-of-draft-vocab rows
    got = oloss.depth_weighted_ce_f64(x, labels, off, decay=decay, want_grad=False)
    num = den = 0.0
    for d in range(4):
        sl = slice(off[d], off[d + 1])
        if not (labels[sl] >= 0).any():
            assert np.isnan(got["depth_loss"][d])
            continue
        ld = torch.nn.functional.cross_entropy(torch.from_numpy(x[sl]), torch.from_numpy(labels[sl]),
                                               ignore_index=-1, reduction="mean").item()
        assert abs(got["depth_loss"][d] - ld) < 1e-12
        num += decay ** d * ld
        den += decay ** d
    assert abs(got["loss"] - num / den) < 1e-12


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(2)
    off = _layout([6, 4, 3])
    T, V = int(off[-1]), 9
    x = rng.standard_normal((T, V))
    labels = rng.integers(0, V, T)
    labels[3] = -1
    got = oloss.depth_weighted_ce_f64(x, labels, off)
    h = 1e-6
    num = np.zeros_like(x)
    for i in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        num[i] = (oloss.depth_weighted_ce_f64(xp, labels, off, want_grad=False)["loss"] -
                  oloss.depth_weighted_ce_f64(xm, labels, off, want_grad=False)["loss"]) / (2 * h)
    np.testing.assert_allclose(got["grad"], num, atol=1e-8)
    assert np.all(got["grad"][3] == 0.0)
    np.testing.assert_allclose(got["grad"].sum(axis=1), 0.0, atol=1e-12)  # softmax - onehot


def test_single_depth_is_the_plain_mean():
    rng = np.random.default_rng(3)
    x, labels = rng.standard_normal((30, 11)), rng.integers(0, 11, 30)
    got = oloss.depth_weighted_ce_f64(x, labels, np.array([0, 30]), want_grad=False)
    lse = np.log(np.exp(x).sum(axis=1))
    assert abs(got["loss"] - np.mean(lse - x[np.arange(30), labels])) < 1e-12


def test_gradient_of_chosen_rows_equals_the_full_gradient():
    rng = np.random.default_rng(4)
    off = _layout([20, 14, 0, 9])
    T, V = int(off[-1]), 13
    x, labels = rng.standard_normal((T, V)), rng.integers(0, V, T)
    labels[[2, 21]] = -1
    full = oloss.depth_weighted_ce_f64(x, labels, off)
    rows = np.array([0, 2, 19, 20, 21, 33, T - 1])
    sub = oloss.depth_weighted_ce_f64(x, labels, off, grad_rows=rows)
    np.testing.assert_allclose(sub["grad"], full["grad"][rows], atol=1e-15)
