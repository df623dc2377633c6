"""GPU parity of the depth-weighted cross-entropy (peagle_depth_ce) against the float64
oracle on the same seeded logits and labels: the loss and the per-depth losses within
relative 1e-5 (fp32 row statistics, fp64 sums), the bf16 gradient within 4e-3 of the
tensor's largest magnitude (bf16 keeps 8 significant bits: rounding moves a value by up to
2^-9 of itself) and relative L2 5e-3; the loss bit for bit on a second run."""
import numpy as np
import pytest

from oracle import cod as ocod
from oracle import loss as oloss
from token_drafting_amd import synth
from tests.helpers import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


def _bf16_to_f64(bits):
    from oracle.bf16 import to_f64
    return to_f64(bits)


def _check(got_loss, got_depth, want, K):
    assert abs(float(got_loss) - want["loss"]) <= 1e-5 * abs(want["loss"]), (got_loss, want["loss"])
    for d in range(K):
        if np.isnan(want["depth_loss"][d]):
            assert np.isnan(got_depth[d]), d
        else:
            assert abs(got_depth[d] - want["depth_loss"][d]) <= 1e-5 * abs(want["depth_loss"][d]), d


CE_SMALL = [
    # (n, K, V, decay, mask a whole depth)
    (256, 4, 8192, 0.8, None),      # the tiny workload's rows, draft vocabulary 8192
    (256, 4, 1001, 0.8, None),      # V odd: element loads
    (300, 8, 4096, 0.5, 2),         # K = 8, depth 2 fully masked
    (130, 1, 32000, 0.8, None),     # K = 1: the plain mean
]


@pytest.mark.parametrize("case", CE_SMALL, ids=[f"n{c[0]}K{c[1]}V{c[2]}" for c in CE_SMALL])
def test_depth_ce_small_full(pe, case):
    n, K, V, decay, masked = case
    sel = ocod.cod_select(n, K, 0.7, 0.2, 1, np.array([0, n]))
    off = sel["depth_off"]
    T = int(off[-1])
    print(f"depth_ce T={T} K={K} V={V}", flush=True)
    inp = synth.ce_inputs(n + V, T, V)
    if masked is not None:
        inp["labels"][off[masked]:off[masked + 1]] = -1
    loss, dloss, grad = pe.depth_ce(to_dev(off.astype(np.int32)), to_dev(inp["logits"]),
                                    to_dev(inp["labels"]), decay=decay)
    want = oloss.depth_weighted_ce_f64(inp["logits"], inp["labels"], off, decay=decay)
    _check(to_host(loss)[0], to_host(dloss), want, K)
    g = _bf16_to_f64(to_host(grad))
    scale = float(np.abs(want["grad"]).max())
    assert_close(g, want["grad"], "dlogits", max_abs=4e-3 * scale)
    masked_rows = inp["labels"] < 0
    assert np.all(g[masked_rows] == 0.0)


def test_depth_ce_full_size(pe):
    """The 83001 draft rows of the 32K-token K = 4 workload over the 8192-id draft
    vocabulary, in the launch the bench times: the loss over every row, the gradient of
    sampled rows (both ends of every depth and a seeded spread), and the same loss bit for
    bit on a second call."""
    import torch
    cfg = synth.CONFIGS[4]
    n, K = cfg["n"], cfg["K"]
    sel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], 4, np.array([0, n]))
    off = sel["depth_off"]
    T, V = int(off[-1]), synth.DRAFT_VOCAB
    print(f"depth_ce full size T={T} V={V}", flush=True)
    inp = synth.ce_inputs(4, T, V)
    d_off, d_logits, d_labels = to_dev(off.astype(np.int32)), to_dev(inp["logits"]), to_dev(inp["labels"])
    loss, dloss, grad = pe.depth_ce(d_off, d_logits, d_labels)
    loss2, _, _ = pe.depth_ce(d_off, d_logits, d_labels, want_grad=False)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([off[:-1], off[1:] - 1, rng.integers(0, T, 48)]))
    want = oloss.depth_weighted_ce_f64(inp["logits"], inp["labels"], off, grad_rows=rows)
    _check(to_host(loss)[0], to_host(dloss), want, K)
    g = _bf16_to_f64(to_host(grad[to_dev(rows)]))
    assert_close(g, want["grad"], "dlogits rows", max_abs=4e-3 * float(np.abs(want["grad"]).max()))
