"""The checker of sampling verification (tests/helpers.check_sampled) on the CPU: it
accepts the oracle's own decisions and rejects a wrong accepted length, a token drawn from
the wrong place of the residual, and a token reported after a fully accepted draft."""
import numpy as np
import pytest

from oracle import verify as over
from token_drafting_amd import synth
from tests.helpers import check_sampled


@pytest.fixture(scope="module")
def case():
    inp = synth.sampled_verify_inputs(5, 24, 6, 400)
    want = over.speculative_accept(inp["draft_logits"], inp["target_logits"], inp["draft_tok"],
                                   inp["u"].astype(np.float64), inp["w"].astype(np.float64), 1.0)
    return inp, want


def test_oracle_outputs_pass_exactly(case):
    inp, want = case
    st = check_sampled(inp, 1.0, want["accept_len"], want["next_tok"])
    assert st["exact"] == st["drafts"] == 24
    assert st["ratio_miss"] == 0.0 and st["cdf_miss"] == 0.0
    assert 0 < st["rejected"] < 24


def test_wrong_accept_length_fails(case):
    inp, want = case
    K = inp["draft_tok"].shape[1]
    # a draft rejected at a depth whose ratio is clearly below u: claim it was accepted
    for i in range(24):
        L = int(want["accept_len"][i])
        if L < K and want["ratio"][i, L] < 0.9 * inp["u"][i, L]:
            got = want["accept_len"].copy()
            got[i] = L + 1
            with pytest.raises(AssertionError, match="accepted with u"):
                check_sampled(inp, 1.0, got, want["next_tok"])
            return
    pytest.fail("no clearly rejected draft in the fixture")


def test_token_from_wrong_place_fails(case):
    inp, want = case
    for i in range(24):
        L = int(want["accept_len"][i])
        if L == inp["draft_tok"].shape[1]:
            continue
        r = over.residual_f64(inp["draft_logits"][i, L], inp["target_logits"][i, L], 1.0)
        t = int(want["next_tok"][i])
        heavy = int(np.argmax(np.where(np.arange(r.size) == t, -1.0, r)))
        got = want["next_tok"].copy()
        got[i] = heavy
        with pytest.raises(AssertionError, match="spans"):
            check_sampled(inp, 1.0, want["accept_len"], got)
        return
    pytest.fail("no rejected draft in the fixture")


def test_token_after_full_accept_fails(case):
    inp, want = case
    K = inp["draft_tok"].shape[1]
    got_len = np.full(24, K, dtype=np.int32)
    u0 = dict(inp, u=np.zeros_like(inp["u"]))  # u = 0 accepts every depth
    with pytest.raises(AssertionError, match="all"):
        check_sampled(u0, 1.0, got_len, np.zeros(24, dtype=np.int32))
    st = check_sampled(u0, 1.0, got_len, np.full(24, -1, dtype=np.int32))
    assert st["exact"] == 24 and st["rejected"] == 0
