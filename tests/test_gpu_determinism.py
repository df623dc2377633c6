"""Bitwise results under a different workgroup schedule.

No output of the draft attention (forward or backward) or of COD may depend on the order in
which workgroups run or the CUs they land on: every output element has one writer, and
partial results (the key-range split's segments, the backward's dK/dV segment slabs) are
merged in a fixed order, never by atomics. These tests repeat each call while a second
stream keeps a chain of fp32 GEMMs running beside it (default priority, like every stream
here), so the call's workgroups are placed and retired in a different order, and compare
the outputs bit for bit with an unloaded run."""
import numpy as np
import pytest

from token_drafting_amd import synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


def _load(side, a, reps=6):
    """Enqueue reps fp32 GEMMs (4096^3, about a millisecond each) on the side stream."""
    import torch
    with torch.cuda.stream(side):
        for _ in range(reps):
            torch.matmul(a, a)


@pytest.mark.parametrize("n,K,Hq,Hkv,D,lens", [
    (2000, 4, 4, 1, 256, None),            # key-range split and merge
    (3300, 4, 16, 16, 64, None),           # unsplit main kernel
    (3000, 8, 32, 8, 128, [1200, 1800]),   # packed sequences, GQA
])
def test_attention_bitwise_under_concurrent_load(pe, n, K, Hq, Hkv, D, lens):
    import torch
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32) if lens else \
        np.array([0, n], dtype=np.int32)
    seed = 61
    dcu = to_dev(cu)
    sel = pe.cod_select(n, K, 0.7, 0.2, seed, dcu)
    T = sel["T"]
    print(f"attention under load n={n} K={K} T={T} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    q, k, v = to_dev(qkv["q"]), to_dev(qkv["k"]), to_dev(qkv["v"])
    dout = to_dev(synth.attn_grad_out(seed, T, Hq, D))
    cos, sin = pe.rope_table(D, 1e4, pe.rope_max_pos(n, K))
    out0, lse0, _ = pe.draft_attn(n, K, sel, dcu, q, k, v, cos, sin)
    grads0 = pe.draft_attn_bwd(n, K, sel, dcu, q, k, v, cos, sin, out0, lse0, dout)[:3]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    for trial in range(3):
        _load(side, a)
        out1, lse1, _ = pe.draft_attn(n, K, sel, dcu, q, k, v, cos, sin)
        grads1 = pe.draft_attn_bwd(n, K, sel, dcu, q, k, v, cos, sin, out1, lse1, dout)[:3]
        torch.cuda.synchronize()
        assert torch.equal(out0, out1) and torch.equal(lse0, lse1), f"forward, trial {trial}"
        for name, x, y in zip(("dq", "dk", "dv"), grads0, grads1):
            assert torch.equal(x, y), f"{name}, trial {trial}"


def test_cod_bitwise_under_concurrent_load(pe):
    import torch
    n, K = 50000, 8
    cu = to_dev(np.array([0, 20000, 20001, 50000], dtype=np.int32))
    ref = pe.cod_select(n, K, 0.7, 0.2, 77, cu)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    for trial in range(3):
        _load(side, a, reps=2)
        got = pe.cod_select(n, K, 0.7, 0.2, 77, cu)
        torch.cuda.synchronize()
        for key in ("idx", "depth_off", "cu_seqlens_d", "row_of"):
            assert torch.equal(ref[key], got[key]), f"{key}, trial {trial}"
