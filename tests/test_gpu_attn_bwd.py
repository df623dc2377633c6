"""GPU parity of the draft attention backward (peagle_draft_attn_bwd) against the float64
backward oracle on the same seeded inputs: dq, dk and dv compared in full on small
layouts (packed sequences, GQA, K from 1 to 16, D in {64, 128, 256}, ragged key blocks),
and at full size on sampled query rows and key rows plus a closed form over every key.

Bar. Gradients have no fixed scale (a key's dv sums over every row that sees it), so the
attention bar is applied relative to the tensor's largest magnitude: max |diff| <=
1e-2 * max(1, max |want|) and relative L2 <= 5e-3. A float64 emulation of the kernels'
roundings (q', k', dO, P and dS to bf16) reproduces the measured errors to within a few
percent: relative L2 about 3.5e-3, of which 2.6e-3 comes from q' and k' alone (the
forward's own MFMA operands)."""
import numpy as np
import pytest

from oracle import attention as oattn
from oracle import cod as ocod
from token_drafting_amd import synth
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _bwd_run(pe, n, K, seed, cu, Hq, Hkv, D, theta):
    sel = ocod.cod_select(n, K, 0.7, 0.2, seed, cu)
    T = int(sel["depth_off"][-1])
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    dout = synth.attn_grad_out(seed, T, Hq, D)
    dcu = to_dev(cu)
    dsel = pe.cod_select(n, K, 0.7, 0.2, seed, dcu)
    cos, sin = pe.rope_table(D, theta, pe.rope_max_pos(n, K))
    q, k, v = to_dev(qkv["q"]), to_dev(qkv["k"]), to_dev(qkv["v"])
    out, lse, _ = pe.draft_attn(n, K, dsel, dcu, q, k, v, cos, sin)
    dq, dk, dv, _ = pe.draft_attn_bwd(n, K, dsel, dcu, q, k, v, cos, sin, out, lse, to_dev(dout))
    want = oattn.draft_attention_backward(qkv["q"], qkv["k"], qkv["v"], sel["idx"],
                                          sel["depth_off"], cu, theta, dout)
    return dict(dq=to_host(dq), dk=to_host(dk), dv=to_host(dv)), want


def _err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    d = got - want
    return dict(max_abs=float(np.abs(d).max()),
                max_scaled=float((np.abs(d) / np.maximum(1.0, np.abs(want))).max()),
                rel_l2=float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-30)),
                scale=float(np.abs(want).max()))


BWD_SMALL = [
    # (n, K, seed, lengths, Hq, Hkv, D, theta)
    (256, 4, 1, None, 4, 1, 64, 1e4),                 # the tiny workload
    (300, 4, 2, [90, 150, 60], 8, 2, 128, 5e5),        # packed, GQA 4, ragged key blocks
    (200, 3, 3, None, 4, 1, 256, 1e4),
    (130, 1, 4, None, 4, 1, 64, 1e4),                  # K = 1: no diagonal keys
    (100, 8, 5, [33, 67], 8, 1, 128, 1e4),             # K = 8, G = 8
    (64, 4, 6, None, 2, 2, 64, 1e4),                   # G = 1
    (1, 4, 7, None, 4, 1, 64, 1e4),                    # one token
    (600, 4, 10, [1] * 5 + [595], 16, 1, 64, 1e4),     # one-token sequences, G = 16
    (520, 4, 11, [260, 260], 32, 8, 128, 5e5),         # Llama-8B heads
    (700, 4, 12, None, 4, 1, 256, 1e4),                # several key blocks at D = 256
    (300, 16, 13, [120, 180], 4, 1, 256, 1e4),         # K = 16
]


@pytest.mark.parametrize("case", BWD_SMALL, ids=[f"n{c[0]}K{c[1]}D{c[6]}H{c[4]}x{c[5]}" for c in BWD_SMALL])
def test_attention_bwd_small_full(pe, case):
    n, K, seed, lens, Hq, Hkv, D, theta = case
    cu = _cu(lens) if lens else np.array([0, n], dtype=np.int32)
    print(f"attention bwd n={n} K={K} Hq={Hq} Hkv={Hkv} D={D} S={len(cu) - 1}", flush=True)
    got, want = _bwd_run(pe, n, K, seed, cu, Hq, Hkv, D, theta)
    for name in ("dq", "dk", "dv"):
        _check_grad(got[name], want[name], name)


def _check_grad(got, want, what):
    e = _err(got, want)
    print(what, {k2: f"{v2:.3e}" for k2, v2 in e.items()}, flush=True)
    assert np.isfinite(got).all(), what
    assert e["max_abs"] <= 1e-2 * max(1.0, e["scale"]), (what, e)
    assert e["rel_l2"] <= 5e-3, (what, e)


def test_attention_bwd_mid_size_full(pe):
    """The 4096-token Gemma-shaped workload (T = 10375, one kv head, D = 256) in full: the
    early depth-0 keys are seen by thousands of rows, so their dk and dv sum many query
    tiles. Every element of dq, dk and dv against the oracle, on workspace and outputs
    pre-filled with non-zero bytes (nothing may read what the call did not write)."""
    import torch
    cfg_id = 2
    cfg = synth.CONFIGS[cfg_id]
    n, K, Hq, Hkv, D, theta = cfg["n"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["theta"]
    cu = synth.cu_seqlens_for(cfg, cfg_id)
    sel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], cfg_id, cu)
    T = int(sel["depth_off"][-1])
    print(f"attention bwd config {cfg_id} in full: n={n} T={T}", flush=True)
    qkv = synth.qkv_inputs(cfg_id, T, Hq, Hkv, D)
    dout = synth.attn_grad_out(cfg_id, T, Hq, D)
    dcu = to_dev(cu)
    dsel = pe.cod_select(n, K, cfg["r"], cfg["r_min"], cfg_id, dcu)
    cos, sin = pe.rope_table(D, theta, pe.rope_max_pos(n, K))
    q, k, v = to_dev(qkv["q"]), to_dev(qkv["k"]), to_dev(qkv["v"])
    out, lse, _ = pe.draft_attn(n, K, dsel, dcu, q, k, v, cos, sin)
    wsb = int(pe.lib().peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D))
    ws = torch.full((wsb,), 0x41, dtype=torch.uint8, device="cuda")
    dq = torch.full((T, Hq, D), 3.0, dtype=torch.float32, device="cuda")
    dk = torch.full((T, Hkv, D), 3.0, dtype=torch.float32, device="cuda")
    dv = torch.full((T, Hkv, D), 3.0, dtype=torch.float32, device="cuda")
    pe.draft_attn_bwd(n, K, dsel, dcu, q, k, v, cos, sin, out, lse, to_dev(dout), dq=dq, dk=dk,
                      dv=dv, workspace=ws)
    torch.cuda.synchronize()
    want = oattn.draft_attention_backward(qkv["q"], qkv["k"], qkv["v"], sel["idx"],
                                          sel["depth_off"], cu, theta, dout)
    got = dict(dq=to_host(dq), dk=to_host(dk), dv=to_host(dv))
    for name in ("dq", "dk", "dv"):
        _check_grad(got[name], want[name], f"{name} cfg{cfg_id}")
    # the keys with the most query tiles behind them, element by element on their own
    for name in ("dk", "dv"):
        _check_grad(got[name][:64], want[name][:64], f"{name} cfg{cfg_id} first 64 keys")


@pytest.mark.parametrize("n,K,Hq,Hkv,D,lens", [(4096, 4, 4, 1, 256, None),
                                               (3000, 4, 32, 8, 128, [1000, 1200, 800])])
def test_attention_bwd_bit_reproducible(pe, n, K, Hq, Hkv, D, lens):
    """Two calls on the same inputs give the same bits: dK and dV sum their query segments
    in a fixed order (no atomics), dq and the depth >= 1 rows have one writer each."""
    import torch
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32) if lens else \
        np.array([0, n], dtype=np.int32)
    seed = 51
    dcu = to_dev(cu)
    dsel = pe.cod_select(n, K, 0.7, 0.2, seed, dcu)
    T = dsel["T"]
    print(f"attention bwd repeat n={n} T={T} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    dout = to_dev(synth.attn_grad_out(seed, T, Hq, D))
    cos, sin = pe.rope_table(D, 1e4, pe.rope_max_pos(n, K))
    q, k, v = to_dev(qkv["q"]), to_dev(qkv["k"]), to_dev(qkv["v"])
    out, lse, _ = pe.draft_attn(n, K, dsel, dcu, q, k, v, cos, sin)
    first = pe.draft_attn_bwd(n, K, dsel, dcu, q, k, v, cos, sin, out, lse, dout)[:3]
    ws = torch.full((int(pe.lib().peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D)),),
                    0x7F, dtype=torch.uint8, device="cuda")
    second = pe.draft_attn_bwd(n, K, dsel, dcu, q, k, v, cos, sin, out, lse, dout,
                               workspace=ws)[:3]
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), first, second):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_attention_bwd_full_size_sampled(pe, cfg_id):
    """The full-size workloads in the launch the bench times: dq of sampled query rows;
    dk and dv of the last depth-0 keys of the sequence and of sampled depth >= 1 rows
    (each seen by few rows, so the oracle recomputes them alone); and over every key,
    sum_j dv_j = sum over rows and q heads of dO (softmax rows sum to one)."""
    import torch
    cfg = synth.CONFIGS[cfg_id]
    n, K, Hq, Hkv, D, theta = cfg["n"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["theta"]
    cu = synth.cu_seqlens_for(cfg, cfg_id)
    sel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], cfg_id, cu)
    T = int(sel["depth_off"][-1])
    print(f"attention bwd config {cfg_id}: n={n} T={T}", flush=True)
    qkv = synth.qkv_inputs(cfg_id, T, Hq, Hkv, D)
    dout = synth.attn_grad_out(cfg_id, T, Hq, D)
    dcu = to_dev(cu)
    dsel = pe.cod_select(n, K, cfg["r"], cfg["r_min"], cfg_id, dcu)
    cos, sin = pe.rope_table(D, theta, pe.rope_max_pos(n, K))
    q, k, v = to_dev(qkv["q"]), to_dev(qkv["k"]), to_dev(qkv["v"])
    out, lse, ws = pe.draft_attn(n, K, dsel, dcu, q, k, v, cos, sin)
    del ws
    dq, dk, dv, _ = pe.draft_attn_bwd(n, K, dsel, dcu, q, k, v, cos, sin, out, lse, to_dev(dout))
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg_id)
    d0 = sel["depth_off"]
    q_rows = np.unique(np.concatenate([[0, n - 1, int(d0[1]), T - 1], rng.integers(0, T, 12)]))
    k_rows = np.unique(np.concatenate([np.arange(n - 6, n), [int(d0[1]), T - 1],
                                       rng.integers(int(d0[1]), T, 6)]))
    want = oattn.draft_attention_backward_rows_f64(
        synth_f64(qkv["q"]), synth_f64(qkv["k"]), synth_f64(qkv["v"]), sel["idx"], d0, cu,
        theta, dout, q_rows, k_rows)
    _check_grad(to_host(dq[to_dev(q_rows)]), want["dq"], f"dq cfg{cfg_id}")
    _check_grad(to_host(dk[to_dev(k_rows)]), want["dk"], f"dk cfg{cfg_id}")
    _check_grad(to_host(dv[to_dev(k_rows)]), want["dv"], f"dv cfg{cfg_id}")
    G = Hq // Hkv
    dv_sum = to_host(dv.double().sum(dim=0))                      # [Hkv, D]
    do_sum = dout.astype(np.float64).reshape(T, Hkv, G, D).sum(axis=(0, 2))
    e = _err(dv_sum, do_sum)
    print("sum dv", e, flush=True)
    assert e["rel_l2"] <= 5e-3, e
    assert np.isfinite(to_host(dq)).all() and np.isfinite(to_host(dk)).all()


def synth_f64(bits):
    from oracle.bf16 import to_f64
    return to_f64(bits)
