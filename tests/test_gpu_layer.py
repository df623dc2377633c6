"""GPU parity of the first draft layer's attention inputs (RMSNorm halves, [emb, hidden]
concat, QKV projection on rows 0..n, broadcast of row n) against the float64 oracle,
which projects every row. q, k and v are bf16 outputs of bf16 operands: within 2e-2
absolute below magnitude 1 and 2e-2 relative above it, and relative L2 <= 5e-3 (the bar
and its derivation are in tests/helpers.py).
Small cases in full; the full-size workloads on sampled rows; and one chain of the fused
stage, this stage and the draft attention against the chained oracles, held to the sum
of the stages' bars.
"""
import numpy as np
import pytest

from oracle import attention as oattn
from oracle import cod as ocod
from oracle import fuse as ofuse
from oracle import layer as olayer
from token_drafting_amd import synth
from tests.helpers import assert_close, assert_close_bf16_out, sample_rows, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


def _run(pe, n, K, T, inp, w, Hq, Hkv, D):
    q, k, v = pe.layer1_qkv(n, K, T, to_dev(inp["hidden"]), to_dev(inp["embed"]),
                            to_dev(w["w_norm_emb"]), to_dev(w["w_norm_hidden"]),
                            to_dev(w["w_qkv"]), Hq, Hkv, D)
    return to_host(q), to_host(k), to_host(v)


LAYER_SMALL = [
    # (n, K, H, Hq, Hkv, D): 2H / 64 k-steps with and without a tail of the GEMM ring
    (300, 4, 640, 4, 1, 256),      # Gemma-270M-shaped: 20 k-steps (tail of 2)
    (257, 4, 96, 2, 2, 64),        # 3 k-steps (no tail), ragged M tile
    (513, 8, 256, 8, 2, 128),      # 8 k-steps (tail of 2), K = 8
    (130, 1, 64, 4, 1, 64),        # K = 1: no depth >= 1 rows, no broadcast
    (77, 4, 1024, 32, 8, 128),     # Llama-shaped heads, N = 6144
    (1, 4, 32, 4, 4, 8),           # one anchor, smallest sizes
]


@pytest.mark.parametrize("case", LAYER_SMALL, ids=[f"n{c[0]}K{c[1]}H{c[2]}h{c[3]}x{c[4]}D{c[5]}"
                                                   for c in LAYER_SMALL])
def test_layer1_small_full(pe, case):
    n, K, H, Hq, Hkv, D = case
    T = int(sum(ocod.retained_counts(n, K, 0.7, 0.2)))
    print(f"layer1 n={n} K={K} T={T} H={H} heads={Hq}/{Hkv} D={D}", flush=True)
    inp = synth.layer1_inputs(n + H, n, T, H)
    w = synth.layer1_weights(n + H, H, Hq, Hkv, D)
    q, k, v = _run(pe, n, K, T, inp, w, Hq, Hkv, D)
    want = olayer.layer1_qkv(inp["hidden"], inp["embed"], w["w_norm_emb"], w["w_norm_hidden"],
                             w["w_qkv"], Hq, Hkv, D)
    for name, got in (("q", q), ("k", k), ("v", v)):
        assert_close_bf16_out(synth_bf16(got), want[name], name)


def synth_bf16(bits):
    from oracle.bf16 import to_f64
    return to_f64(bits)


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_layer1_full_size_sampled(pe, cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    n, K, H, Hq, Hkv, D = cfg["n"], cfg["K"], cfg["H"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    cu = synth.cu_seqlens_for(cfg, cfg_id)
    sel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], cfg_id, cu)
    T = int(sel["depth_off"][-1])
    rows = sample_rows(sel["depth_off"], cu, sel["idx"], count=64, seed=cfg_id)
    rows = np.unique(np.concatenate([rows, [0, n - 1, n, T - 1]]))
    print(f"layer1 config {cfg_id}: T={T}, {len(rows)} sampled rows", flush=True)
    inp = synth.layer1_inputs(cfg_id, n, T, H)
    w = synth.layer1_weights(cfg_id, H, Hq, Hkv, D)
    q, k, v = _run(pe, n, K, T, inp, w, Hq, Hkv, D)
    want = olayer.layer1_qkv(inp["hidden"][rows], inp["embed"][rows], w["w_norm_emb"],
                             w["w_norm_hidden"], w["w_qkv"], Hq, Hkv, D)
    for name, got in (("q", q), ("k", k), ("v", v)):
        assert_close_bf16_out(synth_bf16(got[rows]), want[name], f"{name} cfg{cfg_id}")


def test_fuse_layer1_attention_chain(pe):
    """COD -> fused inputs -> first-layer q/k/v -> draft attention on the GPU, against the
    same chain of oracles (each stage fed the previous oracle stage's float64 output)."""
    cfg = dict(synth.CONFIGS[1])
    n, K, Hq, Hkv, D, H = cfg["n"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["H"]
    seed = 21
    base = synth.base_inputs(cfg, seed)
    cu = base["cu_seqlens"]
    w = synth.layer1_weights(seed, H, Hq, Hkv, D)
    # GPU chain
    dcu = to_dev(cu)
    sel = pe.cod_select(n, K, cfg["r"], cfg["r_min"], seed, dcu)
    T = sel["T"]
    hid, emb = pe.fuse_inputs(n, K, T, sel["idx"], to_dev(base["aux"]), to_dev(base["fc_weight"]),
                              to_dev(base["mask_hidden"]), to_dev(base["tokens"]),
                              to_dev(base["embed"]), base["ptd_token_id"])
    q, k, v = pe.layer1_qkv(n, K, T, hid, emb, to_dev(w["w_norm_emb"]),
                            to_dev(w["w_norm_hidden"]), to_dev(w["w_qkv"]), Hq, Hkv, D)
    cos, sin = pe.rope_table(D, cfg["theta"], pe.rope_max_pos(n, K))
    out, lse, _ = pe.draft_attn(n, K, sel, dcu, q, k, v, cos, sin)
    # oracle chain; the attention's inputs are bf16 at the boundary, so the oracle's q, k, v
    # are rounded to bf16 (nearest even) before the attention oracle, as the GPU stores them
    osel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], seed, cu)
    f = ofuse.fuse_inputs(base["aux"], base["fc_weight"], base["mask_hidden"], base["tokens"],
                          base["embed"], base["ptd_token_id"], osel["idx"], osel["depth_off"])
    lw = olayer.layer1_qkv_f64(f["hidden"], synth_bf16(f["embed_rows"]),
                               synth_bf16(w["w_norm_emb"]), synth_bf16(w["w_norm_hidden"]),
                               synth_bf16(w["w_qkv"]), Hq, Hkv, D)
    bits = {t: synth.f32_to_bf16_bits(lw[t].astype(np.float32)) for t in ("q", "k", "v")}
    want = oattn.draft_attention(bits["q"], bits["k"], bits["v"], osel["idx"], osel["depth_off"],
                                 cu, cfg["theta"])
    # The chain compounds two stages, so its bar is the sum of theirs (bf16 projection 2e-2,
    # attention 1e-2; relative L2 5e-3 each). In float64 emulation the layer's bf16
    # rounding alone, carried through an exact attention, moves this output by 1.56e-2 max
    # and 4.0e-3 relative L2.
    assert_close(to_host(out), want["out"], "chained attention out", max_abs=3e-2,
                 max_rel_l2=1e-2)
