"""GPU parity of the stacked draft layers (the 2nd and later: RMSNorm and QKV projection of
every row, then output projection, residual and SwiGLU MLP) against the float64 oracle.
Outputs of bf16 products are held to the bf16-projection bar of tests/helpers.py; small
cases in full, the full-size workloads on sampled rows, and a two-layer draft stack from
COD to the head against the chained oracles, held to the sum of its stages' bars."""
import numpy as np
import pytest

from oracle import cod as ocod
from oracle import fuse as ofuse
from oracle import layer as olayer
from token_drafting_amd import synth
from tests.helpers import assert_close_bf16_out, to_dev, to_host
from tests.test_gpu_layer import check_tokens, synth_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pe():
    import torch
    from token_drafting_amd import peagle
    assert torch.cuda.is_available()
    peagle.lib()
    return peagle


QKV_SMALL = [
    # (T, H, Hq, Hkv, D): H / 64 k-steps with and without a tail of the GEMM ring
    (700, 640, 4, 1, 256),      # Gemma-270M-shaped: 10 k-steps (tail of 1)
    (513, 192, 8, 2, 128),      # 3 k-steps (no tail), ragged M tile
    (65, 64, 4, 4, 64),         # one k-step
    (1, 128, 32, 8, 128),       # one row
    (300, 4096, 32, 8, 128),    # Llama-8B-shaped: 64 k-steps, N = 6144
]


@pytest.mark.parametrize("case", QKV_SMALL, ids=[f"T{c[0]}H{c[1]}h{c[2]}x{c[3]}D{c[4]}"
                                                 for c in QKV_SMALL])
def test_layer_qkv_small_full(pe, case):
    T, H, Hq, Hkv, D = case
    print(f"layer_qkv T={T} H={H} heads={Hq}/{Hkv} D={D}", flush=True)
    h = synth.residual_standin(T + H, T, H)
    w = synth.stacked_layer_weights(T + H, 2, H, Hq, Hkv, D, 64)
    q, k, v = pe.layer_qkv(to_dev(h), to_dev(w["w_norm"]), to_dev(w["w_qkv"]), Hq, Hkv, D)
    want = olayer.layer_qkv_f64(h, synth_bf16(w["w_norm"]), synth_bf16(w["w_qkv"]), Hq, Hkv, D)
    for name, got in (("q", q), ("k", k), ("v", v)):
        assert_close_bf16_out(synth_bf16(to_host(got)), want[name], name)


def _rows(T, seed, extra=60):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.integers(0, T, extra)]))


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_layer_qkv_full_size_sampled(pe, cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    H, Hq, Hkv, D = cfg["H"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    T = int(sum(ocod.retained_counts(cfg["n"], cfg["K"], cfg["r"], cfg["r_min"])))
    rows = _rows(T, cfg_id)
    print(f"layer_qkv config {cfg_id}: T={T} H={H}, {len(rows)} rows", flush=True)
    h = synth.residual_standin(cfg_id, T, H)
    w = synth.stacked_layer_weights(cfg_id, 2, H, Hq, Hkv, D, 64)
    q, k, v = pe.layer_qkv(to_dev(h), to_dev(w["w_norm"]), to_dev(w["w_qkv"]), Hq, Hkv, D)
    want = olayer.layer_qkv_f64(h[rows], synth_bf16(w["w_norm"]), synth_bf16(w["w_qkv"]), Hq, Hkv,
                                D)
    for name, got in (("q", q), ("k", k), ("v", v)):
        assert_close_bf16_out(synth_bf16(to_host(got[to_dev(rows)])), want[name],
                              f"{name} cfg{cfg_id}")


def _post(pe, T, H, Hq, D, I, seed, rows=None, inplace=False):
    QW = Hq * D
    h = synth.residual_standin(seed, T, H)
    att = synth.attention_out_standin(seed, T, QW)
    w = synth.stacked_layer_weights(seed, 3, H, Hq, 1, D, I)
    d = {k: to_dev(v) for k, v in w.items()}
    dh = to_dev(h)
    h2 = pe.layer_post(to_dev(att), dh, d["w_o"], d["w_post"], d["w_gate"], d["w_up"], d["w_down"],
                       h2=dh if inplace else None)
    rows = np.arange(T) if rows is None else rows
    wf = {k: synth_bf16(v) for k, v in w.items()}
    want = olayer.post_attention_f64(att[rows], h[rows], wf["w_o"], wf["w_post"], wf["w_gate"],
                                     wf["w_up"], wf["w_down"])
    return to_host(h2)[rows], want


POST_SMALL = [
    # (T, H, Hq, D, I)
    (700, 640, 4, 256, 2048),     # Gemma-270M-shaped
    (129, 128, 3, 64, 320),       # 2/3/5 k-steps
    (5, 64, 1, 64, 64),           # smallest sizes
]


@pytest.mark.parametrize("case", POST_SMALL, ids=[f"T{c[0]}H{c[1]}QW{c[2] * c[3]}I{c[4]}"
                                                  for c in POST_SMALL])
def test_layer_post_small_full(pe, case):
    T, H, Hq, D, I = case
    print(f"layer_post T={T} H={H} QW={Hq * D} I={I}", flush=True)
    got, want = _post(pe, T, H, Hq, D, I, seed=T + I)
    assert_close_bf16_out(got, want["h2"], "h2")


def test_layer_post_in_place(pe):
    """h2_out = h: the residual stream is updated in place with the same result."""
    got, want = _post(pe, 300, 256, 4, 64, 512, seed=8, inplace=True)
    assert_close_bf16_out(got, want["h2"], "h2 in place")


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_layer_post_full_size_sampled(pe, cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    H, Hq, D = cfg["H"], cfg["Hq"], cfg["D"]
    I = synth.LAYER_SHAPES[cfg_id]["I"]
    T = int(sum(ocod.retained_counts(cfg["n"], cfg["K"], cfg["r"], cfg["r_min"])))
    rows = _rows(T, cfg_id + 10)
    print(f"layer_post config {cfg_id}: T={T} H={H} I={I}, {len(rows)} rows", flush=True)
    got, want = _post(pe, T, H, Hq, D, I, seed=cfg_id, rows=rows)
    assert_close_bf16_out(got, want["h2"], f"h2 cfg{cfg_id}")


def test_two_layer_stack_chain(pe):
    """COD -> fused inputs -> first layer -> stacked layer 2 -> head on the GPU, each layer's
    attention by the draft attention kernel, against the stack oracle fed the fused
    oracle's outputs. One layer's chain is held to 5e-2 / 1.5e-2 (attention chain 3e-2 +
    bf16 projections 2e-2); two layers to twice that. Layer 2 is also checked alone, its
    oracle fed the GPU's layer-1 output, to the one-layer bar."""
    cfg = dict(synth.CONFIGS[1])
    n, K, Hq, Hkv, D, H = cfg["n"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["H"]
    QW, I, V, seed = Hq * D, 512, 1024, 29
    base = synth.base_inputs(cfg, seed)
    cu = base["cu_seqlens"]
    w1 = {**synth.layer1_weights(seed, H, Hq, Hkv, D), **synth.layer1_post_weights(seed, H, QW, I, V)}
    w2 = synth.stacked_layer_weights(seed, 2, H, Hq, Hkv, D, I)
    d1 = {k: to_dev(v) for k, v in w1.items()}
    d2 = {k: to_dev(v) for k, v in w2.items()}
    dcu = to_dev(cu)
    sel = pe.cod_select(n, K, cfg["r"], cfg["r_min"], seed, dcu)
    T = sel["T"]
    hid, emb = pe.fuse_inputs(n, K, T, sel["idx"], to_dev(base["aux"]), to_dev(base["fc_weight"]),
                              to_dev(base["mask_hidden"]), to_dev(base["tokens"]),
                              to_dev(base["embed"]), base["ptd_token_id"])
    cos, sin = pe.rope_table(D, cfg["theta"], pe.rope_max_pos(n, K))
    q, k, v = pe.layer1_qkv(n, K, T, hid, emb, d1["w_norm_emb"], d1["w_norm_hidden"], d1["w_qkv"],
                            Hq, Hkv, D)
    out, _, _ = pe.draft_attn(n, K, sel, dcu, q, k, v, cos, sin)
    h = pe.layer1_post(n, K, T, out, hid, d1["w_norm_hidden"], d1["w_o"], d1["w_post"],
                       d1["w_gate"], d1["w_up"], d1["w_down"])
    h1_gpu = to_host(h).copy()
    q, k, v = pe.layer_qkv(h, d2["w_norm"], d2["w_qkv"], Hq, Hkv, D)
    out, _, _ = pe.draft_attn(n, K, sel, dcu, q, k, v, cos, sin)
    h = pe.layer_post(out, h, d2["w_o"], d2["w_post"], d2["w_gate"], d2["w_up"], d2["w_down"],
                      h2=h)
    tok = pe.draft_head(h, d1["w_final"], d1["w_head"])
    osel = ocod.cod_select(n, K, cfg["r"], cfg["r_min"], seed, cu)
    f = ofuse.fuse_inputs(base["aux"], base["fc_weight"], base["mask_hidden"], base["tokens"],
                          base["embed"], base["ptd_token_id"], osel["idx"], osel["depth_off"])
    wf1 = {k2: synth_bf16(v2) for k2, v2 in w1.items()}
    wf2 = {k2: synth_bf16(v2) for k2, v2 in w2.items()}
    want = olayer.stack_forward_f64(f["hidden"], synth_bf16(f["embed_rows"]), wf1, [wf2],
                                    osel["idx"], osel["depth_off"], cu, cfg["theta"], Hq, Hkv, D)
    alone = olayer.layer_forward_f64(h1_gpu, wf2, osel["idx"], osel["depth_off"], cu,
                                     cfg["theta"], Hq, Hkv, D)
    assert_close_bf16_out(to_host(h), alone["h2"], "layer 2 fed the GPU's layer 1",
                          max_abs=5e-2, max_rel_l2=1.5e-2)
    assert_close_bf16_out(h1_gpu, want["h"][0], "chained layer 1", max_abs=5e-2, max_rel_l2=1.5e-2)
    assert_close_bf16_out(to_host(h), want["h"][1], "chained layer 2", max_abs=1e-1,
                          max_rel_l2=3e-2)
    check_tokens(to_host(tok), want["logits"], "chained tokens", tie=0.2)
