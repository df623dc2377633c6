"""Seeded synthetic inputs for the P-EAGLE draft forward.

This module only draws random numbers and packs them into the buffers the draft
forward consumes. It holds none of the method's arithmetic: how many rows survive
COD sampling, which rows they are, the projection, RoPE, attention and the
acceptance rule all live elsewhere. Callers pass the row count ``T`` in.

Every tensor has its own generator, ``numpy.random.default_rng([seed, tag])``,
so any tensor can be drawn without drawing the others first. Floating tensors
are drawn as float32 normals and rounded to bfloat16 with round-to-nearest-even;
they are returned as raw bf16 bit patterns (``uint16``), exactly the bytes that
cross the C boundary.

The workload shapes follow the pages: an EAGLE-3 drafter fed the concatenation
of three target hidden states (speculators P-EAGLE guide, "Architecture"), a
learnable ``mask_hidden`` of width 3 x target hidden (NeMo Automodel PR 2376,
description), packed conversations delimited by ``cu_seqlens`` (snxtyle/P_Eagle
README, data-preparation list), and K parallel depths with COD ratios 0.7 / 0.2
(speculators guide, "Key Parameters").
"""
from __future__ import annotations

import numpy as np

# Tensor tags: each input draws from default_rng([seed, TAG]).
TAG_LENGTHS, TAG_AUX, TAG_W, TAG_MASK, TAG_EMBED, TAG_TOKENS = 1, 2, 3, 4, 5, 6
TAG_Q, TAG_K, TAG_V, TAG_LOGITS = 7, 8, 9, 10
TAG_CACHE_K, TAG_CACHE_V, TAG_NEW_Q, TAG_NEW_K, TAG_NEW_V = 11, 12, 13, 14, 15
TAG_NORM_EMB, TAG_NORM_HID, TAG_WQKV, TAG_L1_HID, TAG_L1_EMB = 16, 17, 18, 19, 20
TAG_WO, TAG_NORM_POST, TAG_WGATE, TAG_WUP, TAG_WDOWN, TAG_NORM_FINAL, TAG_WHEAD, TAG_ATTN = (
    21, 22, 23, 24, 25, 26, 27, 28)
TAG_D2T, TAG_FC_NORM = 29, 30
TAG_SPEC_LOGITS, TAG_SPEC_TOK, TAG_SPEC_U, TAG_SPEC_W = 31, 32, 33, 34
# stacked layer L >= 2 draws from tags TAG_STACK + 8 (L - 2) + 0 .. 7
TAG_STACK = 40
TAG_DOUT = 35
TAG_CE_LOGITS, TAG_CE_LABELS = 36, 37
TAG_SPEC_BONUS = 38   # (40 and up belong to the stacked layers)

# Rest of the draft layer: MLP intermediate size of the Gemma-3-270M and Llama-3-8B shaped
# layers, and the draft vocabulary (8192 in the NeMo PR's validation run).
LAYER_SHAPES = {2: dict(I=2048), 4: dict(I=2048), 3: dict(I=14336), 5: dict(I=14336)}
DRAFT_VOCAB = 8192

VOCAB_IN = 32000          # input-embedding vocabulary of the synthetic drafter
PLANT_VALUE_BITS = 0x4180  # bf16 bit pattern of 16.0 (exact), the planted maximum

# The five synthetic workloads. Shapes only; no derived quantity lives here.
CONFIGS = {
    1: dict(workload="tiny-256", n=256, K=4, r=0.7, r_min=0.2, H=256, aux_dim=3 * 512,
            Hq=4, Hkv=1, D=64, theta=1.0e4, num_seqs=1),
    2: dict(workload="gemma270m-draft-4k", n=4096, K=4, r=0.7, r_min=0.2, H=640,
            aux_dim=3 * 2560, Hq=4, Hkv=1, D=256, theta=1.0e4, num_seqs=1),
    3: dict(workload="packed8-llama8b-draft-4k", n=4096, K=4, r=0.7, r_min=0.2, H=4096,
            aux_dim=3 * 4096, Hq=32, Hkv=8, D=128, theta=5.0e5, num_seqs=8,
            len_lo=256, len_hi=1024),
    4: dict(workload="gemma270m-draft-32k-K4", n=32768, K=4, r=0.7, r_min=0.2, H=640,
            aux_dim=3 * 2560, Hq=4, Hkv=1, D=256, theta=1.0e4, num_seqs=1),
    5: dict(workload="llama8b-draft-16k-K8", n=16384, K=8, r=0.7, r_min=0.2, H=4096,
            aux_dim=3 * 4096, Hq=32, Hkv=8, D=128, theta=5.0e5, num_seqs=1,
            verify=dict(drafts=4096, K=8, V=32000, p_plant=0.7)),
}

# Inference (decode-shaped) workloads: B requests, each with a KV cache of a context length
# drawn uniform in [ctx_lo, ctx_hi], and K new rows (the anchor and K-1 mask rows). Heads
# and RoPE base follow the Gemma-270M and Llama-8B shaped draft layers above.
DECODE_CONFIGS = {
    "gemma270m": dict(workload="decode-gemma270m-B64-ctx1k-32k-K4", B=64, ctx_lo=1024,
                      ctx_hi=32768, K=4, Hq=4, Hkv=1, D=256, theta=1.0e4),
    "llama8b": dict(workload="decode-llama8b-B64-ctx1k-32k-K8", B=64, ctx_lo=1024,
                    ctx_hi=32768, K=8, Hq=32, Hkv=8, D=128, theta=5.0e5),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the uint16 bits.

    Inputs are finite normals, so the NaN/overflow corner of the rounding is not
    reached.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag)])


def normal_bf16(seed: int, tag: int, shape, std: float = 1.0,
                chunk_rows: int = 1 << 20) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples of the given shape, drawn in row chunks."""
    shape = tuple(int(s) for s in shape)
    rng = _rng(seed, tag)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.uint16)
    step = max(1, chunk_rows * (shape[-1] if shape else 1))
    for lo in range(0, total, step):
        hi = min(total, lo + step)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def packed_lengths(seed: int, n: int, num_seqs: int, lo: int, hi: int) -> np.ndarray:
    """Lengths of ``num_seqs`` conversations packed with no padding into n tokens.

    Draw num_seqs-1 integers uniform in [lo, hi]; the last length is what is left
    of n. Redraw from the same stream until the last one also lies in [lo, hi].
    This is uniform over the packings with every length in range.
    """
    rng = _rng(seed, TAG_LENGTHS)
    for _ in range(100000):
        first = rng.integers(lo, hi + 1, size=num_seqs - 1)
        last = n - int(first.sum())
        if lo <= last <= hi:
            return np.concatenate([first, [last]]).astype(np.int64)
    raise RuntimeError("no valid packing found")


def cu_seqlens_for(cfg: dict, seed: int) -> np.ndarray:
    """int32 [S+1] sequence starts of the packed buffer (0 ... n)."""
    n, S = cfg["n"], cfg.get("num_seqs", 1)
    if S == 1:
        return np.array([0, n], dtype=np.int32)
    lens = packed_lengths(seed, n, S, cfg["len_lo"], cfg["len_hi"])
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def base_inputs(cfg: dict, seed: int) -> dict:
    """Everything the fused input stage needs: cu_seqlens, aux, fc weight,
    mask_hidden, embedding table, tokens and the reserved ptd token id."""
    n, H, A = cfg["n"], cfg["H"], cfg["aux_dim"]
    vocab = cfg.get("vocab_in", VOCAB_IN)
    out = dict(
        cu_seqlens=cu_seqlens_for(cfg, seed),
        aux=normal_bf16(seed, TAG_AUX, (n, A)),
        fc_weight=normal_bf16(seed, TAG_W, (H, A), std=0.02),
        mask_hidden=normal_bf16(seed, TAG_MASK, (A,)),
        embed=normal_bf16(seed, TAG_EMBED, (vocab, H)),
        # tokens never take the last id, which is reserved as the ptd token
        tokens=_rng(seed, TAG_TOKENS).integers(0, vocab - 1, size=n).astype(np.int32),
        ptd_token_id=vocab - 1,
        vocab=vocab,
    )
    return out


def qkv_inputs(seed: int, T: int, Hq: int, Hkv: int, D: int) -> dict:
    """Pre-RoPE q [T,Hq,D], k and v [T,Hkv,D], bf16 bits of N(0,1)."""
    return dict(q=normal_bf16(seed, TAG_Q, (T, Hq, D)),
                k=normal_bf16(seed, TAG_K, (T, Hkv, D)),
                v=normal_bf16(seed, TAG_V, (T, Hkv, D)))


def verify_logits(seed: int, drafts: int, K: int, V: int, p_plant: float,
                  chunk: int = 256) -> dict:
    """Draft and target logits [drafts, K, V] as bf16 bits of N(0,1) noise, with
    planted shared maxima.

    For each draft, depth d gets a plant with probability p_plant, but only while
    every earlier depth was planted too. A plant writes 16.0 (exact in bf16, far
    above any N(0,1) sample of this size) at one uniform position t* in both the
    draft and the target row. ``planted`` holds how many leading depths were
    planted per draft.
    """
    rng = _rng(seed, TAG_LOGITS)
    plant_rng = _rng(seed, TAG_LOGITS + 100)
    draft = np.empty((drafts, K, V), dtype=np.uint16)
    target = np.empty((drafts, K, V), dtype=np.uint16)
    for lo in range(0, drafts, chunk):
        hi = min(drafts, lo + chunk)
        m = (hi - lo) * K * V
        draft[lo:hi] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32)).reshape(hi - lo, K, V)
        target[lo:hi] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32)).reshape(hi - lo, K, V)
    coins = plant_rng.random((drafts, K)) < p_plant
    where = plant_rng.integers(0, V, size=(drafts, K))
    planted = np.zeros(drafts, dtype=np.int32)
    for i in range(drafts):
        for d in range(K):
            if not coins[i, d]:
                break
            draft[i, d, where[i, d]] = PLANT_VALUE_BITS
            target[i, d, where[i, d]] = PLANT_VALUE_BITS
            planted[i] += 1
    return dict(draft_logits=draft, target_logits=target, planted=planted)


def verify_logits_device(seed: int, drafts: int, K: int, V: int, p_plant: float,
                         device="cuda") -> dict:
    """The recipe of verify_logits drawn on the device with torch's seeded generator
    (gigabytes of logits at full size): N(0, 1) bf16 logits, and along a geometric prefix
    of depths (each planted with probability p_plant while all earlier ones were) 16.0 at
    one uniform position of both rows. Logits as int16 bf16 bit patterns."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + TAG_LOGITS)
    draft = torch.empty((drafts, K, V), dtype=torch.int16, device=device)
    target = torch.empty_like(draft)
    rows = max(1, (1 << 25) // (K * V))
    for lo in range(0, drafts, rows):
        hi = min(drafts, lo + rows)
        draft[lo:hi] = torch.randn((hi - lo, K, V), generator=g, device=device).to(
            torch.bfloat16).view(torch.int16)
        target[lo:hi] = torch.randn((hi - lo, K, V), generator=g, device=device).to(
            torch.bfloat16).view(torch.int16)
    coins = torch.rand((drafts, K), generator=g, device=device) < p_plant
    planted = torch.cumprod(coins.to(torch.int32), dim=1).bool()      # leading run only
    where = torch.randint(0, V, (drafts, K), generator=g, device=device)
    flat = (torch.arange(drafts * K, device=device) * V + where.flatten())[planted.flatten()]
    draft.view(-1)[flat] = PLANT_VALUE_BITS
    target.view(-1)[flat] = PLANT_VALUE_BITS
    return dict(draft_logits=draft, target_logits=target,
                planted=planted.sum(dim=1).to(torch.int32))


def decode_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Context length of each of B requests, uniform in [lo, hi]."""
    return _rng(seed, TAG_LENGTHS).integers(lo, hi + 1, size=B).astype(np.int64)


def decode_inputs(seed: int, lens, K: int, Hq: int, Hkv: int, D: int) -> dict:
    """Host inputs of the decode shape: cu_ctx int32 [B+1]; k_cache and v_cache
    [sum(lens), Hkv, D] (the cache keys are taken as already rotated); q [B, K, Hq, D] and
    k, v [B, K, Hkv, D] of the new rows (pre-RoPE). bf16 bits of N(0, 1)."""
    lens = np.asarray(lens, dtype=np.int64)
    B, L = len(lens), int(lens.sum())
    return dict(cu_ctx=np.concatenate([[0], np.cumsum(lens)]).astype(np.int32),
                k_cache=normal_bf16(seed, TAG_CACHE_K, (L, Hkv, D)),
                v_cache=normal_bf16(seed, TAG_CACHE_V, (L, Hkv, D)),
                q=normal_bf16(seed, TAG_NEW_Q, (B, K, Hq, D)),
                k=normal_bf16(seed, TAG_NEW_K, (B, K, Hkv, D)),
                v=normal_bf16(seed, TAG_NEW_V, (B, K, Hkv, D)))


def decode_inputs_device(seed: int, lens, K: int, Hq: int, Hkv: int, D: int, device="cuda"):
    """The same shapes drawn on the device with torch's seeded generator (for caches of
    gigabytes, where host generation would dominate). N(0, 1) rounded to bf16 (nearest
    even); returned as int16 bit patterns, cu_ctx as int32."""
    import torch
    lens = np.asarray(lens, dtype=np.int64)
    B, L = len(lens), int(lens.sum())

    def draw(tag, shape):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed) * 1000003 + tag)
        out = torch.empty(shape, dtype=torch.int16, device=device)
        flat = out.view(-1)
        step = 1 << 26
        for lo in range(0, flat.numel(), step):
            hi = min(flat.numel(), lo + step)
            x = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
            flat[lo:hi] = x.to(torch.bfloat16).view(torch.int16)
        return out

    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(cu_ctx=torch.from_numpy(cu).to(device),
                k_cache=draw(TAG_CACHE_K, (L, Hkv, D)), v_cache=draw(TAG_CACHE_V, (L, Hkv, D)),
                q=draw(TAG_NEW_Q, (B, K, Hq, D)), k=draw(TAG_NEW_K, (B, K, Hkv, D)),
                v=draw(TAG_NEW_V, (B, K, Hkv, D)))


def layer1_weights(seed: int, H: int, Hq: int, Hkv: int, D: int) -> dict:
    """Random-init weights of the first draft layer's attention input: the two RMSNorm
    weight vectors (bf16 of 1 + N(0, 0.1^2), near the unit init of a trained norm) and the
    stacked q/k/v projection [(Hq + 2 Hkv) D, 2H] (bf16 of N(0, 1/(2H)), fan-in scaled:
    unit-RMS rows in give q, k, v of unit variance, the scale of the attention's own
    synthetic inputs)."""
    def near_one(tag):
        x = 1.0 + 0.1 * _rng(seed, tag).standard_normal(H, dtype=np.float32)
        return f32_to_bf16_bits(x.astype(np.float32))
    return dict(w_norm_emb=near_one(TAG_NORM_EMB), w_norm_hidden=near_one(TAG_NORM_HID),
                w_qkv=normal_bf16(seed, TAG_WQKV, ((Hq + 2 * Hkv) * D, 2 * H),
                                  std=float(1.0 / np.sqrt(2 * H))))


def layer1_inputs(seed: int, n: int, T: int, H: int) -> dict:
    """Stand-ins for the fused stage's outputs with their structure: hidden float32
    [T, H] and embed bf16 [T, H] of N(0, 1), rows n .. T-1 (the depth >= 1 rows) all equal
    to row n."""
    hidden = _rng(seed, TAG_L1_HID).standard_normal((min(T, n + 1), H), dtype=np.float32)
    embed = normal_bf16(seed, TAG_L1_EMB, (min(T, n + 1), H))
    if T > n + 1:
        hidden = np.concatenate([hidden, np.repeat(hidden[n:n + 1], T - n - 1, axis=0)])
        embed = np.concatenate([embed, np.repeat(embed[n:n + 1], T - n - 1, axis=0)])
    return dict(hidden=np.ascontiguousarray(hidden), embed=np.ascontiguousarray(embed))


def layer1_post_weights(seed: int, H: int, QW: int, I: int, V: int = DRAFT_VOCAB) -> dict:
    """Random-init weights of the rest of the first layer and the draft head: RMSNorm
    weights bf16 of 1 + N(0, 0.1^2); projections bf16 of N(0, 1/fan_in) (W_o [H, QW],
    W_gate and W_up [I, H], W_down [H, I], W_head [V, H])."""
    def near_one(tag):
        x = 1.0 + 0.1 * _rng(seed, tag).standard_normal(H, dtype=np.float32)
        return f32_to_bf16_bits(x.astype(np.float32))
    return dict(w_o=normal_bf16(seed, TAG_WO, (H, QW), std=float(1 / np.sqrt(QW))),
                w_post=near_one(TAG_NORM_POST),
                w_gate=normal_bf16(seed, TAG_WGATE, (I, H), std=float(1 / np.sqrt(H))),
                w_up=normal_bf16(seed, TAG_WUP, (I, H), std=float(1 / np.sqrt(H))),
                w_down=normal_bf16(seed, TAG_WDOWN, (H, I), std=float(1 / np.sqrt(I))),
                w_final=near_one(TAG_NORM_FINAL),
                w_head=normal_bf16(seed, TAG_WHEAD, (V, H), std=float(1 / np.sqrt(H))))


def stacked_layer_weights(seed: int, layer: int, H: int, Hq: int, Hkv: int, D: int,
                          I: int) -> dict:
    """Random-init weights of stacked draft layer `layer` (2, 3, ...): RMSNorm weights bf16
    of 1 + N(0, 0.1^2); projections bf16 of N(0, 1/fan_in) (W_qkv [(Hq + 2 Hkv) D, H], W_o
    [H, Hq D], W_gate and W_up [I, H], W_down [H, I])."""
    t0 = TAG_STACK + 8 * (layer - 2)

    def near_one(tag):
        x = 1.0 + 0.1 * _rng(seed, tag).standard_normal(H, dtype=np.float32)
        return f32_to_bf16_bits(x.astype(np.float32))
    QW = Hq * D
    return dict(w_norm=near_one(t0),
                w_qkv=normal_bf16(seed, t0 + 1, ((Hq + 2 * Hkv) * D, H), std=float(1 / np.sqrt(H))),
                w_o=normal_bf16(seed, t0 + 2, (H, QW), std=float(1 / np.sqrt(QW))),
                w_post=near_one(t0 + 3),
                w_gate=normal_bf16(seed, t0 + 4, (I, H), std=float(1 / np.sqrt(H))),
                w_up=normal_bf16(seed, t0 + 5, (I, H), std=float(1 / np.sqrt(H))),
                w_down=normal_bf16(seed, t0 + 6, (H, I), std=float(1 / np.sqrt(I))))


def residual_standin(seed: int, T: int, H: int) -> np.ndarray:
    """Stand-in for a layer's output h [T, H] (float32 N(0, 1), every row distinct), the
    input of the next stacked layer."""
    return _rng(seed, TAG_STACK + 7).standard_normal((T, H), dtype=np.float32)


def attention_out_standin(seed: int, T: int, QW: int) -> np.ndarray:
    """A stand-in for the attention output [T, QW] (float32): softmax-weighted averages of
    N(0, 1) values have magnitudes below 1; drawn as N(0, 0.3^2)."""
    return (0.3 * _rng(seed, TAG_ATTN).standard_normal((T, QW), dtype=np.float32)).astype(np.float32)


def verify_logits_d2t(seed: int, drafts: int, K: int, Vd: int, Vt: int, p_plant: float,
                      chunk: int = 256) -> dict:
    """Verification inputs with a draft vocabulary of Vd ids inside a target vocabulary of
    Vt: d2t is a seeded sorted subset of [0, Vt) (int32 [Vd]); draft logits [drafts, K, Vd]
    and target logits [drafts, K, Vt] are bf16 bits of N(0, 1), with planted shared maxima
    (16.0 at draft id j and at target id d2t[j]) along a geometric prefix as in
    verify_logits."""
    d2t = np.sort(_rng(seed, TAG_D2T).choice(Vt, size=Vd, replace=False)).astype(np.int32)
    rng = _rng(seed, TAG_LOGITS)
    plant_rng = _rng(seed, TAG_LOGITS + 100)
    draft = np.empty((drafts, K, Vd), dtype=np.uint16)
    target = np.empty((drafts, K, Vt), dtype=np.uint16)
    for lo in range(0, drafts, chunk):
        hi = min(drafts, lo + chunk)
        draft[lo:hi] = f32_to_bf16_bits(rng.standard_normal((hi - lo) * K * Vd, dtype=np.float32)).reshape(hi - lo, K, Vd)
        target[lo:hi] = f32_to_bf16_bits(rng.standard_normal((hi - lo) * K * Vt, dtype=np.float32)).reshape(hi - lo, K, Vt)
    coins = plant_rng.random((drafts, K)) < p_plant
    where = plant_rng.integers(0, Vd, size=(drafts, K))
    planted = np.zeros(drafts, dtype=np.int32)
    for i in range(drafts):
        for d in range(K):
            if not coins[i, d]:
                break
            draft[i, d, where[i, d]] = PLANT_VALUE_BITS
            target[i, d, d2t[where[i, d]]] = PLANT_VALUE_BITS
            planted[i] += 1
    return dict(draft_logits=draft, target_logits=target, d2t=d2t, planted=planted)


def fc_norm_weight(seed: int, H: int) -> np.ndarray:
    """bf16 bits of 1 + N(0, 0.1^2): the RMSNorm weight after fc (near its unit init)."""
    x = 1.0 + 0.1 * _rng(seed, TAG_FC_NORM).standard_normal(H, dtype=np.float32)
    return f32_to_bf16_bits(x.astype(np.float32))


def sampled_verify_inputs(seed: int, drafts: int, K: int, V: int, spread: float = 2.0,
                          noise: float = 0.5, chunk: int = 64) -> dict:
    """Inputs of sampling verification: draft and target logits [drafts, K, V] (bf16 bits)
    that share a N(0, spread^2) base and differ by independent N(0, noise^2) terms; one
    drafted token per row, uniform over the vocabulary, whose draft logit is raised by
    b ~ U(0, 6) and target logit by b + N(0, 1) so the acceptance ratios spread around 1;
    uniforms u [drafts, K] and w [drafts] (float32, in [0, 1))."""
    rng = _rng(seed, TAG_SPEC_LOGITS)
    draft = np.empty((drafts, K, V), dtype=np.uint16)
    target = np.empty((drafts, K, V), dtype=np.uint16)
    trng = _rng(seed, TAG_SPEC_TOK)
    tok = trng.integers(0, V, size=(drafts, K)).astype(np.int32)
    b_d = trng.uniform(0.0, 6.0, size=(drafts, K)).astype(np.float32)
    b_t = (b_d + trng.standard_normal((drafts, K))).astype(np.float32)
    for lo in range(0, drafts, chunk):
        hi = min(drafts, lo + chunk)
        shape = (hi - lo, K, V)
        base = spread * rng.standard_normal(shape, dtype=np.float32)
        dl = base + noise * rng.standard_normal(shape, dtype=np.float32)
        tl = base + noise * rng.standard_normal(shape, dtype=np.float32)
        ii, dd = np.meshgrid(np.arange(hi - lo), np.arange(K), indexing="ij")
        dl[ii, dd, tok[lo:hi]] += b_d[lo:hi]
        tl[ii, dd, tok[lo:hi]] += b_t[lo:hi]
        draft[lo:hi] = f32_to_bf16_bits(dl)
        target[lo:hi] = f32_to_bf16_bits(tl)
    u = _rng(seed, TAG_SPEC_U).random((drafts, K), dtype=np.float32)
    w = _rng(seed, TAG_SPEC_W).random(drafts, dtype=np.float32)
    return dict(draft_logits=draft, target_logits=target, draft_tok=tok, u=u, w=w)


def with_bonus_row(inp: dict, seed: int, spread: float = 2.0) -> dict:
    """The same inputs with a K+1-th target row per draft (the target's distribution after
    the last drafted token): bf16 of N(0, spread^2) logits, target_logits [drafts, K+1, V]."""
    N, K, V = inp["target_logits"].shape
    rng = _rng(seed, TAG_SPEC_BONUS)
    row = f32_to_bf16_bits(spread * rng.standard_normal((N, 1, V), dtype=np.float32))
    return dict(inp, target_logits=np.concatenate([inp["target_logits"], row], axis=1))


def sampled_verify_inputs_device(seed: int, drafts: int, K: int, V: int, spread: float = 2.0,
                                 noise: float = 0.5, device="cuda") -> dict:
    """The recipe of sampled_verify_inputs drawn on the device with torch's seeded
    generator (gigabytes of logits at full size). Logits as int16 bf16 bit patterns."""
    import torch

    def gen(tag):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed) * 1000003 + tag)
        return g

    g_tok, g_log = gen(TAG_SPEC_TOK), gen(TAG_SPEC_LOGITS)
    tok = torch.randint(0, V, (drafts, K), generator=g_tok, device=device, dtype=torch.int32)
    b_d = 6.0 * torch.rand((drafts, K), generator=g_tok, device=device)
    b_t = b_d + torch.randn((drafts, K), generator=g_tok, device=device)
    draft = torch.empty((drafts, K, V), dtype=torch.int16, device=device)
    target = torch.empty_like(draft)
    rows = max(1, (1 << 25) // (K * V))
    for lo in range(0, drafts, rows):
        hi = min(drafts, lo + rows)
        shape = (hi - lo, K, V)
        base = spread * torch.randn(shape, generator=g_log, device=device)
        dl = base + noise * torch.randn(shape, generator=g_log, device=device)
        tl = base + noise * torch.randn(shape, generator=g_log, device=device)
        idx = tok[lo:hi].long().unsqueeze(-1)
        dl.scatter_add_(2, idx, b_d[lo:hi].unsqueeze(-1))
        tl.scatter_add_(2, idx, b_t[lo:hi].unsqueeze(-1))
        draft[lo:hi] = dl.to(torch.bfloat16).view(torch.int16)
        target[lo:hi] = tl.to(torch.bfloat16).view(torch.int16)
        del base, dl, tl
    u = torch.rand((drafts, K), generator=gen(TAG_SPEC_U), device=device)
    w = torch.rand(drafts, generator=gen(TAG_SPEC_W), device=device)
    return dict(draft_logits=draft, target_logits=target, draft_tok=tok, u=u, w=w)


def attn_grad_out(seed: int, T: int, Hq: int, D: int) -> np.ndarray:
    """dL/d out of the draft attention [T, Hq, D]: float32 N(0, 1) (the backward's input)."""
    return _rng(seed, TAG_DOUT).standard_normal((T, Hq, D), dtype=np.float32)


def ce_inputs(seed: int, T: int, V: int, p_mask: float = 0.05, spread: float = 2.0) -> dict:
    """Draft-vocab logits [T, V] (bf16 bits of N(0, spread^2)) and labels [T] (int32,
    uniform over [0, V), a p_mask share set to -1: targets outside the draft vocabulary)."""
    logits = normal_bf16(seed, TAG_CE_LOGITS, (T, V), std=spread)
    rng = _rng(seed, TAG_CE_LABELS)
    labels = rng.integers(0, V, size=T).astype(np.int32)
    labels[rng.random(T) < p_mask] = -1
    return dict(logits=logits, labels=labels)
