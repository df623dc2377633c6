"""Benchmark of the P-EAGLE draft forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic inputs resident in
HBM: COD index build, fused input stage (fc GEMM + mask/ptd substitution), RoPE table,
RoPE gather + draft attention, and greedy verification. The default workload is the
32K-context, K=4 Gemma-270M-shaped drafter (n = 32768, 4 q heads / 1 kv head, head dim
256); its verification stage scores 4096 drafts of K=4 tokens over a 32000 vocabulary.

Prints one JSON line. `value` is useful draft-attention TFLOP/s over the whole step
(4 * D * Hq * allowed query-key pairs, divided by the step time); the attention call
alone, drafted tokens/s and the per-kernel split are reported beside it.

The decode-shaped draft attention (K new rows per request over a KV cache) is timed
beside it on its two inference workloads and reported under "decode": HBM GB/s of the
whole call (cache bytes plus new rows and outputs over the call time) and drafted
tokens/s. `--decode only` prints a line for it alone.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle sample size in query rows (0: sized for about 10-20 s of "
                         "host time from the oracle's cost per row, Hq * T * D)")
    ap.add_argument("--k-sweep", action="store_true",
                    help="time only the draft attention at n = 32768 (4 q / 1 kv heads, head "
                         "dim 256, r = 0.7, r_min = 0.2) for K = 1, 2, 4, 8, 16")
    ap.add_argument("--decode", choices=["all", "none", "only"], default="all",
                    help="also time the decode-shaped draft attention on its inference "
                         "workloads (all), skip it (none), or time only it (only)")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the step of the chosen workload (no draft layers, backward, "
                         "loss or verification variants)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other four workloads and the depth sweep on the Llama-8B "
                         "shape")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the timed steps, "
                         "so a counter run can scale its byte counters against known traffic")
    return ap.parse_args()


TRAFFIC_RECORDS = {4: "profiles/attn_core_gemma270m_32k_K4_traffic.md",
                   5: "profiles/attn_core_llama8b_16k_K8_traffic.md",
                   3: "profiles/attn_core_packed8_llama8b_4k_traffic.md",
                   2: "profiles/attn_core_gemma270m_4k_traffic.md",
                   1: "profiles/attn_core_tiny256_traffic.md"}
DECODE_TRAFFIC_RECORD = "profiles/decode_attn_B64_ctx1k-32k_traffic.md"


def traffic_bytes(config):
    """HBM bytes per attention-core call from the stored counter record (calibrated
    FETCH_SIZE + WRITE_SIZE), or None when there is none for this workload or it was taken
    on different kernel sources."""
    from token_drafting_amd import profiling
    path = TRAFFIC_RECORDS.get(config)
    if path is None:
        return None
    rec = profiling.recorded_traffic(os.path.join(os.path.dirname(os.path.abspath(__file__)), path))
    return None if rec is None else int(round(rec["core_call_bytes"]))


def useful_pairs(idx, depth_off, cu):
    """Allowed (query row, key row) pairs per head: sum over rows of (p - a_s + 1) + d."""
    idx = idx.astype(np.int64)
    depth = np.repeat(np.arange(len(depth_off) - 1), np.diff(depth_off))
    seq = np.searchsorted(cu, idx, side="right") - 1
    return int(np.sum(idx - cu[seq] + 1 + depth)), idx - cu[seq] + 1 + depth


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the draft forward has no multi-GPU path; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from token_drafting_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibration_copy_mib:
        nbytes = args.calibration_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.k_sweep:
        print(json.dumps({"k_sweep": [k_sweep_point(K, args.steps, args.warmup)
                                      for K in (1, 2, 4, 8, 16)]}), flush=True)
        return
    if args.decode == "only":
        res = {name: decode_bench(name, args.steps, args.warmup)
               for name in sorted(synth.DECODE_CONFIGS)}
        loop = {name: decode_loop_bench(name, args.steps, args.warmup)
                for name in sorted(synth.DECODE_CONFIGS)}
        print(json.dumps({"decode": res, "decode_loop": loop}), flush=True)
        return

    head, ctx = step_bench(args.config, args.steps, args.warmup, cpu=not args.no_cpu_baseline,
                           cpu_rows=args.cpu_rows, keep=True)
    cfg = synth.CONFIGS[args.config]
    result = {
        "metric": "draft-attn fwd TFLOP/s + drafted tokens/s, 32K ctx K=4; % of bf16 MFMA peak",
        "value": head["step_attn_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "attn_core_tflops": head["attn_core_tflops"],
        "attn_core_frac_bf16_peak": head["attn_core_frac_bf16_peak"],
        "drafted_tokens_per_s": head["drafted_tokens_per_s"],
        "pipeline_tokens_per_s": head["pipeline_tokens_per_s"],
        "stage_ms": head["stage_ms"],
        "stage_rate": head["stage_rate"],
        "stage_rate_cold": head["stage_rate_cold"],
        "roofline": {"kernel": "attn_core_kernel (the launches of one peagle_draft_attn_core call)",
                     "bound": "mfma", "achieved": head["attn_core_tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": head["attn_core_frac_bf16_peak"],
                     "traffic": traffic_bytes(args.config)},
        "input_gen_s": head["input_gen_s"],
        "wall_s_timed": head["wall_s_timed"],
    }
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]

    if args.step_only:
        print(json.dumps(result), flush=True)
        return
    seed, n, K, T, H = args.config, cfg["n"], cfg["K"], head["config"]["draft_rows"], cfg["H"]
    d, sel, q, k, v = ctx["d"], ctx["sel"], ctx["q"], ctx["k"], ctx["v"]
    from token_drafting_amd import peagle
    wn = torch.from_numpy(synth.fc_norm_weight(seed, H).view(np.int16)).to(q.device)
    ms_fcn = _time_calls(lambda: peagle.fuse_inputs(
        n, K, T, sel["idx"], d["aux"], d["fc_weight"], d["mask_hidden"], d["tokens"], d["embed"],
        ctx["ptd"], ctx["hidden"], ctx["emb"], fc_norm_weight=wn), args.steps, args.warmup)
    result["fuse_fc_norm"] = {"ms_per_call": round(ms_fcn, 4),
                              "ms_without_fc_norm": head["stage_ms"]["fuse_inputs"]}
    result["attn_bwd"] = attn_bwd_bench(n, K, sel, d["cu_seqlens"], q, k, v, ctx["cos"], ctx["sin"],
                                        ctx["out"], ctx["lse"], seed, head["config"][
                                            "useful_pairs_per_head"], args.steps, args.warmup)
    result["depth_ce"] = depth_ce_bench(sel["depth_off"], args.steps, args.warmup)
    result["verify_d2t"] = verify_d2t_bench(args.steps, args.warmup)
    result["verify_sampled"] = verify_sampled_bench(args.steps, args.warmup)
    result["draft_layer"] = layer_bench(args.config, cfg, seed, n, K, T, ctx["hidden"], ctx["emb"],
                                        ctx["out"], args.steps, args.warmup)
    del d, sel, q, k, v, wn
    ctx.clear()
    torch.cuda.empty_cache()

    if args.decode == "all":
        result["decode"] = {name: decode_bench(name, args.steps, args.warmup)
                            for name in sorted(synth.DECODE_CONFIGS)}
        result["decode_loop"] = {name: decode_loop_bench(name, args.steps, args.warmup)
                                 for name in sorted(synth.DECODE_CONFIGS)}
    if not args.headline_only:
        # the other four workloads, each a whole step of its own with the oracle beside it
        result["configs"] = {}
        for c in sorted(synth.CONFIGS):
            if c != args.config:
                result["configs"][str(c)] = step_bench(c, args.steps, args.warmup,
                                                       cpu=not args.no_cpu_baseline)[0]
                torch.cuda.empty_cache()
        # depth sweep on the Llama-8B-shaped drafter at n = 16384
        result["k_sweep_llama8b_16k"] = [
            k_sweep_point(Kx, args.steps, args.warmup, n=16384, Hq=32, Hkv=8, D=128,
                          theta=5.0e5) for Kx in (1, 2, 4, 8)]
    print(json.dumps(result), flush=True)


def _cold_ms(call, evict, reps):
    """Mean time of `call` with the 256 MB last-level cache (MALL) evicted before each rep by
    writing `evict` (>= 512 MB) on the same stream."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        evict.fill_(i + 1)
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))


def step_bench(cfg_id, steps, warmup, cpu=True, cpu_rows=0, keep=False):
    """One workload: W untimed and K timed steps of the whole path (COD select, fused
    inputs, RoPE table, attention prepare + core, verification), per-stage HIP events, then
    the HBM-bound stages again with the last-level cache evicted (cold), and the oracle on a
    bounded sample. Returns (summary dict, tensors kept for further timing when `keep`)."""
    import torch
    from token_drafting_amd import peagle, synth

    cfg = synth.CONFIGS[cfg_id]
    seed = cfg_id
    n, K, Hq, Hkv, D = cfg["n"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- inputs (seeded) -> HBM
    t0 = time.time()
    m, T = peagle.cod_counts(n, K, cfg["r"], cfg["r_min"])
    base = synth.base_inputs(cfg, seed)
    qkv = synth.qkv_inputs(seed, T, Hq, Hkv, D)
    vcfg = cfg.get("verify") or dict(drafts=4096, K=K, V=32000, p_plant=0.7)
    logits = synth.verify_logits_device(seed, vcfg["drafts"], vcfg["K"], vcfg["V"], vcfg["p_plant"])
    cu_h = base["cu_seqlens"]
    d = {k2: to_dev(v2) for k2, v2 in base.items() if isinstance(v2, np.ndarray)}
    q, k, v = (to_dev(qkv[t]) for t in ("q", "k", "v"))
    dl, tl = logits["draft_logits"], logits["target_logits"]
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    S = cu_h.size - 1
    H = cfg["H"]
    max_pos = peagle.rope_max_pos(n, K)
    sel = dict(m=m, T=T, idx=torch.empty(T, dtype=torch.int32, device=dev),
               depth_off=torch.empty(K + 1, dtype=torch.int32, device=dev),
               cu_seqlens_d=torch.empty((K, S + 1), dtype=torch.int32, device=dev),
               row_of=torch.empty((K, n), dtype=torch.int32, device=dev),
               workspace=torch.empty(peagle.cod_workspace_bytes(n, K), dtype=torch.uint8,
                                     device=dev))
    hidden = torch.empty((T, H), dtype=torch.float32, device=dev)
    emb = torch.empty((T, H), dtype=torch.int16, device=dev)
    cos = torch.empty((max_pos + 1, D // 2), dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(peagle.attn_workspace_bytes(n, T, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    Nd, Kv = vcfg["drafts"], vcfg["K"]
    dtok = torch.empty((Nd, Kv), dtype=torch.int32, device=dev)
    ttok = torch.empty((Nd, Kv), dtype=torch.int32, device=dev)
    alen = torch.empty(Nd, dtype=torch.int32, device=dev)
    lib = peagle.lib()

    stages = ["cod_select", "fuse_inputs", "rope_table", "attn_prepare", "attn_core", "accept_prefix"]
    calls = [
        lambda: peagle.cod_select_into(n, K, cfg["r"], cfg["r_min"], seed, d["cu_seqlens"], sel),
        lambda: peagle.fuse_inputs(n, K, T, sel["idx"], d["aux"], d["fc_weight"], d["mask_hidden"],
                                   d["tokens"], d["embed"], base["ptd_token_id"], hidden, emb),
        lambda: peagle._check("peagle_rope_table", lib.peagle_rope_table(
            D, cfg["theta"], max_pos, peagle._ptr(cos), peagle._ptr(sin), peagle._stream())),
        lambda: peagle.draft_attn(n, K, sel, d["cu_seqlens"], q, k, v, cos, sin, out, lse, ws,
                                  phase="prepare"),
        lambda: peagle.draft_attn(n, K, sel, d["cu_seqlens"], q, k, v, cos, sin, out, lse, ws,
                                  phase="core"),
        lambda: peagle.accept_prefix(dl, tl, dtok, ttok, alen),
    ]

    def step(ev=None):
        for i, call in enumerate(calls):
            if ev is not None:
                ev[i].record()
            call()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(len(calls))]
                    for i in range(steps)])
    stage_ms = dict(zip(stages, per.mean(axis=0).tolist()))
    ms_step = wall * 1e3 / steps

    # HBM-bound stages with the last-level cache evicted before each call
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_reps = max(3, min(steps, 10))
    cold_ms = {name: _cold_ms(calls[i], evict, cold_reps)
               for i, name in enumerate(stages) if name in ("cod_select", "attn_prepare",
                                                            "accept_prefix")}
    del evict

    # ---------------- accounting
    idx_h = sel["idx"].cpu().numpy()
    off_h = sel["depth_off"].cpu().numpy()
    P, _ = useful_pairs(idx_h, off_h, cu_h)
    attn_flop = 4.0 * D * Hq * P
    core_ms = stage_ms["attn_core"]
    attn_call_ms = stage_ms["attn_prepare"] + core_ms
    core_tflops = attn_flop / (core_ms * 1e-3) / 1e12
    # algorithmic bytes of the HBM-bound stages
    rope_bytes = T * (Hq + Hkv) * D * 2 * 2 + T * D * 4
    verify_bytes = 2 * Nd * Kv * vcfg["V"] * 2 + 8 * Nd * Kv + 4 * Nd
    cod_bytes = 4 * T + 4 * K * n + 4 * K * (S + 1) + 4 * (K + 1)
    fc_flop = 2.0 * (n + 1) * cfg["aux_dim"] * H

    def gbps(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 2)

    summary = {
        "config": {"workload": cfg["workload"], "n": n, "K": K, "r": cfg["r"], "r_min": cfg["r_min"],
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "draft_rows": T,
                   "packed_sequences": S, "useful_pairs_per_head": P,
                   "verify": f"{Nd}x{Kv}x{vcfg['V']}"},
        "ms_per_step": round(ms_step, 4),
        "step_attn_tflops": round(attn_flop / (ms_step * 1e-3) / 1e12, 3),
        "attn_core_tflops": round(core_tflops, 2),
        "attn_core_frac_bf16_peak": round(core_tflops / PEAK_BF16_TFLOPS, 4),
        "drafted_tokens_per_s": round(T / (attn_call_ms * 1e-3), 1),
        "pipeline_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "stage_ms": {k2: round(v2, 4) for k2, v2 in stage_ms.items()},
        "stage_rate": {
            "cod_select_GBps": gbps(cod_bytes, stage_ms["cod_select"]),
            "fuse_fc_TFLOPs": round(fc_flop / (stage_ms["fuse_inputs"] * 1e-3) / 1e12, 2),
            "fuse_fc_frac_bf16_peak": round(fc_flop / (stage_ms["fuse_inputs"] * 1e-3) / 1e12
                                            / PEAK_BF16_TFLOPS, 4),
            "attn_prepare_rope_GBps": gbps(rope_bytes, stage_ms["attn_prepare"]),
            "accept_prefix_GBps": gbps(verify_bytes, stage_ms["accept_prefix"]),
        },
        "stage_rate_cold": {
            "note": "the 256 MB last-level cache evicted (512 MB written) before each call",
            "cod_select_GBps": gbps(cod_bytes, cold_ms["cod_select"]),
            "attn_prepare_rope_GBps": gbps(rope_bytes, cold_ms["attn_prepare"]),
            "accept_prefix_GBps": gbps(verify_bytes, cold_ms["accept_prefix"]),
            "frac_hbm_peak": {
                "cod_select": round(cod_bytes / (cold_ms["cod_select"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                "attn_prepare_rope": round(rope_bytes / (cold_ms["attn_prepare"] * 1e-3) / 1e9
                                           / PEAK_HBM_GBPS, 4),
                "accept_prefix": round(verify_bytes / (cold_ms["accept_prefix"] * 1e-3) / 1e9
                                       / PEAK_HBM_GBPS, 4)},
        },
        "roofline": {"kernel": "attention core (the launches of one peagle_draft_attn_core call)",
                     "bound": "mfma", "achieved": round(core_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(core_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_bytes(cfg_id)},
        "input_gen_s": round(gen_s, 1),
        "wall_s_timed": round(wall, 4),
    }
    if cpu:
        summary["cpu_baseline"] = cpu_baseline(cfg, seed, qkv, cu_h, idx_h, off_h, cpu_rows)
    ctx = {}
    if keep:
        ctx = dict(d=d, sel=sel, q=q, k=k, v=v, cos=cos, sin=sin, out=out, lse=lse,
                   hidden=hidden, emb=emb, ptd=base["ptd_token_id"])
    del dl, tl, logits, ws
    return summary, ctx


def k_sweep_point(K, steps, warmup, n=32768, Hq=4, Hkv=1, D=256, r=0.7, r_min=0.2,
                  theta=1.0e4):
    """Draft attention (prepare + core) for one depth count K on the headline shape; q, k, v
    drawn on the device (the work does not depend on their values)."""
    import torch
    from token_drafting_amd import peagle

    dev = torch.device("cuda:0")
    cu = torch.tensor([0, n], dtype=torch.int32, device=dev)
    sel = peagle.cod_select(n, K, r, r_min, K, cu)
    T = sel["T"]
    g = torch.Generator(device="cuda")
    g.manual_seed(K)
    q = torch.randn((T, Hq, D), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    k = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    v = torch.randn((T, Hkv, D), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    cos, sin = peagle.rope_table(D, theta, peagle.rope_max_pos(n, K))
    out, lse, ws = peagle.draft_attn(n, K, sel, cu, q, k, v, cos, sin)
    ms = _time_calls(lambda: peagle.draft_attn(n, K, sel, cu, q, k, v, cos, sin, out, lse, ws),
                     steps, warmup)
    P, _ = useful_pairs(sel["idx"].cpu().numpy(), sel["depth_off"].cpu().numpy(),
                        np.array([0, n]))
    tflops = 4.0 * D * Hq * P / (ms * 1e-3) / 1e12
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return {"K": K, "draft_rows": T, "useful_pairs_per_head": P, "attention_ms": round(ms, 4),
            "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "drafted_tokens_per_s": round(T / (ms * 1e-3), 1)}


def verify_d2t_bench(steps, warmup, N=4096, K=8, Vd=8192, Vt=32000):
    """Time peagle_accept_prefix_d2t on 4096 drafts of K = 8 with a draft vocabulary of
    8192 ids inside a 32000-id target vocabulary (logits drawn on the device with torch's
    seeded generator; the argmaxes do not change the work)."""
    import torch
    from token_drafting_amd import peagle

    g = torch.Generator(device="cuda")
    g.manual_seed(29)
    dl = torch.randn((N, K, Vd), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    tl = torch.randn((N, K, Vt), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    d2t = torch.sort(torch.randperm(Vt, generator=g, device="cuda")[:Vd]).values.to(torch.int32)
    outs = [torch.empty((N, K), dtype=torch.int32, device="cuda") for _ in range(2)]
    alen = torch.empty(N, dtype=torch.int32, device="cuda")
    ms = _time_calls(lambda: peagle.accept_prefix_d2t(dl, tl, d2t, outs[0], outs[1], alen), steps,
                     warmup)
    nbytes = N * K * (Vd + Vt) * 2 + N * K * 8 + N * 4
    del dl, tl
    torch.cuda.empty_cache()
    return {"drafts": N, "K": K, "draft_vocab": Vd, "target_vocab": Vt, "ms_per_call": round(ms, 4),
            "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def attn_bwd_bench(n, K, sel, cu, q, k, v, cos, sin, out, lse, seed, pairs, steps, warmup):
    """Time peagle_draft_attn_bwd on the step's own attention inputs and results (the
    forward's out and lse), with a seeded N(0, 1) dL/d out. Algorithmic work: five products
    over the useful (query, key) pairs (S recomputed, dP, dV, dK, dQ), 2 D flop each per
    pair and q head."""
    import torch
    from token_drafting_amd import peagle, synth

    T, Hq, D = q.shape
    Hkv = k.shape[1]
    dout = torch.from_numpy(synth.attn_grad_out(seed, T, Hq, D)).to(q.device)
    dq = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((T, Hkv, D), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    ws = torch.empty(int(peagle.lib().peagle_draft_attn_bwd_workspace_bytes(n, T, Hq, Hkv, D)),
                     dtype=torch.uint8, device=q.device)
    ms = _time_calls(lambda: peagle.draft_attn_bwd(n, K, sel, cu, q, k, v, cos, sin, out, lse,
                                                   dout, dq, dk, dv, ws), steps, warmup)
    flop = 10.0 * D * Hq * pairs
    tf = flop / (ms * 1e-3) / 1e12
    del dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"ms_per_call": round(ms, 4), "tflops": round(tf, 1),
            "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "includes": "forward preparation (RoPE, row list), dO cast, tile layouts, dK/dV, dQ, "
                        "inverse RoPE"}


def depth_ce_bench(depth_off, steps, warmup, V=8192):
    """Time peagle_depth_ce (depth-weighted cross-entropy and its bf16 gradient) over the
    step's draft rows and the 8192-id draft vocabulary; logits N(0, 4) and uniform labels
    drawn on the device with torch's seeded generator. Algorithmic bytes: the logits read
    once and the gradient written once (plus labels)."""
    import torch
    from token_drafting_amd import peagle

    T = int(depth_off[-1].item())
    g = torch.Generator(device="cuda")
    g.manual_seed(37)
    logits = (2.0 * torch.randn((T, V), generator=g, device="cuda")).to(torch.bfloat16).view(torch.int16)
    labels = torch.randint(0, V, (T,), generator=g, device="cuda", dtype=torch.int32)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    dl = torch.empty(depth_off.numel() - 1, dtype=torch.float32, device="cuda")
    grad = torch.empty_like(logits)
    ws = torch.empty(int(peagle.lib().peagle_depth_ce_workspace_bytes(T, depth_off.numel() - 1)),
                     dtype=torch.uint8, device="cuda")
    ms = _time_calls(lambda: peagle.depth_ce(depth_off, logits, labels, 0.8, True, loss, dl, grad,
                                             ws), steps, warmup)
    nbytes = 2 * T * V * 2 + T * 4
    del logits, grad
    torch.cuda.empty_cache()
    return {"rows": T, "vocab": V, "ms_per_call": round(ms, 4),
            "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "loss": round(float(loss.item()), 4)}


def verify_sampled_bench(steps, warmup, N=4096, K=8, V=32000):
    """Time peagle_accept_sampled (speculative-sampling verification) on 4096 drafts of
    K = 8 over a 32000-id vocabulary, inputs of the seeded recipe drawn on the device.
    Algorithmic bytes: both logit tensors read once plus the per-depth inputs and outputs;
    the kernel also re-reads the row pair of the rejected depth (residual draw)."""
    import torch
    from token_drafting_amd import peagle, synth

    d = synth.sampled_verify_inputs_device(41, N, K, V)
    alen = torch.empty(N, dtype=torch.int32, device="cuda")
    nxt = torch.empty(N, dtype=torch.int32, device="cuda")
    ms = _time_calls(lambda: peagle.accept_sampled(d["draft_logits"], d["target_logits"],
                                                   d["draft_tok"], d["u"], d["w"], 1.0, alen,
                                                   nxt), steps, warmup)
    rejected = int((alen < K).sum())
    nbytes = N * K * V * 2 * 2 + N * K * 8 + N * 12
    del d
    torch.cuda.empty_cache()
    return {"drafts": N, "K": K, "vocab": V, "rejected_drafts": rejected,
            "ms_per_call": round(ms, 4), "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def _time_calls(call, steps, warmup):
    import torch
    for _ in range(warmup):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))


def layer_bench(cfg_id, cfg, seed, n, K, T, hidden, emb, attn_out, steps, warmup):
    """Time the first draft layer's other stages on the step's own tensors: attention
    inputs (RMSNorm halves and concat, QKV GEMM on rows 0..n, copy of row n) from the fused
    stage's outputs; the rest of the layer (output projection and residual, RMSNorm,
    SwiGLU MLP and residual) from the step's attention output; the draft-vocab head with
    its fused argmax on the result."""
    import torch
    from token_drafting_amd import peagle, synth

    H, Hq, Hkv, D = cfg["H"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    QW, I, V = Hq * D, synth.LAYER_SHAPES.get(cfg_id, {"I": 4 * H})["I"], synth.DRAFT_VOCAB
    dev = hidden.device
    dw = {k2: torch.from_numpy(v2.view(np.int16)).to(dev)
          for k2, v2 in {**synth.layer1_weights(seed, H, Hq, Hkv, D),
                         **synth.layer1_post_weights(seed, H, QW, I, V)}.items()}
    q = torch.empty((T, Hq, D), dtype=torch.int16, device=dev)
    k = torch.empty((T, Hkv, D), dtype=torch.int16, device=dev)
    v = torch.empty((T, Hkv, D), dtype=torch.int16, device=dev)
    ws_qkv = torch.empty(peagle.layer1_qkv_workspace_bytes(n, T, H), dtype=torch.uint8, device=dev)
    h2 = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_post = torch.empty(int(peagle.lib().peagle_layer1_post_workspace_bytes(n, T, H, QW, I)),
                          dtype=torch.uint8, device=dev)
    tokens = torch.empty(T, dtype=torch.int32, device=dev)
    ws_head = torch.empty(int(peagle.lib().peagle_draft_head_workspace_bytes(T, H, V)),
                          dtype=torch.uint8, device=dev)
    ms_qkv = _time_calls(lambda: peagle.layer1_qkv(
        n, K, T, hidden, emb, dw["w_norm_emb"], dw["w_norm_hidden"], dw["w_qkv"], Hq, Hkv, D,
        q=q, k=k, v=v, workspace=ws_qkv), steps, warmup)
    ms_post = _time_calls(lambda: peagle.layer1_post(
        n, K, T, attn_out, hidden, dw["w_norm_hidden"], dw["w_o"], dw["w_post"], dw["w_gate"],
        dw["w_up"], dw["w_down"], h2=h2, workspace=ws_post), steps, warmup)
    ms_head = _time_calls(lambda: peagle.draft_head(h2, dw["w_final"], dw["w_head"],
                                                    tokens=tokens, workspace=ws_head),
                          steps, warmup)
    # a stacked (2nd) layer on the first layer's output: every row projected
    w2 = {k2: torch.from_numpy(v2.view(np.int16)).to(dev)
          for k2, v2 in synth.stacked_layer_weights(seed, 2, H, Hq, Hkv, D, I).items()}
    ws2_qkv = torch.empty(int(peagle.lib().peagle_layer_qkv_workspace_bytes(T, H)),
                          dtype=torch.uint8, device=dev)
    ws2_post = torch.empty(int(peagle.lib().peagle_layer_post_workspace_bytes(T, H, QW, I)),
                           dtype=torch.uint8, device=dev)
    h3 = torch.empty_like(h2)
    ms_qkv2 = _time_calls(lambda: peagle.layer_qkv(h2, w2["w_norm"], w2["w_qkv"], Hq, Hkv, D, q=q,
                                                   k=k, v=v, workspace=ws2_qkv), steps, warmup)
    ms_post2 = _time_calls(lambda: peagle.layer_post(attn_out, h2, w2["w_o"], w2["w_post"],
                                                     w2["w_gate"], w2["w_up"], w2["w_down"],
                                                     h2=h3, workspace=ws2_post), steps, warmup)
    del w2, ws2_qkv, ws2_post, h3
    M = n + 1 if T > n else n
    f_qkv = 2.0 * M * (Hq + 2 * Hkv) * D * 2 * H
    f_post = 2.0 * T * H * (QW + 3 * I)
    f_head = 2.0 * T * H * V
    del q, k, v, ws_qkv, h2, ws_post, tokens, ws_head, dw
    torch.cuda.empty_cache()
    tf = lambda f, ms: round(f / (ms * 1e-3) / 1e12, 1)
    return {"intermediate": I, "draft_vocab": V,
            "qkv": {"rows_projected": M, "draft_rows": T, "gemm": f"{M}x{(Hq + 2 * Hkv) * D}x{2 * H}",
                    "ms_per_call": round(ms_qkv, 4), "tflops": tf(f_qkv, ms_qkv),
                    "flop_saved_vs_all_rows": round(1.0 - M / T, 4)},
            "post": {"gemms": f"{T}x{H}x{QW}, {T}x{2 * I}x{H}, {T}x{H}x{I}",
                     "ms_per_call": round(ms_post, 4), "tflops": tf(f_post, ms_post)},
            "head": {"gemm": f"{T}x{V}x{H} with fused argmax", "ms_per_call": round(ms_head, 4),
                     "tflops": tf(f_head, ms_head)},
            "layer_ms_excluding_attention": round(ms_qkv + ms_post + ms_head, 4),
            "stacked_layer": {
                "qkv": {"gemm": f"{T}x{(Hq + 2 * Hkv) * D}x{H}", "ms_per_call": round(ms_qkv2, 4),
                        "tflops": tf(2.0 * T * (Hq + 2 * Hkv) * D * H, ms_qkv2)},
                "post": {"ms_per_call": round(ms_post2, 4), "tflops": tf(f_post, ms_post2)},
                "ms_excluding_attention": round(ms_qkv2 + ms_post2, 4)}}


def decode_bench(name, steps, warmup):
    """Time peagle_draft_decode_attn (prep, split-KV attention, combine) on one inference
    workload with its inputs resident in HBM; the V cache is laid out in tiles first, as a
    server keeps it, and that conversion is not timed."""
    import torch
    from token_drafting_amd import peagle, synth

    cfg = synth.DECODE_CONFIGS[name]
    seed = 31
    B, K, Hq, Hkv, D = cfg["B"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    lens = synth.decode_lengths(seed, B, cfg["ctx_lo"], cfg["ctx_hi"])
    inp = synth.decode_inputs_device(seed, lens, K, Hq, Hkv, D)
    max_ctx = int(lens.max())
    cos, sin = peagle.rope_table(D, cfg["theta"], max_ctx + K - 1)
    vt = peagle.decode_pack_v(inp["cu_ctx"], max_ctx, inp["v_cache"])
    del inp["v_cache"]
    dev = vt.device
    out = torch.empty((B, K, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, K, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(peagle.decode_workspace_bytes(B, K, Hq, Hkv, D, int(lens.sum()), max_ctx),
                     dtype=torch.uint8, device=dev)

    def call():
        peagle.draft_decode_attn(inp["cu_ctx"], max_ctx, inp["k_cache"], vt, inp["q"], inp["k"],
                                 inp["v"], cos, sin, out, lse, ws)

    for _ in range(warmup):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    total = int(lens.sum())
    cache_bytes = 2 * total * Hkv * D * 2
    io_bytes = B * K * Hq * D * 2 + 2 * B * K * Hkv * D * 2 + B * K * Hq * D * 4 + B * K * Hq * 4
    gbps = (cache_bytes + io_bytes) / (ms * 1e-3) / 1e9
    del inp, vt, out, lse, ws
    torch.cuda.empty_cache()
    from token_drafting_amd import profiling
    rec = profiling.recorded_decode_traffic(
        os.path.join(os.path.dirname(os.path.abspath(__file__)), DECODE_TRAFFIC_RECORD),
        cfg["workload"])
    return {"workload": cfg["workload"], "requests": B, "context_tokens": total, "K": K,
            "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "ms_per_call": round(ms, 4),
            "bytes_per_call": cache_bytes + io_bytes, "hbm_GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "drafted_tokens_per_s": round(B * K / (ms * 1e-3), 1),
            "roofline": {"kernel": "whole peagle_draft_decode_attn call (prep, split-KV "
                                   "attention, combine)",
                         "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                         "traffic": None if rec is None else int(round(rec["call_bytes"]))}}


def decode_loop_bench(name, steps, warmup):
    """Time one iteration of the decode loop on an inference workload over a cache that
    grows in place: decode attention of the K new rows over the current lengths,
    verification of [B, K, 32000] draft/target logits, and the append of accept_len + 1
    rows per request (keys rotated at their positions, values into their V tiles). Each
    request's capacity is its context plus room for every timed iteration; inputs drawn on
    the device with torch's seeded generator."""
    import torch
    from token_drafting_amd import peagle, synth

    cfg = synth.DECODE_CONFIGS[name]
    B, K, Hq, Hkv, D = cfg["B"], cfg["K"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    lens0 = synth.decode_lengths(31, B, cfg["ctx_lo"], cfg["ctx_hi"])
    cap = lens0 + (K + 1) * (steps + warmup + 1)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(cap)]).astype(np.int32)).cuda()
    total, max_cap = int(cap.sum()), int(cap.max())
    g = torch.Generator(device="cuda")
    g.manual_seed(43)

    def bf16(shape):
        return torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    kc, v_full = bf16((total, Hkv, D)), bf16((total, Hkv, D))
    lens = [torch.from_numpy(lens0.astype(np.int32)).cuda(), torch.empty(B, dtype=torch.int32, device="cuda")]
    vt = peagle.decode_pack_v_lens(cu, lens[0], max_cap, v_full)
    del v_full
    q, k, v = bf16((B, K, Hq, D)), bf16((B, K, Hkv, D)), bf16((B, K, Hkv, D))
    dl, tl = bf16((B, K, 32000)), bf16((B, K, 32000))
    k_app, v_app = bf16((B, K + 1, Hkv, D)), bf16((B, K + 1, Hkv, D))
    cos, sin = peagle.rope_table(D, cfg["theta"], max_cap + K - 1)
    out = torch.empty((B, K, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, K, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(peagle.decode_workspace_bytes(B, K, Hq, Hkv, D, total, max_cap),
                     dtype=torch.uint8, device="cuda")
    dtok = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ttok, alen = torch.empty_like(dtok), torch.empty(B, dtype=torch.int32, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def iteration(i, e=None):
        src, dst = lens[i % 2], lens[(i + 1) % 2]
        if e is not None:
            e[0].record()
        peagle.draft_decode_attn_lens(cu, src, max_cap, kc, vt, q, k, v, cos, sin, out, lse, ws)
        if e is not None:
            e[1].record()
        peagle.accept_prefix(dl, tl, dtok, ttok, alen)
        if e is not None:
            e[2].record()
        peagle.decode_append(cu, src, alen, 1, max_cap, k_app, v_app, cos, sin, kc, vt, dst)
        if e is not None:
            e[3].record()

    for i in range(warmup):
        iteration(i)
    torch.cuda.synchronize()
    for i in range(steps):
        iteration(warmup + i, ev[i])
    torch.cuda.synchronize()
    part = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(3)] for i in range(steps)])
    grown = int((lens[(warmup + steps) % 2].cpu().numpy() - lens0).sum())
    del kc, vt, ws, dl, tl
    torch.cuda.empty_cache()
    m = part.mean(axis=0)
    return {"workload": cfg["workload"], "ms_per_iteration": round(float(m.sum()), 4),
            "decode_attn_ms": round(float(m[0]), 4), "verify_ms": round(float(m[1]), 4),
            "append_ms": round(float(m[2]), 4), "context_tokens_added": grown}


def cpu_baseline(cfg, seed, qkv, cu, idx, depth_off, rows_wanted):
    """The float64 oracle's draft attention on a seeded sample of query rows of the same
    workload (dense mask over all key rows, as the oracle always computes it)."""
    from threadpoolctl import threadpool_info
    from oracle import attention as oattn

    T = int(depth_off[-1])
    if rows_wanted <= 0:
        # the dense oracle costs ~Hq * T * D per query row; 6144 rows of the 32K, K=4,
        # D=256 workload (4 * 83001 * 256 per row) take about 11 s on 16 host threads
        rows_wanted = int(round(6144 * (4 * 83001 * 256) / (cfg["Hq"] * T * cfg["D"])))
        rows_wanted = max(64, rows_wanted)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(T, size=min(rows_wanted, T), replace=False))
    _, keys = useful_pairs(idx, depth_off, cu)
    flop = 4.0 * cfg["D"] * cfg["Hq"] * float(keys[rows].sum())
    t0 = time.perf_counter()
    oattn.draft_attention(qkv["q"], qkv["k"], qkv["v"], idx, depth_off, cu, cfg["theta"], rows=rows)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"oracle draft attention (float64, dense mask) on {len(rows)} seeded random "
                      f"query rows of {T}, all heads; {dt:.1f} s"}


if __name__ == "__main__":
    main()
