"""HBM traffic of the draft-attention core from rocprofv3 byte counters.

Two counter runs of the headline bench (``FETCH_SIZE``, then ``WRITE_SIZE``, each in
KiB per dispatch) are scaled by what the same counters read for a plain device copy of
known size that bench.py performs first (``--calibration-copy-mib``): the copy moves
exactly that many bytes each way, so ``bytes / counter`` is the correction factor of each
counter. The record also stores a digest of the kernel's source files; bench.py reports
the traffic only while the sources still match, since a changed kernel moves different
bytes.

    python -m token_drafting_amd.profiling --fetch <runs>/pmc_fetch \\
        --write <runs>/pmc_write --copy-mib 1024 --out profiles/<name>.md --command "..."
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ("csrc/attn.hip", "csrc/common.h", "csrc/kernels.h")
DECODE_SOURCES = ("csrc/decode.hip", "csrc/common.h", "csrc/kernels.h")
# the launches of one core call: main (or work list, split and merge) and exact kernels
CORE_KERNELS = ("attn_core_kernel", "attn_items_kernel", "attn_combine_kernel")
RECORD_TAG = "traffic_record:"
DECODE_TAG = "decode_traffic_record:"


def kernel_source_digest(sources=ATTN_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("peagle::", "")
    return re.sub(r"\(.*", "", name)


def _read(folder: str, counter: str):
    """[(dispatch id, kernel name, grid size, KiB)] of one counter run."""
    out = []
    for root, _, files in os.walk(folder):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        if r["Counter_Name"] == counter:
                            out.append((int(r["Dispatch_Id"]), _short(r["Kernel_Name"]),
                                        int(r["Grid_Size"]), float(r["Counter_Value"])))
    if not out:
        raise SystemExit(f"no {counter} rows under {folder}")
    return sorted(out)


def _read_all(folder: str):
    """{dispatch id: {"name", "dur_ns", counter: value}} of one counter run."""
    out = {}
    for root, _, files in os.walk(folder):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        d = out.setdefault(int(r["Dispatch_Id"]), {
                            "name": _short(r["Kernel_Name"]),
                            "dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                        d[r["Counter_Name"]] = float(r["Counter_Value"])
    if not out:
        raise SystemExit(f"no counter rows under {folder}")
    return out


def _calibration(rows, copy_bytes: int, counter: str) -> float:
    """bytes per counter KiB, from the largest plain-copy dispatch of the run."""
    copies = [r for r in rows if "copyBuffer" in r[1]]
    if not copies:
        raise SystemExit(f"{counter}: no copy dispatch found for calibration")
    kib = max(copies, key=lambda r: r[3])[3]
    return copy_bytes / kib


def _is_main_core(name: str) -> bool:
    """attn_core_kernel<D, role> with role 0 (one launch for the whole call) or 1 (the split
    path's segments): one such dispatch per core call."""
    m = re.match(r"attn_core_kernel<\s*\d+\s*,\s*(\w+)", name)
    return bool(m) and m.group(1) in ("0", "1")


def summarize(fetch_dir: str, write_dir: str, copy_mib: int) -> dict:
    copy_bytes = copy_mib << 20
    fetch, write = _read(fetch_dir, "FETCH_SIZE"), _read(write_dir, "WRITE_SIZE")
    f_fac = _calibration(fetch, copy_bytes, "FETCH_SIZE")
    w_fac = _calibration(write, copy_bytes, "WRITE_SIZE")
    per_kernel = {}
    for rows, key, fac in ((fetch, "fetch", f_fac), (write, "write", w_fac)):
        acc = defaultdict(list)
        for _, name, _, kib in rows:
            if "copyBuffer" in name or name.startswith("at::"):
                continue
            acc[name].append(kib)
        for name, v in acc.items():
            d = per_kernel.setdefault(name, {"calls": len(v)})
            d[key + "_kib_raw"] = sum(v) / len(v)
            d[key + "_bytes"] = sum(v) / len(v) * fac
    core = {name: d for name, d in per_kernel.items() if any(k in name for k in CORE_KERNELS)}
    # one role-0 or role-1 dispatch per core call; a split call adds the work list, merge and
    # redo launches, so a call's bytes are each kernel's total over the calls
    n_calls = max(1, sum(d["calls"] for name, d in core.items() if _is_main_core(name)))

    def per_call(key):
        return sum(d.get(key, 0.0) * d["calls"] for d in core.values()) / n_calls

    rec = {
        "kernel_source_sha256": kernel_source_digest(),
        "fetch_factor_bytes_per_kib": f_fac,
        "write_factor_bytes_per_kib": w_fac,
        "core_call_fetch_bytes": per_call("fetch_bytes"),
        "core_call_write_bytes": per_call("write_bytes"),
    }
    rec["core_call_bytes"] = rec["core_call_fetch_bytes"] + rec["core_call_write_bytes"]
    return {"record": rec, "per_kernel": per_kernel,
            "decode": _decode_traffic(fetch, write, f_fac, w_fac)}


def _workload_runs(calls, n: int):
    """The first n runs of consecutive calls with the same attention kernel (element 0 of
    each call). bench.py times the plain decode call of each inference workload in sorted
    name order, then the decode loop's calls; the workloads use different attention
    kernels, so run i holds workload i's plain calls."""
    runs = []
    for c in calls:
        if runs and runs[-1][0][0] == c[0]:
            runs[-1].append(c)
        else:
            runs.append([c])
    return runs[:n]


def _decode_traffic(fetch, write, f_fac: float, w_fac: float):
    """Per-call bytes of the decode attention (prep, attention and combine launches) for
    each inference workload, or None when the runs hold no decode calls."""
    from . import synth

    def calls(rows, fac):
        seq = [(name, kib * fac) for _, name, _, kib in rows
               if any(k in name for k in ("decode_prep_kernel", "decode_attn_kernel",
                                          "decode_combine_kernel"))]
        out = []
        for i in range(0, len(seq) - 2, 3):
            (a, x), (b, y), (c, z) = seq[i:i + 3]
            if "prep" in a and "attn" in b and "combine" in c:
                out.append((b, x + y + z))
        return out

    names = sorted(synth.DECODE_CONFIGS)
    rf, rw = _workload_runs(calls(fetch, f_fac), len(names)), _workload_runs(calls(write, w_fac), len(names))
    if len(rf) != len(names) or [len(r) for r in rf] != [len(r) for r in rw]:
        return None
    rec = {"kernel_source_sha256": kernel_source_digest(DECODE_SOURCES), "workloads": {}}
    for name, runf, runw in zip(names, rf, rw):
        f, w, per = [b for _, b in runf], [b for _, b in runw], len(runf)
        rec["workloads"][synth.DECODE_CONFIGS[name]["workload"]] = {
            "attn_kernel": runf[0][0], "calls": per,
            "call_fetch_bytes": sum(f) / per, "call_write_bytes": sum(w) / per,
            "call_bytes": (sum(f) + sum(w)) / per}
    return rec


def write_decode_summary(path: str, rec: dict, command: str) -> None:
    lines = ["# HBM traffic per call: decode-shaped draft attention, inference workloads", "",
             "Counter runs (each its own process):", "", "```", command, "```", "",
             "Bytes of one peagle_draft_decode_attn call (prep, split-KV attention and combine "
             "launches), FETCH_SIZE and WRITE_SIZE scaled by the plain copy of known size in "
             "the same runs.", "",
             "| workload | attention kernel | calls | read MB | written MB |", "|---|---|---|---|---|"]
    for name, d in rec["workloads"].items():
        lines.append(f"| {name} | `{d['attn_kernel']}` | {d['calls']} | "
                     f"{d['call_fetch_bytes'] / 1e6:.2f} | {d['call_write_bytes'] / 1e6:.2f} |")
    lines += ["", f"{DECODE_TAG} {json.dumps(rec)}", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def recorded_decode_traffic(path: str, workload: str):
    """Bytes per call of one decode workload from the stored record, if it was taken on the
    current decode sources, else None."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(DECODE_TAG):
                    rec = json.loads(line[len(DECODE_TAG):])
                    if rec.get("kernel_source_sha256") != kernel_source_digest(DECODE_SOURCES):
                        return None
                    return rec["workloads"].get(workload)
    except OSError:
        return None
    return None


def write_summary(path: str, summary: dict, command: str) -> None:
    rec = summary["record"]
    lines = [
        "# HBM traffic per dispatch: draft-attention workload gemma270m-draft-32k-K4",
        "",
        "Counter runs (each its own process):",
        "",
        "```",
        command,
        "```",
        "",
        f"Calibration: a plain device copy of known size inside the same run reads "
        f"{rec['fetch_factor_bytes_per_kib']:.2f} bytes per FETCH_SIZE KiB and writes "
        f"{rec['write_factor_bytes_per_kib']:.2f} bytes per WRITE_SIZE KiB.",
        "",
        "| kernel | calls | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | read MB | written MB |",
        "|---|---|---|---|---|---|",
    ]
    for name, d in sorted(summary["per_kernel"].items()):
        lines.append(f"| `{name}` | {d['calls']} | {d.get('fetch_kib_raw', 0):.1f} | "
                     f"{d.get('write_kib_raw', 0):.1f} | {d.get('fetch_bytes', 0) / 1e6:.2f} | "
                     f"{d.get('write_bytes', 0) / 1e6:.2f} |")
    lines += ["", f"Attention core call (all its launches): "
              f"{rec['core_call_fetch_bytes'] / 1e6:.1f} MB read + "
              f"{rec['core_call_write_bytes'] / 1e6:.1f} MB written.", "",
              f"{RECORD_TAG} {json.dumps(rec)}", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


SIMDS = 256 * 4  # MI355X: 256 CUs x 4 SIMDs
XCDS = 8
MFMA_BF16_FLOP_PER_MOP = 512  # SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512-FLOP units
MAX_ENGINE_GHZ = 2.4  # MI355X peak engine clock
# runtime and torch kernels of a bench run (copies, fills, torch's random draws and scans)
FOREIGN_KERNELS = ("copyBuffer", "fillBuffer", "rocprim::", "elementwise_kernel", "at::native")


def kernel_table(mfma_dir: str, fetch_dir: str, write_dir: str, copy_mib: int) -> list:
    """Per kernel: duration, bf16 MFMA FLOP/s, MFMA-busy share of the SIMD cycles, shader
    clock seen by the dispatch, and calibrated HBM bytes and GB/s."""
    copy_bytes = copy_mib << 20
    fetch, write = _read_all(fetch_dir), _read_all(write_dir)
    f_fac = _calibration([(k, v["name"], 0, v["FETCH_SIZE"]) for k, v in fetch.items()],
                         copy_bytes, "FETCH_SIZE")
    w_fac = _calibration([(k, v["name"], 0, v["WRITE_SIZE"]) for k, v in write.items()],
                         copy_bytes, "WRITE_SIZE")
    acc = defaultdict(lambda: defaultdict(list))
    for v in _read_all(mfma_dir).values():
        a = acc[v["name"]]
        a["dur"].append(v["dur_ns"])
        a["mops"].append(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
        a["busy"].append(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0))
        a["gui"].append(v.get("GRBM_GUI_ACTIVE", 0.0))
    for run, key, fac, ctr in ((fetch, "rd", f_fac, "FETCH_SIZE"), (write, "wr", w_fac, "WRITE_SIZE")):
        for v in run.values():
            acc[v["name"]][key].append(v[ctr] * fac)
            acc[v["name"]][key + "_dur"].append(v["dur_ns"])
    rows = []
    for name, a in acc.items():
        if not a["dur"] or any(x in name for x in FOREIGN_KERNELS) or name.startswith("at::"):
            continue
        mean = lambda x: sum(x) / len(x) if x else 0.0
        dur = mean(a["dur"]) * 1e-9
        gui = mean(a["gui"]) / XCDS
        rd, wr = mean(a["rd"]), mean(a["wr"])
        io_dur = mean(a["rd_dur"] + a["wr_dur"]) * 1e-9
        rows.append({
            "kernel": name, "calls": len(a["dur"]), "us": dur * 1e6,
            "bf16_tflops": mean(a["mops"]) * MFMA_BF16_FLOP_PER_MOP / dur / 1e12 if dur else 0.0,
            "mfma_busy": mean(a["busy"]) / (SIMDS * gui) if gui else 0.0,
            "clock_ghz": gui / dur / 1e9 if dur else 0.0,
            "read_mb": rd / 1e6, "write_mb": wr / 1e6,
            "hbm_gbps": (rd + wr) / io_dur / 1e9 if io_dur else 0.0,
        })
    return sorted(rows, key=lambda r: -r["us"])


def write_kernel_table(path: str, rows: list, title: str, command: str) -> None:
    lines = [f"# {title}", "", "Counter runs (each its own process):", "", "```", command, "```", "",
             "Columns: dispatch duration in the MFMA-counter run; bf16 TFLOP/s = "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration; MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); clock = "
             "GRBM_GUI_ACTIVE / 8 / duration; HBM bytes = FETCH_SIZE and WRITE_SIZE scaled by "
             "the plain copy of known size in the same runs; GB/s = those bytes over the "
             "byte runs' own dispatch durations.", "",
             "| kernel | calls | us | bf16 TFLOP/s | MFMA busy | clock GHz | read MB | written MB | HBM GB/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        # a derived clock above the engine's maximum means the counter window was wider than
        # the dispatch: its MFMA-busy denominator is then inflated, so the share is withheld
        ok = r["clock_ghz"] <= MAX_ENGINE_GHZ
        busy = f"{100 * r['mfma_busy']:.1f}%" if ok else "n/a"
        clock = f"{r['clock_ghz']:.2f}" if ok else f"({r['clock_ghz']:.2f}, window > dispatch)"
        lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['us']:.1f} | {r['bf16_tflops']:.1f} | "
                     f"{busy} | {clock} | {r['read_mb']:.2f} | "
                     f"{r['write_mb']:.2f} | {r['hbm_gbps']:.0f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


DECODE_KERNELS = ("decode_prep_kernel", "decode_attn_kernel", "decode_combine_kernel")


def _decode_calls(rows, n_calls: int):
    """Per-call durations (first launch start to last launch end, ns) of the decode
    attention calls in launch order: prep, attention, combine per call."""
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"]))
                 for r in rows if any(k in r["Kernel_Name"] for k in DECODE_KERNELS))
    calls = []
    for i in range(0, len(seq) - 2, 3):
        a, b, c = seq[i], seq[i + 1], seq[i + 2]
        if "prep" in a[2] and "attn" in b[2] and "combine" in c[2]:
            calls.append((c[1] - a[0], b[1] - b[0], b[2]))
    return calls


def write_trace_summary(path: str, trace_dir: str, bench_log: str, title: str, command: str,
                        timed: int) -> None:
    """Kernel-trace summary of the library's kernels: per-kernel durations from rocprofv3's
    kernel trace, and the agreement of the last `timed` calls with bench.py's live timing
    (attention core of the forward; each decode workload's whole call)."""
    rows = []
    for root, _, files in os.walk(trace_dir):
        for fn in files:
            if fn.endswith("kernel_trace.csv"):
                with open(os.path.join(root, fn)) as f:
                    rows += list(csv.DictReader(f))
    rows = [r for r in rows if "peagle::" in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no library kernels in the trace under {trace_dir}")
    per = defaultdict(list)
    for r in rows:
        per[_short(r["Kernel_Name"])].append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    total = sum(d for v in per.values() for _, d in v)
    lines = [f"# {title}", "", "Command (from the repository root):", "", "    " + command, "",
             "Durations in microseconds from the kernel trace (all calls, warm-up included); "
             "library kernels only (the run's input generation and calibration copy are left "
             "out).", "",
             "| kernel | calls | avg us | min us | max us | % of library GPU time |",
             "|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = [x for _, x in v]
        lines.append(f"| `{name}` | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | {min(d) / 1e3:.1f} | "
                     f"{max(d) / 1e3:.1f} | {100 * sum(d) / total:.2f} |")
    core = [k for k in per if any(c in k for c in CORE_KERNELS)]
    # A core call's launches sit between the step's other kernels in start order; a call
    # lasts from its first launch's start to its last launch's end (were any two of its
    # launches to overlap, the span still counts the time once).
    seq = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short(r["Kernel_Name"]))
                 for r in rows)
    spans, cur = [], None
    for st, en, name in seq:
        if any(c in name for c in CORE_KERNELS):
            cur = [st, en] if cur is None else [cur[0], max(cur[1], en)]
        elif cur is not None:
            spans.append(cur)
            cur = None
    if cur is not None:
        spans.append(cur)
    mine = spans[-timed:]
    last = sum(en - st for st, en in mine) / max(1, len(mine)) / 1e3
    live, dec_live = None, {}
    with open(bench_log) as f:
        for line in f:
            if line.startswith("{"):
                j = json.loads(line)
                live = j["stage_ms"]["attn_core"] * 1e3 if "stage_ms" in j else None
                dec_live = j.get("decode", {})
    lines += ["", f"Agreement with the live timing: over the last {timed} calls the attention core "
              f"launches ({', '.join('`' + k + '`' for k in sorted(core))}) span {last:.1f} us "
              f"per call in the trace (first start to last end); bench.py's HIP events on the "
              f"launch stream measured {live:.1f} us per call in the same run."
              if live is not None else ""]
    calls = _decode_calls(rows, timed)
    if dec_live and calls:
        # calls are (duration, attention duration, attention kernel): key the runs on the kernel
        runs = _workload_runs([(c[2], c) for c in calls], len(dec_live))
        for (name, res), run in zip(sorted(dec_live.items()), runs):
            mine = [c for _, c in run][-timed:]
            call_us = sum(c[0] for c in mine) / len(mine) / 1e3
            attn_us = sum(c[1] for c in mine) / len(mine) / 1e3
            lines.append(
                f"Decode workload {res['workload']}: over its last {len(mine)} calls the trace "
                f"gives {call_us:.1f} us per call (prep start to combine end; `{mine[0][2]}` "
                f"{attn_us:.1f} us of it); bench.py measured {res['ms_per_call'] * 1e3:.1f} us "
                f"per call.")
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))


def recorded_traffic(path: str):
    """The stored record if it was taken on the current kernel sources, else None."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(RECORD_TAG):
                    rec = json.loads(line[len(RECORD_TAG):])
                    if rec.get("kernel_source_sha256") == kernel_source_digest():
                        return rec
                    return None
    except OSError:
        return None
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--fetch", help="rocprofv3 output folder of the FETCH_SIZE run")
    ap.add_argument("--write", help="rocprofv3 output folder of the WRITE_SIZE run")
    ap.add_argument("--trace", help="rocprofv3 kernel-trace folder; with --bench-log, write the "
                    "kernel-trace summary")
    ap.add_argument("--bench-log", help="stdout of the traced bench.py run")
    ap.add_argument("--timed", type=int, default=5, help="timed steps of the traced run")
    ap.add_argument("--mfma", help="rocprofv3 output folder of the MFMA counter run; with it, "
                    "write the per-kernel table instead of the traffic record")
    ap.add_argument("--copy-mib", type=int, default=0, help="calibration copy size of the runs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--decode-out", help="with --fetch/--write: also write the decode "
                    "attention's per-call traffic record here")
    ap.add_argument("--title", default="Per-kernel counters")
    ap.add_argument("--command", required=True, help="the counter commands, for the record")
    a = ap.parse_args()
    if a.trace:
        write_trace_summary(a.out, a.trace, a.bench_log, a.title, a.command, a.timed)
        return
    if not (a.fetch and a.write and a.copy_mib):
        raise SystemExit("--fetch, --write and --copy-mib are required for counter summaries")
    if a.mfma:
        rows = kernel_table(a.mfma, a.fetch, a.write, a.copy_mib)
        write_kernel_table(a.out, rows, a.title, a.command)
        print(json.dumps(rows[:3]))
        return
    s = summarize(a.fetch, a.write, a.copy_mib)
    write_summary(a.out, s, a.command)
    print(json.dumps(s["record"]))
    if a.decode_out and s["decode"]:
        write_decode_summary(a.decode_out, s["decode"], a.command)
        print(json.dumps(s["decode"]))


if __name__ == "__main__":
    main()
