"""HBM traffic of the draft-attention core from rocprofv3 byte counters.

Two counter runs of the headline bench (``FETCH_SIZE``, then ``WRITE_SIZE``, each in
KiB per dispatch) are scaled by what the same counters read for a plain device copy of
known size that bench.py performs first (``--calibration-copy-mib``): the copy moves
exactly that many bytes each way, so ``bytes / counter`` is the correction factor of each
counter. The record also stores a digest of the kernel's source files; bench.py reports
the traffic only while the sources still match, since a changed kernel moves different
bytes.

    python -m token_drafting_amd.profiling --fetch gpurun_out/pmc_fetch \\
        --write gpurun_out/pmc_write --copy-mib 1024 --out profiles/<name>.md --command "..."
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
CORE_KERNELS = ("attn_core_kernel",)  # both launches (main and exact) of one core call
RECORD_TAG = "traffic_record:"


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
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


def _calibration(rows, copy_bytes: int, counter: str) -> float:
    """bytes per counter KiB, from the largest plain-copy dispatch of the run."""
    copies = [r for r in rows if "copyBuffer" in r[1]]
    if not copies:
        raise SystemExit(f"{counter}: no copy dispatch found for calibration")
    kib = max(copies, key=lambda r: r[3])[3]
    return copy_bytes / kib


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
    core = [d for name, d in per_kernel.items() if any(k in name for k in CORE_KERNELS)]
    rec = {
        "kernel_source_sha256": kernel_source_digest(),
        "fetch_factor_bytes_per_kib": f_fac,
        "write_factor_bytes_per_kib": w_fac,
        "core_call_fetch_bytes": sum(d.get("fetch_bytes", 0.0) for d in core),
        "core_call_write_bytes": sum(d.get("write_bytes", 0.0) for d in core),
    }
    rec["core_call_bytes"] = rec["core_call_fetch_bytes"] + rec["core_call_write_bytes"]
    return {"record": rec, "per_kernel": per_kernel}


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
    lines += ["", f"Attention core call (both launches): "
              f"{rec['core_call_fetch_bytes'] / 1e6:.1f} MB read + "
              f"{rec['core_call_write_bytes'] / 1e6:.1f} MB written.", "",
              f"{RECORD_TAG} {json.dumps(rec)}", ""]
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
    ap.add_argument("--fetch", required=True, help="rocprofv3 output folder of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="rocprofv3 output folder of the WRITE_SIZE run")
    ap.add_argument("--copy-mib", type=int, required=True, help="calibration copy size of the runs")
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", required=True, help="the counter commands, for the record")
    a = ap.parse_args()
    s = summarize(a.fetch, a.write, a.copy_mib)
    write_summary(a.out, s, a.command)
    print(json.dumps(s["record"]))


if __name__ == "__main__":
    main()
