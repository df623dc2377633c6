"""Host logic of the rocprofv3 summaries bench.py relies on (no GPU needed).

The traffic record must scale each byte counter by the calibration copy found in the same
run, sum both attention-core launches, and be reported only while the attention sources
it was taken on are unchanged.
"""
import csv
import json
import os

from token_drafting_amd import profiling

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_run(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({k: 0 for k in FIELDS} | {
                "Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 1024,
                "Counter_Name": counter, "Counter_Value": value,
                "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + 500})


def test_traffic_record_scales_by_the_copy_and_sums_core_launches(tmp_path):
    main = "void peagle::(anonymous namespace)::attn_core_kernel<256, 0>(peagle::AttnParams)"
    exact = "void peagle::(anonymous namespace)::attn_items_kernel(peagle::AttnParams)"
    # the 1 MiB copy reads as 512 KiB (128-byte requests counted as 64) and writes 1024 KiB
    _write_run(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512.0), (main, 100.0),
                                              (exact, 10.0), ("other_kernel", 7.0)])
    _write_run(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1024.0), (main, 50.0),
                                              (exact, 5.0), ("other_kernel", 3.0)])
    s = profiling.summarize(str(tmp_path / "f"), str(tmp_path / "w"), copy_mib=1)
    rec = s["record"]
    assert rec["fetch_factor_bytes_per_kib"] == 2048.0
    assert rec["write_factor_bytes_per_kib"] == 1024.0
    assert rec["core_call_fetch_bytes"] == (100.0 + 10.0) * 2048.0
    assert rec["core_call_write_bytes"] == (50.0 + 5.0) * 1024.0
    assert rec["core_call_bytes"] == rec["core_call_fetch_bytes"] + rec["core_call_write_bytes"]
    assert rec["kernel_source_sha256"] == profiling.kernel_source_digest()


def test_recorded_traffic_is_withheld_when_sources_differ(tmp_path):
    good = {"kernel_source_sha256": profiling.kernel_source_digest(), "core_call_bytes": 123.0}
    stale = dict(good, kernel_source_sha256="0" * 64)
    p_good, p_stale = tmp_path / "good.md", tmp_path / "stale.md"
    p_good.write_text("# summary\n\n" + profiling.RECORD_TAG + " " + json.dumps(good) + "\n")
    p_stale.write_text(profiling.RECORD_TAG + " " + json.dumps(stale) + "\n")
    assert profiling.recorded_traffic(str(p_good))["core_call_bytes"] == 123.0
    assert profiling.recorded_traffic(str(p_stale)) is None
    assert profiling.recorded_traffic(str(tmp_path / "missing.md")) is None


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_decode_traffic_groups_calls_per_workload(tmp_path):
    """Decode calls are (prep, attention, combine) triples in launch order; bench.py times
    the workloads in sorted name order, the same number of calls each."""
    from token_drafting_amd import synth
    names = sorted(synth.DECODE_CONFIGS)
    prep = "peagle::(anonymous namespace)::decode_prep_kernel(int const*)"
    comb = "peagle::(anonymous namespace)::decode_combine_kernel(int const*)"
    attn = ["void peagle::(anonymous namespace)::decode_attn_kernel<256, 1, 1>(peagle::P)",
            "void peagle::(anonymous namespace)::decode_attn_kernel<128, 2, 4>(peagle::P)"]
    f_rows, w_rows = [("__amd_rocclr_copyBuffer", 512.0)], [("__amd_rocclr_copyBuffer", 1024.0)]
    for i in range(len(names)):
        for _ in range(2):                       # two calls per workload
            f_rows += [(prep, 1.0), (attn[i], 100.0 * (i + 1)), (comb, 2.0)]
            w_rows += [(prep, 1.0), (attn[i], 10.0 * (i + 1)), (comb, 1.0)]
    _write_run(tmp_path / "f", "FETCH_SIZE", f_rows)
    _write_run(tmp_path / "w", "WRITE_SIZE", w_rows)
    s = profiling.summarize(str(tmp_path / "f"), str(tmp_path / "w"), copy_mib=1)
    rec = s["decode"]
    assert rec["kernel_source_sha256"] == profiling.kernel_source_digest(profiling.DECODE_SOURCES)
    for i, name in enumerate(names):
        d = rec["workloads"][synth.DECODE_CONFIGS[name]["workload"]]
        assert d["calls"] == 2
        assert d["call_fetch_bytes"] == (1.0 + 100.0 * (i + 1) + 2.0) * 2048.0
        assert d["call_write_bytes"] == (1.0 + 10.0 * (i + 1) + 1.0) * 1024.0
    path = tmp_path / "dec.md"
    profiling.write_decode_summary(str(path), rec, "cmd")
    wl = synth.DECODE_CONFIGS[names[0]]["workload"]
    assert profiling.recorded_decode_traffic(str(path), wl)["calls"] == 2
    stale = dict(rec, kernel_source_sha256="0" * 64)
    profiling.write_decode_summary(str(path), stale, "cmd")
    assert profiling.recorded_decode_traffic(str(path), wl) is None


def test_decode_calls_grouped_by_workload_runs():
    """Plain decode calls of each workload come first (sorted names, different attention
    kernels), then the decode loop's: each workload's record takes its own first run."""
    from token_drafting_amd.profiling import _workload_runs
    seq = [("k256", 1), ("k256", 2), ("k128", 3), ("k128", 4), ("k256", 5), ("k128", 6)]
    runs = _workload_runs(seq, 2)
    assert [[x for _, x in r] for r in runs] == [[1, 2], [3, 4]]
    assert _workload_runs(seq[:2], 2) == [seq[:2]]


def test_core_call_bytes_take_each_kernel_total_per_call(tmp_path):
    # two split core calls: work list, segments (role 1), merge and redo (role 2) each; a
    # call's bytes are each kernel's total over the calls
    main = "void peagle::attn_core_kernel<256, 1>(peagle::AttnParams)"
    items = "void peagle::attn_items_kernel(peagle::AttnParams)"
    redo = "void peagle::attn_core_kernel<256, 2>(peagle::AttnParams)"
    rows = [("__amd_rocclr_copyBuffer", 512.0), (items, 10.0), (main, 100.0), (redo, 2.0),
            (items, 10.0), (main, 100.0), (redo, 2.0)]
    _write_run(tmp_path / "f", "FETCH_SIZE", rows)
    _write_run(tmp_path / "w", "WRITE_SIZE", [(n, 2 * v if "copy" in n else v) for n, v in rows])
    rec = profiling.summarize(str(tmp_path / "f"), str(tmp_path / "w"), copy_mib=1)["record"]
    kib_per_call = 100.0 + 10.0 + 2.0
    assert abs(rec["core_call_fetch_bytes"] - kib_per_call * 2048.0) < 1e-6
    assert abs(rec["core_call_write_bytes"] - kib_per_call * 1024.0) < 1e-6


def test_trace_agreement_takes_each_core_call_wall_span(tmp_path):
    # a call lasts from its first launch's start to its last launch's end: overlapping
    # launches count once, not as the sum of their durations
    trace = tmp_path / "trace"
    os.makedirs(trace)
    names = {"main": "void peagle::attn_core_kernel<256, 1>(peagle::AttnParams)",
             "short": "void peagle::attn_core_kernel<256, 2>(peagle::AttnParams)",
             "prep": "void peagle::rope_rotate_kernel<unsigned int>(int)",
             "acc": "void peagle::accept_kernel<unsigned int, false>(int)"}
    launches = []
    t = 0
    for _ in range(3):   # prep, then main [t+10, t+1010] beside short [t+20, t+520], redo, accept
        launches += [("prep", t, t + 5), ("short", t + 20, t + 520), ("main", t + 10, t + 1010),
                     ("short", t + 1012, t + 1016), ("acc", t + 1020, t + 1100)]
        t += 2000
    with open(trace / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for k, st, en in launches:
            w.writerow({"Kernel_Name": names[k], "Start_Timestamp": st * 1000,
                        "End_Timestamp": en * 1000})
    log = tmp_path / "bench.log"
    log.write_text(json.dumps({"stage_ms": {"attn_core": 1.006}}) + "\n")
    out = tmp_path / "summary.md"
    profiling.write_trace_summary(str(out), str(trace), str(log), "t", "cmd", timed=2)
    text = out.read_text()
    assert "span 1006.0 us per call" in text   # 10 .. 1016, not 1000 + 500 + 4
    assert "measured 1006.0 us" in text
