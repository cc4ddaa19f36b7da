"""Turn rocprofv3 CSV output into the short summaries kept under ``profiles/``.

Two inputs are read:

* ``--kernel-trace --stats`` output (``*_kernel_stats.csv``): per-kernel call
  count and average duration.
* two ``--pmc`` runs of the same command, one with ``FETCH_SIZE`` and one with
  ``WRITE_SIZE`` (``*_counter_collection.csv``, KiB per dispatch). The raw
  counters are scaled by what they read for a plain device copy of known size
  in the same run (the benchmark's 2 GiB ``copy_`` ceiling shows up as the
  runtime's ``copyBuffer`` kernel), so the reported bytes are HBM bytes.

Usage::

    python -m paged_kv_cache_260_amd.profiling --name NAME --command "CMD" \\
        --stats STATS.csv --fetch FETCH.csv --write WRITE.csv \\
        --fetch-command "CMD1" --write-command "CMD2" \\
        --algorithmic-bytes N --copy-bytes 2147483648 --out DIR

writes ``DIR/NAME_kernel_stats.md``, ``DIR/NAME_traffic.md`` and
``DIR/NAME_traffic.json`` (the last one is read by ``bench.py``, which reports
the traffic only while the decode source still has the recorded hash).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
# sources that define the decode kernel's code
DECODE_SRCS = tuple(os.path.join(PKG, "csrc", f) for f in ("decode.hip", "attn_common.h", "kernels.h"))
DECODE_KERNEL = "paged_decode_kernel"
MERGE_KERNEL = "paged_decode_reduce_kernel"
MERGE_FEW_KERNEL = "paged_decode_merge_few_kernel"
COPY_KERNEL = "copyBuffer"
# kernels of one paged_attn_decode call (the merge kernels run only for split
# sequences whose partitions are not merged inside the decode kernel)
CALL_KERNELS = (DECODE_KERNEL, MERGE_KERNEL, MERGE_FEW_KERNEL)


def code_text(src: str) -> str:
    """C++ source without its comments, one token run per line: string and
    character literals are kept as written, every comment is dropped and each
    stretch of whitespace becomes one space, so that edits to comments or
    layout leave it unchanged."""
    out = []
    i, n = 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(paths=DECODE_SRCS) -> str:
    """Hash of the decode kernel's code (comments and layout ignored): the
    traffic summaries record it, and the benchmark reuses their figures only
    while it is unchanged."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


# the decode kernel's last template argument: what its work items' rows are
_DECODE_MODES = {"0": "", "1": " (chunk rows)", "2": " (shared prefix)", "3": " (private tokens)",
                 "4": " (shared prefix, one launch)", "5": " (append)"}


def short_name(name: str) -> str:
    for key in (*CALL_KERNELS, "paged_chunk_reduce_kernel", "paged_chunk_kernel", "kv_cache_write_fp8_kernel",
                "kv_cache_write_kernel",
                "zero_i32_kernel", "copy_blocks_kernel", "stream_read_kernel", "gather_tiles_kernel", COPY_KERNEL):
        if key in name:
            # the mode, then (when present) whether the work order came from the host
            m = re.search(r"ELi(\d)(?:ELb([01]))?EEEvNS_10DecodeArgsE$", name) if key == DECODE_KERNEL else None
            if m:
                label = key + _DECODE_MODES.get(m.group(1), "")
                return label[:-1] + ", host order)" if m.group(2) == "1" and label.endswith(")") else label
            return key
    return name[:60]


def read_stats(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_ns": float(r["AverageNs"]), "pct": float(r["Percentage"]),
                         "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])})
    return rows


def read_counter(path, counter):
    """{kernel short name: [value per dispatch in dispatch order]}."""
    per = defaultdict(list)
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        if r["Counter_Name"] == counter:
            per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def read_trace(path):
    """{kernel short name: [duration ns per dispatch, in dispatch order]}."""
    per = defaultdict(list)
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per


def summarize(name, command, stats_csv, fetch_csv, write_csv, algorithmic_bytes, copy_bytes, out,
              fetch_command=None, write_command=None, trace_csv=None, skip=0, take=0, only=None):
    os.makedirs(out, exist_ok=True)
    stats = read_stats(stats_csv)
    lines = [f"# {name}: rocprofv3 kernel statistics", "", "Command (repository root):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short_name(r['name'])} | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | "
                     f"{r['min_ns'] / 1e3:.2f} | {r['max_ns'] / 1e3:.2f} | {r['pct']:.1f} |")
    timed = {}
    if trace_csv and take > 0:
        # the statistics above average every call, warm-up included (the clocks
        # ramp up during the first tens of milliseconds); the benchmark's figure
        # comes from the calls it times, dispatches [skip, skip + take) of each
        # kernel in the same trace
        trace = read_trace(trace_csv)
        lines += ["", f"Calls the benchmark times (dispatches {skip} to {skip + take - 1} of each kernel, "
                  f"from the kernel trace of the same run):", "",
                  "| kernel | calls | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
        for k, durs in trace.items():
            win = sorted(durs[skip:skip + take])
            if len(win) < take:
                continue
            avg = sum(win) / len(win)
            timed[k] = avg / 1e3
            lines.append(f"| {k} | {len(win)} | {avg / 1e3:.2f} | {win[len(win) // 2] / 1e3:.2f} | "
                         f"{win[0] / 1e3:.2f} | {win[-1] / 1e3:.2f} |")
    with open(os.path.join(out, f"{name}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    result = {"name": name, "decode_source_hash": source_hash(), "command": command,
              "algorithmic_bytes": int(algorithmic_bytes),
              "kernel_avg_us": {short_name(r["name"]): r["avg_ns"] / 1e3 for r in stats}}
    if timed:
        result["timed_calls_avg_us"] = timed
    if fetch_csv and write_csv:
        fetch = read_counter(fetch_csv, "FETCH_SIZE")
        write = read_counter(write_csv, "WRITE_SIZE")
        copy_kib = copy_bytes / 1024.0
        f_scale = copy_kib / max(fetch[COPY_KERNEL]) if fetch.get(COPY_KERNEL) else 1.0
        w_scale = copy_kib / max(write[COPY_KERNEL]) if write.get(COPY_KERNEL) else 1.0

        def avg(d, k):
            v = d.get(k, [])[1:] or d.get(k, [])  # skip the first (cold) dispatch
            return sum(v) / len(v) if v else 0.0

        per_kernel = {}
        # the call's kernels under their labels (the decode kernel carries its mode)
        for k in sorted(fetch):
            if not any(k == c or k.startswith(c + " (") for c in CALL_KERNELS):
                continue
            if only and k not in only:  # a run that times several kinds of call
                continue
            per_kernel[k] = {"fetch_kib_raw": avg(fetch, k), "write_kib_raw": avg(write, k),
                             "fetch_bytes": avg(fetch, k) * f_scale * 1024,
                             "write_bytes": avg(write, k) * w_scale * 1024}
        traffic = sum(v["fetch_bytes"] + v["write_bytes"] for v in per_kernel.values())
        result.update({"fetch_scale": f_scale, "write_scale": w_scale, "per_kernel": per_kernel,
                       "traffic_bytes_per_call": traffic,
                       "traffic_over_algorithmic": traffic / algorithmic_bytes})
        t = [f"# {name}: HBM traffic of one decode call", "",
             "Two rocprofv3 counter runs (repository root), one per counter:", "",
             "```", fetch_command or "(FETCH_SIZE run)", write_command or "(WRITE_SIZE run)", "```", "",
             "Counters are KiB per dispatch. Scale: the",
             f"run's {copy_bytes / 2**30:.0f} GiB device copy ({COPY_KERNEL}) reads "
             f"{max(fetch.get(COPY_KERNEL, [0])):.0f} KiB of FETCH_SIZE and "
             f"{max(write.get(COPY_KERNEL, [0])):.0f} KiB of WRITE_SIZE for {copy_kib:.0f} KiB moved,",
             f"so FETCH_SIZE x {f_scale:.4f} and WRITE_SIZE x {w_scale:.4f} give bytes.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |",
             "|---|---|---|---|---|"]
        for k, v in per_kernel.items():
            t.append(f"| {k} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | "
                     f"{v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} |")
        t += ["", f"Total per call: {traffic / 1e6:.2f} MB against {algorithmic_bytes / 1e6:.2f} MB "
              f"algorithmic (K/V + Q + O, plus the stored new rows for the append call): "
              f"{traffic / algorithmic_bytes:.3f}x.",
              f"Decode source hash: `{result['decode_source_hash']}`."]
        with open(os.path.join(out, f"{name}_traffic.md"), "w") as f:
            f.write("\n".join(t) + "\n")
        with open(os.path.join(out, f"{name}_traffic.json"), "w") as f:
            json.dump(result, f, indent=1)
    return result


# Hardware counters read in the counter passes, with what they count (per
# dispatch, summed over the chip by rocprofv3).
COUNTER_NOTES = {
    "SQ_WAVES": "waves launched",
    "SQ_INSTS_VALU": "vector ALU instructions issued (wave level; MFMA included)",
    "SQ_INSTS_MFMA": "MFMA instructions issued",
    "SQ_INSTS_LDS": "LDS instructions issued",
    "SQ_INSTS_VMEM_RD": "vector memory read instructions",
    "SQ_INSTS_VMEM_WR": "vector memory write instructions",
    "SQ_INSTS_SALU": "scalar ALU instructions",
    "SQ_INSTS_VALU_MFMA_MOPS_BF16": "bf16 MFMA work in units of 512 flops",
    "SQ_INSTS_VALU_MFMA_MOPS_F16": "fp16 MFMA work in units of 512 flops",
    "SQ_WAVE_CYCLES": "wave-cycles resident (summed over waves)",
    "SQ_BUSY_CYCLES": "cycles the sequencers had work",
    "SQ_WAIT_ANY": "wave-cycles waiting for anything",
    "SQ_WAIT_INST_ANY": "wave-cycles waiting for an instruction's dependency (memory data, mostly)",
    "SQ_ACTIVE_INST_VALU": "wave-cycles issuing VALU instructions",
    "SQ_ACTIVE_INST_ANY": "wave-cycles issuing any instruction",
    "SQ_VALU_MFMA_BUSY_CYCLES": "SIMD-cycles the matrix cores were busy",
    "SQ_LDS_BANK_CONFLICT": "cycles lost to LDS bank conflicts",
    "SQ_LDS_IDX_ACTIVE": "cycles the LDS was processing indexed accesses",
    "SQ_ACTIVE_INST_LDS": "wave-cycles issuing LDS instructions",
    "SQ_ACTIVE_INST_VMEM": "wave-cycles issuing vector memory instructions",
    "SQ_INST_LEVEL_VMEM": "vector memory instructions in flight, summed per cycle",
    "GRBM_GUI_ACTIVE": "GPU-busy cycles (elapsed clock)",
}


def counters(name, kernel, commands, csvs, out, units=None, unit_name=None, simds=1024, xcds=8, skip_first=1):
    """Summary of counter passes (one CSV per rocprofv3 --pmc run) for the
    dispatches of `kernel` (a short name as short_name gives it): the average
    of each counter per dispatch, and ratios that say what bounds the kernel."""
    vals = {}
    for path in csvs:
        with open(path) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
        per = defaultdict(list)
        for r in rows:
            if short_name(r["Kernel_Name"]) == kernel:
                per[r["Counter_Name"]].append(float(r["Counter_Value"]))
        for c, v in per.items():
            v = v[skip_first:] or v
            vals[c] = sum(v) / len(v)
    g = lambda c: vals.get(c)
    lines = [f"# {name}: hardware counters of `{kernel}`", "",
             "Counter passes (repository root), one rocprofv3 run each:", "", "```", *commands, "```", "",
             f"Averages per dispatch (the first dispatch skipped), {len(vals)} counters:", "",
             "| counter | per dispatch | what it counts |", "|---|---|---|"]
    for c in sorted(vals):
        lines.append(f"| {c} | {vals[c]:.4g} | {COUNTER_NOTES.get(c, '')} |")
    derived = []

    def ratio(label, num, den, scale=1.0, fmt="{:.3g}"):
        if num is not None and den:
            derived.append((label, fmt.format(scale * num / den)))

    # GRBM_GUI_ACTIVE comes summed over the XCDs: per XCD it is the elapsed clock
    ratio("elapsed us at 2.4 GHz (GRBM_GUI_ACTIVE per XCD)", g("GRBM_GUI_ACTIVE"), xcds * 2400.0)
    ratio("MFMA busy, % of SIMD-cycles", g("SQ_VALU_MFMA_BUSY_CYCLES"),
          (g("GRBM_GUI_ACTIVE") or 0) / xcds * simds, 100.0)
    ratio("VALU issue, % of resident wave-cycles", g("SQ_ACTIVE_INST_VALU"), g("SQ_WAVE_CYCLES"), 100.0)
    ratio("any issue, % of resident wave-cycles", g("SQ_ACTIVE_INST_ANY"), g("SQ_WAVE_CYCLES"), 100.0)
    ratio("waiting on a dependency, % of resident wave-cycles", g("SQ_WAIT_INST_ANY"), g("SQ_WAVE_CYCLES"), 100.0)
    ratio("waiting for anything (dependencies, barriers), % of resident wave-cycles", g("SQ_WAIT_ANY"),
          g("SQ_WAVE_CYCLES"), 100.0)
    ratio("LDS busy with indexed accesses, % of CU-cycles", g("SQ_LDS_IDX_ACTIVE"),
          (g("GRBM_GUI_ACTIVE") or 0) / xcds * (simds // 4), 100.0)
    ratio("LDS bank-conflict cycles, % of LDS-active cycles", g("SQ_LDS_BANK_CONFLICT"), g("SQ_LDS_IDX_ACTIVE"), 100.0)
    ratio("MFMA share of VALU instructions, %", g("SQ_INSTS_MFMA"), g("SQ_INSTS_VALU"), 100.0)
    ratio("vector memory instructions in flight (average)", g("SQ_INST_LEVEL_VMEM"), g("SQ_ACTIVE_INST_VMEM"))
    if units:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
            ratio(f"{c} per {unit_name}", g(c), units)
        mops = (g("SQ_INSTS_VALU_MFMA_MOPS_BF16") or 0) + (g("SQ_INSTS_VALU_MFMA_MOPS_F16") or 0)
        if mops:
            derived.append((f"MFMA flops per {unit_name}", f"{512 * mops / units:.4g}"))
    if derived:
        lines += ["", "| derived | value |", "|---|---|"] + [f"| {a} | {b} |" for a, b in derived]
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, f"{name}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return vals, derived


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        ap = argparse.ArgumentParser()
        ap.add_argument("cmd")
        ap.add_argument("--name", required=True)
        ap.add_argument("--kernel", required=True)
        ap.add_argument("--csv", action="append", required=True)
        ap.add_argument("--command", action="append", required=True)
        ap.add_argument("--units", type=float)
        ap.add_argument("--unit-name")
        ap.add_argument("--out", required=True)
        a = ap.parse_args()
        vals, derived = counters(a.name, a.kernel, a.command, a.csv, a.out, a.units, a.unit_name)
        print(json.dumps({"counters": vals, "derived": dict(derived)}))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--algorithmic-bytes", type=int, required=True)
    ap.add_argument("--copy-bytes", type=int, default=2 * 2 ** 30)
    ap.add_argument("--out", required=True)
    ap.add_argument("--fetch-command")
    ap.add_argument("--write-command")
    ap.add_argument("--trace", help="kernel trace CSV of the statistics run")
    ap.add_argument("--skip", type=int, default=0, help="untimed calls before the timed ones")
    ap.add_argument("--take", type=int, default=0, help="timed calls")
    ap.add_argument("--only", action="append",
                    help="count only this kernel label in the call's traffic (repeatable)")
    a = ap.parse_args()
    r = summarize(a.name, a.command, a.stats, a.fetch, a.write, a.algorithmic_bytes, a.copy_bytes,
                  a.out, a.fetch_command, a.write_command, a.trace, a.skip, a.take, a.only)
    print(json.dumps(r))


if __name__ == "__main__":
    main()
