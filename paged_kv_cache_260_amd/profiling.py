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


def source_hash(paths=DECODE_SRCS) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the decode kernel's last template argument: what its work items' rows are
_DECODE_MODES = {"0": "", "1": " (chunk rows)", "2": " (shared prefix)", "3": " (private tokens)",
                 "4": " (shared prefix, one launch)", "5": " (append)"}


def short_name(name: str) -> str:
    for key in (*CALL_KERNELS, "paged_chunk_reduce_kernel", "paged_chunk_kernel", "kv_cache_write_fp8_kernel",
                "kv_cache_write_kernel",
                "zero_i32_kernel", "copy_blocks_kernel", COPY_KERNEL):
        if key in name:
            if key == DECODE_KERNEL and name.endswith("EEEvNS_10DecodeArgsE") and "ELi" in name:
                mode = name[: -len("EEEvNS_10DecodeArgsE")].rsplit("ELi", 1)[-1]
                return key + _DECODE_MODES.get(mode, "")
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


def summarize(name, command, stats_csv, fetch_csv, write_csv, algorithmic_bytes, copy_bytes, out,
              fetch_command=None, write_command=None):
    os.makedirs(out, exist_ok=True)
    stats = read_stats(stats_csv)
    lines = [f"# {name}: rocprofv3 kernel statistics", "", "Command (repository root):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short_name(r['name'])} | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | "
                     f"{r['min_ns'] / 1e3:.2f} | {r['max_ns'] / 1e3:.2f} | {r['pct']:.1f} |")
    with open(os.path.join(out, f"{name}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    result = {"name": name, "decode_source_hash": source_hash(), "command": command,
              "algorithmic_bytes": int(algorithmic_bytes),
              "kernel_avg_us": {short_name(r["name"]): r["avg_ns"] / 1e3 for r in stats}}
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


def main():
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
    a = ap.parse_args()
    r = summarize(a.name, a.command, a.stats, a.fetch, a.write, a.algorithmic_bytes, a.copy_bytes,
                  a.out, a.fetch_command, a.write_command)
    print(json.dumps(r))


if __name__ == "__main__":
    main()
