"""Summarise rocprofv3 results of a bench run: per-kernel durations and HBM bytes.

Input: three rocprofv3 SQLite result databases of the same command, one from
``--kernel-trace --stats``, one from ``--pmc FETCH_SIZE`` and one from
``--pmc WRITE_SIZE``.  The command must have run one plain device copy of
1 GiB first (``bench.py --copy-calibration``): the counters are scaled by what
they read for that copy, whose true traffic is known (1 GiB read, 1 GiB
written).

Output: a Markdown table (stdout, or ``--md``) and, with ``--json``, a record
of each library kernel's measured HBM bytes per launch together with a SHA-256
of the source files it is built from, so that a consumer can tell whether the
kernel has changed since the counters were taken.

    python -m dynamic_sparse_attention_dsv_amd.profile_summary KT.db FETCH.db WRITE.db \
        --command "..." --md out.md --json out.json
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# library timing name -> (device kernel name prefix, source files it is compiled from)
KERNELS = {
    "proj_kernel(q)": ("proj_bf16_kernel", ["predict.hip", "common.hpp", "topk_row.hpp"]),
    "scores_kernel": ("scores_bf16_kernel", ["predict.hip", "common.hpp", "topk_row.hpp"]),
    "rep_select_kernel": ("rep_select_bf16_kernel", ["predict.hip", "common.hpp", "topk_row.hpp"]),
    "select_topk_kernel": ("select_topk_kernel", ["select.hip", "common.hpp", "topk_row.hpp"]),
    "attn_fwd_kernel": ("attn_fwd_bf16_kernel", ["attn_fwd.hip", "common.hpp"]),
    "bwd_pre_kernel": ("bwd_pre_bf16_kernel", ["attn_bwd.hip", "common.hpp"]),
    "attn_bwd_dkdv_kernel": ("attn_bwd_dkdv_bf16_kernel", ["attn_bwd.hip", "common.hpp"]),
    "attn_bwd_dq_kernel": ("attn_bwd_dq_bf16_kernel", ["attn_bwd.hip", "common.hpp"]),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_KIB = 1 << 20  # 1 GiB


def source_hash(timing_name: str) -> str | None:
    """SHA-256 over the kernel's source files and the compiler flags they are built with (the
    common flags and the kernel file's own, from build.py; other edits of build.py do not count)."""
    if timing_name not in KERNELS:
        return None
    from . import build as B

    h = hashlib.sha256()
    files = KERNELS[timing_name][1]
    for path in [os.path.join(CSRC, f) for f in files]:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + fh.read())
    flags = [f for f in B.HIP_FLAGS if not f.startswith(B.ROOT)] + B.FILE_FLAGS.get(files[0], [])
    h.update(b"flags\0" + " ".join(flags).encode())
    return h.hexdigest()


def short(name: str) -> str:
    name = re.sub(r"\(.*", "", name)
    return name.replace("void ", "").replace("dsv::", "").strip()


def _counters(db: str, counter: str) -> dict:
    vals = collections.defaultdict(list)
    con = sqlite3.connect(db)
    for name, val in con.execute("select kernel_name, value from counters_collection where counter_name=?",
                                 (counter,)):
        vals[short(name)].append(val)
    return {k: sum(v) / len(v) for k, v in vals.items()}


def summarise(kt_db: str, fetch_db: str, write_db: str):
    rows = list(sqlite3.connect(kt_db).execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels"))
    fetch, write = _counters(fetch_db, "FETCH_SIZE"), _counters(write_db, "WRITE_SIZE")
    if COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        raise SystemExit("the profiled command ran no 1 GiB calibration copy (bench.py --copy-calibration)")
    cal = {"fetch_scale": COPY_KIB / fetch[COPY_KERNEL], "write_scale": COPY_KIB / write[COPY_KERNEL],
           "fetch_kib_for_copy": fetch[COPY_KERNEL], "write_kib_for_copy": write[COPY_KERNEL]}
    table = []
    for name, calls, _total, avg_us, pct in rows:  # top_kernels durations are in microseconds
        s = short(name)
        f = fetch.get(s)
        w = write.get(s)
        table.append({"kernel": s, "calls": calls, "avg_ms": avg_us / 1e3, "pct": pct,
                      "read_bytes": None if f is None else f * cal["fetch_scale"] * 1024,
                      "write_bytes": None if w is None else w * cal["write_scale"] * 1024})
    return cal, table


def to_markdown(cal, table, command: str, title: str) -> str:
    out = [f"# {title}", "", "Commands (repository root, one MI355X, `export TMPDIR=/tmp`):", ""]
    out += ["    " + c for c in command.split("\n")] + [""]
    out += [f"Counters are per dispatch, scaled by what they read for the 1 GiB calibration copy: "
            f"FETCH_SIZE {cal['fetch_kib_for_copy']:.0f} KiB -> x{cal['fetch_scale']:.3f}, "
            f"WRITE_SIZE {cal['write_kib_for_copy']:.0f} KiB -> x{cal['write_scale']:.3f}.", ""]
    out += ["| kernel | calls | avg ms | % time | HBM read GB/launch | HBM write GB/launch |",
            "|---|---|---|---|---|---|"]
    for r in table:
        rd = "-" if r["read_bytes"] is None else f"{r['read_bytes'] / 1e9:.3f}"
        wr = "-" if r["write_bytes"] is None else f"{r['write_bytes'] / 1e9:.3f}"
        out.append(f"| {r['kernel']} | {r['calls']} | {r['avg_ms']:.3f} | {r['pct']:.2f} | {rd} | {wr} |")
    return "\n".join(out) + "\n"


def to_record(cal, table, command: str, workload: str) -> dict:
    kernels = {}
    for timing_name, (prefix, _srcs) in KERNELS.items():
        hits = [r for r in table if r["kernel"].startswith(prefix)]
        if not hits or hits[0]["read_bytes"] is None or hits[0]["write_bytes"] is None:
            continue
        r = hits[0]
        kernels[timing_name] = {"device_kernel": r["kernel"], "avg_ms": r["avg_ms"], "read_bytes": r["read_bytes"],
                                "write_bytes": r["write_bytes"], "source_sha256": source_hash(timing_name)}
    return {"workload": workload, "command": command, "calibration": cal, "kernels": kernels}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("kernel_trace_db")
    ap.add_argument("fetch_db")
    ap.add_argument("write_db")
    ap.add_argument("--command", required=True, help="the commands that produced the databases")
    ap.add_argument("--title", default="Kernel profile")
    ap.add_argument("--workload", default="")
    ap.add_argument("--md")
    ap.add_argument("--json")
    a = ap.parse_args()
    cal, table = summarise(a.kernel_trace_db, a.fetch_db, a.write_db)
    md = to_markdown(cal, table, a.command, a.title)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(md)
    else:
        print(md)
    if a.json:
        with open(a.json, "w") as fh:
            json.dump(to_record(cal, table, a.command, a.workload), fh, indent=1)
            fh.write("\n")


if __name__ == "__main__":
    main()
